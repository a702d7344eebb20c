"""The tap mailbox on one MI355X, through the C ABI: a producer stream writes
one tap per microbatch and a consumer stream waits for it and reads it (both at
the default priority, ordered by events both ways), and a scripted sequence of
refusals; bytes and statuses against the plain model (oracle/tapchannel.py)."""
import numpy as np
import pytest
import torch

from oracle import tapchannel as T

from gpu_util import say

pytestmark = pytest.mark.gpu

sda = pytest.importorskip("speculative_draft_branch_amd")
from speculative_draft_branch_amd import tapchannel as tc  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bytes(n, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g)


def test_microbatches_across_two_streams():
    cap = (3 << 20) + 40
    sizes = [1 << 20, (3 << 20) + 40, 17, 0, (2 << 20) + 5, 4096]
    srcs_h = [_bytes(n, i) for i, n in enumerate(sizes)]
    srcs = [x.cuda() for x in srcs_h]
    dsts = [torch.full((cap,), 0xAB, dtype=torch.uint8, device="cuda") for _ in sizes]
    st_w = torch.full((len(sizes),), -1, dtype=torch.int32, device="cuda")
    st_r = torch.full((len(sizes),), -1, dtype=torch.int32, device="cuda")
    nb = torch.zeros(len(sizes), dtype=torch.int64, device="cuda")
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(prod):
        slot = tc.Slot(cap)
    torch.cuda.synchronize()
    say(f"[tap] {len(sizes)} microbatches, slot of {cap} bytes")
    read_done = None
    for i, n in enumerate(sizes):
        stamp = i + 1
        written = torch.cuda.Event()
        with torch.cuda.stream(prod):
            if read_done is not None:
                prod.wait_event(read_done)  # the reader has taken the previous tap
            slot.write(srcs[i], stamp, st_w[i:i + 1], done_event=written)
        with torch.cuda.stream(cons):
            slot.read(dsts[i], stamp, st_r[i:i + 1], nb[i:i + 1], written_event=written)
            read_done = torch.cuda.Event()
            read_done.record(cons)
    torch.cuda.synchronize()
    assert st_w.tolist() == [T.OK] * len(sizes)
    assert st_r.tolist() == [T.OK] * len(sizes)
    assert nb.tolist() == sizes
    for i, n in enumerate(sizes):
        d = dsts[i].cpu()
        assert torch.equal(d[:n], srcs_h[i]), i
        assert bool((d[n:] == 0xAB).all()), i  # nothing past the tap is written


def test_scripted_statuses_and_bytes_match_the_model():
    cap = 1000
    model = T.Slot(cap)
    slot = tc.Slot(cap)
    script = [("r", 1, 1000), ("w", 1, 999), ("w", 2, 10), ("r", 2, 1000), ("r", 1, 1000), ("r", 1, 1000),
              ("w", 1, 5), ("w", 3, 1000), ("r", 2, 1000), ("r", 3, 999), ("r", 3, 1000), ("w", 4, 1001),
              ("w", 4, 333), ("r", 4, 1000), ("w", 7, 1), ("r", 5, 8), ("r", 7, 8)]
    st = torch.full((len(script),), -1, dtype=torch.int32, device="cuda")
    nb = torch.zeros(len(script), dtype=torch.int64, device="cuda")
    dsts, want = [], []
    for i, (who, stamp, n) in enumerate(script):
        if who == "w":
            data = _bytes(n, 100 + i)
            slot.write(data.cuda(), stamp, st[i:i + 1])
            want.append((model.write(bytes(data.numpy()), stamp), None))
            dsts.append(None)
        else:
            dst = torch.full((n,), 0xCD, dtype=torch.uint8, device="cuda")
            slot.read(dst, stamp, st[i:i + 1], nb[i:i + 1])
            want.append(model.read(stamp, n))
            dsts.append(dst)
    torch.cuda.synchronize()
    got = st.tolist()
    say("  statuses: " + " ".join(T.NAMES[s] for s in got))
    assert got == [w for w, _ in want]
    for i, (who, stamp, n) in enumerate(script):
        if who != "r":
            continue
        d = dsts[i].cpu().numpy()
        status, data = want[i]
        if status == T.OK:
            assert bytes(d[:len(data)]) == data and int(nb[i]) == len(data)
            assert np.all(d[len(data):] == 0xCD)
        else:
            assert np.all(d == 0xCD), i  # a refused read leaves the destination alone


def test_uninitialised_slot_refuses():
    cap = 64
    mem = torch.zeros(tc.slot_bytes(cap), dtype=torch.uint8, device="cuda")  # no magic: never initialised
    st = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    src = torch.ones(8, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(8, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    from speculative_draft_branch_amd._abi import check
    check(tc.lib.ba_tap_write(mem.data_ptr(), cap, src.data_ptr(), 8, 1, st[0:1].data_ptr(), None, s), "write")
    check(tc.lib.ba_tap_read(mem.data_ptr(), cap, dst.data_ptr(), 8, 1, st[1:2].data_ptr(), None, s), "read")
    torch.cuda.synchronize()
    assert st.tolist() == [T.NOT_READY, T.NOT_READY]
    assert int(dst.sum()) == 0
