"""Packed-batch structures for the branch-attention workloads.

Every workload is a packed batch of main-sequence tokens (``cu_seqlens``), the
main query positions this GPU owns (``q_pos``), and the speculative-draft
branches that hang off anchor tokens (``anchors``, ``cu_branch``, ``modes``).

Branch modes:

* ``TTT`` -- an EAGLE-3 training-time-test branch of depth k: branch query j
  (1-based) sees its anchor's causal main prefix plus branch keys 1..j.
* ``BLOCK`` -- a DFlash-style draft block of B queries: every block query sees
  its anchor's causal main prefix plus all B keys of its own block.

(Draft families and the branch/main split: evolve.pub review, "Summary" and
"Key claims under review"; rcap.io explainer, paragraph on branch attention
under context parallelism.)
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, Optional, Sequence

import numpy as np

TTT = 0
BLOCK = 1

K16 = 16384


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16": the element type of every tensor
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    cu_seqlens: np.ndarray     # int32 [S+1]
    q_pos: np.ndarray          # int32 [Nq], strictly increasing packed positions
    anchors: np.ndarray        # int32 [A], strictly increasing packed positions
    cu_branch: np.ndarray      # int32 [A+1], branch row offsets
    modes: np.ndarray          # uint8 [A], TTT or BLOCK per anchor
    std: float = 0.5           # std of Q/K/V/Qb/Kb/Vb
    grad_std: float = 1.0      # std of dO/dOb
    seed: int = 0
    passes: tuple = ("fwd",)
    description: str = ""
    kv_head_of: Optional[np.ndarray] = None  # int32 [Hq] kv head of each q head; None -> h // (Hq/Hkv)
    softmax_scale: float = 0.0               # 0 -> 1/sqrt(head_dim)

    @property
    def N(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def Nq(self) -> int:
        return int(self.q_pos.shape[0])

    @property
    def A(self) -> int:
        return int(self.anchors.shape[0])

    @property
    def Rb(self) -> int:
        return int(self.cu_branch[-1])

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64).astype(np.int32))


def branches(anchors: Sequence[int], lens: Sequence[int], modes: Sequence[int]):
    """Anchors with per-anchor branch lengths and modes -> (anchors, cu_branch, modes)."""
    anchors = np.asarray(anchors, dtype=np.int64)
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.zeros(len(anchors) + 1, dtype=np.int64)
    np.cumsum(lens, out=cu[1:])
    return _i32(anchors), _i32(cu), np.asarray(modes, dtype=np.uint8)


def make(name, dtype, hq, hkv, d, cu_seqlens, q_pos, anchors, lens, modes, **kw) -> Workload:
    a, cub, m = branches(anchors, lens, modes)
    q_pos = np.arange(int(cu_seqlens[-1])) if q_pos is None else q_pos
    return Workload(name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    cu_seqlens=_i32(cu_seqlens), q_pos=_i32(q_pos), anchors=a,
                    cu_branch=cub, modes=m, **kw)


def seq_offsets(lengths: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(np.asarray(lengths, dtype=np.int64), out=cu[1:])
    return cu


def block_anchors(cu: np.ndarray, seq_ids: Sequence[int], every: int = 16) -> np.ndarray:
    """Anchors at sequence-local positions every-1, 2*every-1, ... (the 16th, 32nd, ... token)."""
    out = []
    for s in seq_ids:
        lo, hi = int(cu[s]), int(cu[s + 1])
        out.append(np.arange(lo + every - 1, hi, every, dtype=np.int64))
    return np.sort(np.concatenate(out)) if out else np.zeros(0, np.int64)


def loguniform_lengths(total: int, lo: int, hi: int, seed: int) -> list:
    """Sequence lengths drawn as round(exp(U(ln lo, ln hi))) until they cover
    ``total`` tokens; the last length is clipped so the sum is exactly ``total``."""
    rng = np.random.default_rng(seed)
    lens, acc = [], 0
    while acc < total:
        L = int(round(float(np.exp(rng.uniform(np.log(lo), np.log(hi))))))
        lens.append(L)
        acc += L
    lens[-1] -= acc - total
    return lens


# ---------------------------------------------------------------------------
# The named workloads.

def tiny_f32() -> Workload:
    """1 sequence of 256 tokens, 2 heads (no GQA), head_dim 64, fp32, N(0,1);
    TTT depth 3 at every position."""
    N = 256
    return make("tiny_f32", "f32", 2, 2, 64, [0, N], None, np.arange(N), [3] * N, [TTT] * N,
                std=1.0, passes=("fwd", "bwd"),
                description="1x256 tokens, 2 heads, d64, fp32, TTT depth 3 at every position")


def qwen3_8b_16k(div: int = 1) -> Workload:
    """GQA 32q/8kv, d128, 4 packed sequences 2K/4K/4K/6K, TTT depth 7 everywhere."""
    lens = [2048 // div, 4096 // div, 4096 // div, 6144 // div]
    cu = seq_offsets(lens)
    N = int(cu[-1])
    sfx = "" if div == 1 else f"_div{div}"
    return make("qwen3_8b_16k" + sfx, "bf16", 32, 8, 128, cu, None, np.arange(N), [7] * N, [TTT] * N,
                passes=("fwd", "bwd"),
                description=f"Qwen3-8B-like GQA 32/8 d128, packed {lens}, TTT depth 7 at every position")


def dflash_64k(n_tokens: int = 65536) -> Workload:
    """GQA 32q/8kv, d128, one sequence, 16-query draft blocks anchored every 16th token."""
    cu = np.array([0, n_tokens])
    anc = block_anchors(cu, [0], 16)
    sfx = "" if n_tokens == 65536 else f"_{n_tokens}"
    return make("dflash_64k" + sfx, "bf16", 32, 8, 128, cu, None, anc, [16] * len(anc), [BLOCK] * len(anc),
                passes=("fwd", "bwd"),
                description=f"block-draft GQA 32/8 d128, 1x{n_tokens} tokens, 16-query blocks every 16th token")


def ctx256k_rank3(chunk: int = K16) -> Workload:
    """One rank's share of a 16-chunk zigzag layout (CP=8, rank 3): queries of chunks 3 and 12,
    causal over all preceding keys (chunks 0..12 present), TTT depth 7 on every local position."""
    n_keys = 13 * chunk
    q_pos = np.concatenate([np.arange(3 * chunk, 4 * chunk), np.arange(12 * chunk, 13 * chunk)])
    sfx = "" if chunk == K16 else f"_chunk{chunk}"
    return make("ctx256k_rank3" + sfx, "bf16", 32, 8, 128, [0, n_keys], q_pos, q_pos,
                [7] * len(q_pos), [TTT] * len(q_pos), passes=("fwd", "bwd"),
                description=(f"{16 * chunk}-token sequence in 16 zigzag chunks of {chunk}; rank 3 of CP=8 holds "
                             f"chunks 3 and 12; GQA 32/8 d128; TTT depth 7 on local anchors"))


def gptoss_128k_mixed(total: int = 131072, lo: int = 2048, hi: int = 32768, seed: int = 0) -> Workload:
    """GQA 64q/8kv, d64, log-uniform packed lengths; TTT depth 7 at every position of odd
    sequences, 16-query blocks every 16th token of even sequences (0-based indices)."""
    lens = loguniform_lengths(total, lo, hi, seed)
    cu = seq_offsets(lens)
    anc, ln, md = [], [], []
    for s in range(len(lens)):
        lo_s, hi_s = int(cu[s]), int(cu[s + 1])
        if s % 2 == 1:
            a = np.arange(lo_s, hi_s)
            anc.append(a); ln += [7] * len(a); md += [TTT] * len(a)
        else:
            a = np.arange(lo_s + 15, hi_s, 16)
            anc.append(a); ln += [16] * len(a); md += [BLOCK] * len(a)
    anc = np.concatenate(anc)  # sequences are visited in order, so anchors are increasing
    sfx = "" if (total, lo, hi) == (131072, 2048, 32768) else f"_{total}"
    return make("gptoss_128k_mixed" + sfx, "bf16", 64, 8, 64, cu, None, anc, ln, md, seed=seed,
                passes=("fwd", "bwd"),
                description=f"GPT-OSS-120B-like GQA 64/8 d64, {total} tokens log-uniform [{lo},{hi}] "
                            f"(seed {seed}), mixed TTT-7 / 16-blocks")


_REGISTRY: Dict[str, Callable[[], Workload]] = {
    "tiny_f32": tiny_f32,
    "qwen3_8b_16k": qwen3_8b_16k,
    "dflash_64k": dflash_64k,
    "ctx256k_rank3": ctx256k_rank3,
    "gptoss_128k_mixed": gptoss_128k_mixed,
    # reduced sizes of the same structures, small enough for a dense CPU oracle
    "qwen3_8b_16k_div16": lambda: qwen3_8b_16k(16),
    "dflash_64k_1024": lambda: dflash_64k(1024),
    "ctx256k_rank3_chunk64": lambda: ctx256k_rank3(64),
    "ctx256k_rank3_chunk256": lambda: ctx256k_rank3(256),
    "ctx256k_rank3_chunk80": lambda: ctx256k_rank3(80),
    "gptoss_128k_mixed_2048": lambda: gptoss_128k_mixed(2048, 32, 512, 0),
}


def names():
    return list(_REGISTRY)


def get(name: str) -> Workload:
    return _REGISTRY[name]()


def custom(name: str, dtype: str, hq: int, hkv: int, d: int, seq_lens: Sequence[int],
           q_pos: Optional[Sequence[int]], anchors: Sequence[int], lens: Sequence[int],
           modes: Sequence[int], **kw) -> Workload:
    """A hand-built workload (edge cases in tests)."""
    cu = seq_offsets(seq_lens)
    return make(name, dtype, hq, hkv, d, cu, None if q_pos is None else np.asarray(q_pos),
                np.asarray(anchors, dtype=np.int64), lens, modes, **kw)
