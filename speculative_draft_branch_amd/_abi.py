"""ctypes declarations of the C ABI (include/branch_attn.h) and the Plan wrapper."""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

BA_OK, BA_EINVAL, BA_EUNSUPPORTED, BA_EWORKSPACE, BA_EHIP = 0, 1, 2, 3, 4
BA_F32, BA_BF16 = 0, 1
BA_TTT, BA_BLOCK = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libbranch_attn.so")


class BranchAttnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class _Problem(C.Structure):
    _fields_ = [
        ("dtype", C.c_int),
        ("num_q_heads", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("softmax_scale", C.c_float),
        ("kv_head_of", C.POINTER(C.c_int32)),
        ("num_seqs", C.c_int32),
        ("cu_seqlens", C.POINTER(C.c_int32)),
        ("num_q", C.c_int32),
        ("q_pos", C.POINTER(C.c_int32)),
        ("num_anchors", C.c_int32),
        ("anchors", C.POINTER(C.c_int32)),
        ("cu_branch", C.POINTER(C.c_int32)),
        ("branch_len", C.c_int32),
        ("mode", C.POINTER(C.c_uint8)),
        ("uniform_mode", C.c_int),
    ]


def _load():
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python speculative_draft_branch_amd/build.py` "
                          f"(there is no fallback path)")
    L = C.CDLL(path)
    vp, sz, i64, i32, f32p = C.c_void_p, C.c_size_t, C.c_int64, C.c_int32, C.POINTER(C.c_float)
    st = C.c_int
    L.ba_plan_create.argtypes = [C.POINTER(_Problem), C.POINTER(vp)]
    L.ba_plan_create.restype = st
    L.ba_plan_destroy.argtypes = [vp]
    L.ba_plan_destroy.restype = None
    L.ba_workspace_bytes.argtypes = [vp, C.c_int]
    L.ba_workspace_bytes.restype = sz
    L.ba_plan_sizes.argtypes = [vp, C.POINTER(i64)]
    L.ba_plan_sizes.restype = st
    L.ba_plan_pairs.argtypes = [vp, C.POINTER(i64)]
    L.ba_plan_pairs.restype = st
    L.branch_attn_fwd.argtypes = [vp] + [vp] * 6 + [vp, vp, vp, vp] + [vp, sz, vp]
    L.branch_attn_fwd.restype = st
    L.branch_attn_fwd_noalloc.argtypes = [vp] + [vp] * 6 + [vp, vp, vp, vp] + [vp]
    L.branch_attn_fwd_noalloc.restype = st
    L.ba_fwd_noalloc_max_bytes.argtypes = []
    L.ba_fwd_noalloc_max_bytes.restype = sz
    L.branch_attn_bwd.argtypes = [vp] + [vp] * 6 + [vp, vp, vp, vp] + [vp, vp] + [vp] * 6 + [vp, sz, vp]
    L.branch_attn_bwd.restype = st
    L.lse_merge.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, C.c_int, vp, vp]
    L.lse_merge.restype = st
    L.ba_main_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.ba_main_fwd.restype = st
    L.ba_branch_local_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.ba_branch_local_fwd.restype = st
    L.ba_ring_step_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, sz, vp]
    L.ba_ring_step_fwd.restype = st
    L.ba_status_str.argtypes = [st]
    L.ba_status_str.restype = C.c_char_p
    L.ba_last_error.argtypes = []
    L.ba_last_error.restype = C.c_char_p
    L.ba_abi_version.argtypes = []
    L.ba_abi_version.restype = C.c_int
    L.ba_timing_enable.argtypes = [C.c_int]
    L.ba_timing_enable.restype = st
    L.ba_timing_reset.argtypes = []
    L.ba_timing_reset.restype = st
    L.ba_timing_kernels.argtypes = []
    L.ba_timing_kernels.restype = C.c_int
    L.ba_timing_kernel_name.argtypes = [C.c_int]
    L.ba_timing_kernel_name.restype = C.c_char_p
    L.ba_timing_read.argtypes = [C.c_int, C.POINTER(C.c_double), C.POINTER(i64)]
    L.ba_timing_read.restype = st
    return L


lib = _load()


def abi_version() -> int:
    return int(lib.ba_abi_version())


def exported_symbols() -> list:
    return ["ba_plan_create", "ba_plan_destroy", "ba_workspace_bytes", "ba_plan_sizes", "ba_plan_pairs",
            "branch_attn_fwd", "branch_attn_fwd_noalloc", "ba_fwd_noalloc_max_bytes", "branch_attn_bwd", "lse_merge", "ba_main_fwd", "ba_branch_local_fwd",
            "ba_ring_step_fwd",
            "ba_status_str", "ba_last_error", "ba_abi_version", "ba_timing_enable", "ba_timing_reset",
            "ba_timing_kernels", "ba_timing_kernel_name", "ba_timing_read"]


def timing_enable(on: bool = True):
    check(lib.ba_timing_enable(1 if on else 0), "ba_timing_enable")


def timing_reset():
    check(lib.ba_timing_reset(), "ba_timing_reset")


def timing_read() -> dict:
    """{kernel name: (total ms, launches)} recorded since the last reset (waits for the events)."""
    out = {}
    for i in range(int(lib.ba_timing_kernels())):
        ms, n = C.c_double(), C.c_int64()
        check(lib.ba_timing_read(i, C.byref(ms), C.byref(n)), "ba_timing_read")
        out[lib.ba_timing_kernel_name(i).decode()] = (float(ms.value), int(n.value))
    return out


def check(status: int, where: str):
    if status != BA_OK:
        raise BranchAttnError(status, where, (lib.ba_last_error() or b"").decode())


def _i32(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64).astype(np.int32))


def _ptr(a: Optional[np.ndarray], ctype):
    return None if a is None else a.ctypes.data_as(C.POINTER(ctype))


class Plan:
    """Owns a ba_plan_t built from host arrays (copied by the library)."""

    def __init__(self, dtype: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 cu_seqlens: Sequence[int], q_pos: Optional[Sequence[int]], anchors: Sequence[int],
                 cu_branch: Optional[Sequence[int]], modes: Optional[Sequence[int]],
                 branch_len: int = 0, uniform_mode: int = BA_TTT, softmax_scale: float = 0.0,
                 kv_head_of: Optional[Sequence[int]] = None):
        self._h = None
        cu = _i32(cu_seqlens)
        qp = _i32(q_pos)
        an = _i32(anchors) if anchors is not None else np.zeros(0, np.int32)
        cb = _i32(cu_branch)
        md = None if modes is None else np.ascontiguousarray(np.asarray(modes, dtype=np.uint8))
        kh = _i32(kv_head_of)
        p = _Problem()
        p.dtype = int(dtype)
        p.num_q_heads, p.num_kv_heads, p.head_dim = int(num_q_heads), int(num_kv_heads), int(head_dim)
        p.softmax_scale = float(softmax_scale)
        p.kv_head_of = _ptr(kh, C.c_int32)
        p.num_seqs = int(len(cu) - 1)
        p.cu_seqlens = _ptr(cu, C.c_int32)
        p.num_q = 0 if qp is None else int(len(qp))
        p.q_pos = _ptr(qp, C.c_int32)
        p.num_anchors = int(len(an))
        p.anchors = _ptr(an, C.c_int32) if len(an) else None
        p.cu_branch = _ptr(cb, C.c_int32)
        p.branch_len = int(branch_len)
        p.mode = _ptr(md, C.c_uint8) if md is not None and len(md) else None
        p.uniform_mode = int(uniform_mode)
        h = C.c_void_p()
        check(lib.ba_plan_create(C.byref(p), C.byref(h)), "ba_plan_create")
        self._h = h
        self.dtype = int(dtype)
        self.hq, self.hkv, self.d = int(num_q_heads), int(num_kv_heads), int(head_dim)
        sizes = (C.c_int64 * 5)()
        check(lib.ba_plan_sizes(h, sizes), "ba_plan_sizes")
        self.N, self.Nq, self.Rb, self.n_qtiles, self.n_ktiles = (int(x) for x in sizes)
        pairs = (C.c_int64 * 3)()
        check(lib.ba_plan_pairs(h, pairs), "ba_plan_pairs")
        self.pairs = tuple(int(x) for x in pairs)

    @classmethod
    def from_workload(cls, w, softmax_scale: Optional[float] = None, kv_head_of=None) -> "Plan":
        """Plan of a workload description; its own head map and scale unless overridden."""
        if softmax_scale is None:
            softmax_scale = getattr(w, "softmax_scale", 0.0) or 0.0
        if kv_head_of is None:
            kv_head_of = getattr(w, "kv_head_of", None)
        return cls(BA_BF16 if w.dtype == "bf16" else BA_F32, w.num_q_heads, w.num_kv_heads, w.head_dim,
                   w.cu_seqlens, w.q_pos, w.anchors, w.cu_branch, w.modes, softmax_scale=softmax_scale,
                   kv_head_of=kv_head_of)

    @property
    def handle(self):
        return self._h

    def workspace_bytes(self, pass_: int) -> int:
        return int(lib.ba_workspace_bytes(self._h, int(pass_)))

    def flops_fwd(self) -> int:
        return 4 * self.d * self.hq * sum(self.pairs)

    def flops_bwd(self) -> int:
        return 10 * self.d * self.hq * sum(self.pairs)

    def close(self):
        if self._h is not None and self._h.value:
            lib.ba_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
