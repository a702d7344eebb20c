"""MI355X (gfx950) speculative-draft branch attention.

A thin binding over ``libbranch_attn.so`` (C ABI in ``include/branch_attn.h``):
argument marshalling only. Every step of the operator runs in the library's
HIP kernels; PyTorch supplies device memory and the current stream. If the
library is not built this package raises on import -- there is no fallback.

    plan = Plan.from_workload(w)            # or Plan(hq, hkv, d, cu_seqlens, ...)
    o, lse, ob, lseb = fwd(plan, q, k, v, qb, kb, vb)
    dq, dk, dv, dqb, dkb, dvb = bwd(plan, q, k, v, qb, kb, vb, o, lse, ob, lseb, do, dob)
"""
from ._abi import (  # noqa: F401
    BA_OK, BA_EINVAL, BA_EUNSUPPORTED, BA_EWORKSPACE, BA_EHIP, BA_F32, BA_BF16, BA_TTT, BA_BLOCK,
    BranchAttnError, Plan, lib, library_path, abi_version, exported_symbols, timing_enable, timing_reset,
    timing_read,
)
from .ops import (  # noqa: F401
    branch_attn_fwd, branch_attn_fwd_noalloc, fwd_noalloc_max_bytes, branch_attn_bwd, lse_merge, ba_main_fwd, ba_branch_local_fwd, ba_ring_step_fwd, fwd, bwd,
    workspace,
)
