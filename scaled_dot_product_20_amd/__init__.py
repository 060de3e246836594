"""Fused scaled-dot-product attention (forward + backward) for the MI355X
(gfx950): hand-written HIP kernels behind the C ABI of ``include/attn.h``.

``attn_fwd`` / ``attn_bwd`` are thin ctypes wrappers; the seeded workload
generators live in ``workloads``.
"""
from .binding import WINDOW_INF, AttnError, attn_bwd, attn_fwd, workspace_size  # noqa: F401
