"""Python binding of libprism.so, the gfx950 dynamic block-shape,
block-sparse video self-attention library.

The five C entry points are exposed under their C names with the C argument
order (device pointers as ints, ``stream`` as a hipStream_t handle):
``prism_zone_shapes``, ``prism_pool_blocks``, ``prism_select_blocks``,
``prism_sparse_attn_fwd``, ``prism_sparse_attn_bwd``; so are the two calls of
the forward-only variant that keeps a pooled stand-in of the unselected
blocks, ``prism_dropped_terms`` and ``prism_sparse_attn_fwd_corrected``.  This module only
marshals arguments; every step runs in the library's HIP kernels.  There is
no fallback: if the library is missing, loading fails with an error.

Torch-tensor helpers (``zone_shapes``, ``pool_blocks``, ``select_blocks``,
``sparse_attn_fwd``, ``sparse_attn_bwd``, ``dropped_terms``,
``sparse_attn_fwd_corrected``) allocate outputs with torch on the
current device and pass the current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "PrismError", "lib", "LIB_PATH", "PRISM_FP32", "PRISM_BF16",
    "prism_zone_shapes", "prism_zone_shapes_noalloc", "prism_pool_blocks",
    "prism_select_blocks", "prism_route_blocks",
    "prism_route_blocks_workspace_bytes", "route_blocks",
    "prism_sparse_attn_fwd", "prism_sparse_attn_bwd",
    "prism_zone_shapes_workspace_bytes", "prism_sparse_attn_bwd_workspace_bytes",
    "prism_sparse_attn_fwd_workspace_bytes", "prism_shape_table",
    "prism_dropped_terms", "prism_dropped_terms_workspace_bytes",
    "prism_sparse_attn_fwd_corrected",
    "prism_a2v_bridge", "prism_a2v_bridge_workspace_bytes", "a2v_bridge",
    "prism_last_error", "prism_version", "prism_profile_enable",
    "prism_profile_reset", "prism_profile_count", "prism_profile_name",
    "prism_profile_ms", "kernel_times",
    "zone_shapes", "pool_blocks", "select_blocks", "sparse_attn_fwd",
    "sparse_attn_bwd", "shape_table", "dropped_terms",
    "sparse_attn_fwd_corrected",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libprism.so")
PRISM_FP32 = 0
PRISM_BF16 = 1
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "SHAPE", 3: "UNSUPPORTED",
          4: "WORKSPACE", 5: "HIP"}

_c_int, _c_sz, _c_dbl, _c_flt, _c_p = (ctypes.c_int, ctypes.c_size_t,
                                       ctypes.c_double, ctypes.c_float,
                                       ctypes.c_void_p)

_SIGS = {
    "prism_last_error": (ctypes.c_char_p, []),
    "prism_version": (_c_int, []),
    "prism_profile_enable": (_c_int, [_c_int]),
    "prism_profile_reset": (None, []),
    "prism_profile_count": (_c_int, []),
    "prism_profile_name": (ctypes.c_char_p, [_c_int]),
    "prism_profile_ms": (_c_flt, [_c_int]),
    "prism_shape_table": (_c_int, [_c_p]),
    "prism_zone_shapes_workspace_bytes": (_c_sz, [_c_int] * 8),
    "prism_zone_shapes": (_c_int, [_c_p, _c_p, _c_int, _c_int, _c_int, _c_int,
                                   _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _c_dbl, _c_int, _c_p, _c_p, _c_p, _c_p,
                                   _c_p, _c_sz, _c_p]),
    "prism_zone_shapes_noalloc": (_c_int, [_c_p, _c_p, _c_int, _c_int, _c_int,
                                           _c_int, _c_int, _c_int, _c_int,
                                           _c_int, _c_int, _c_dbl, _c_int,
                                           _c_p, _c_p, _c_p, _c_p, _c_p]),
    "prism_pool_blocks": (_c_int, [_c_p, _c_p, _c_int, _c_p, _c_int, _c_int,
                                   _c_int, _c_int, _c_p, _c_p, _c_p, _c_p]),
    "prism_route_blocks_workspace_bytes": (_c_sz, [_c_int] * 4),
    "prism_route_blocks": (_c_int, [_c_p, _c_p, _c_int, _c_p, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_dbl, _c_p, _c_p,
                                    _c_p, _c_p, _c_int, _c_p, _c_sz, _c_p]),
    "prism_select_blocks": (_c_int, [_c_p, _c_int, _c_int, _c_int, _c_int,
                                     _c_dbl, _c_p, _c_p, _c_int, _c_p]),
    "prism_sparse_attn_fwd_workspace_bytes": (_c_sz, [_c_int] * 4),
    "prism_sparse_attn_fwd": (_c_int, [_c_p, _c_p, _c_p, _c_int, _c_p, _c_p,
                                       _c_p, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_flt, _c_p, _c_p, _c_p, _c_sz,
                                       _c_p]),
    "prism_dropped_terms_workspace_bytes": (_c_sz, [_c_int] * 4),
    "prism_dropped_terms": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_int, _c_p,
                                     _c_p, _c_p, _c_int, _c_int, _c_int,
                                     _c_int, _c_int, _c_p, _c_p, _c_p, _c_sz,
                                     _c_p]),
    "prism_sparse_attn_fwd_corrected": (_c_int, [_c_p, _c_p, _c_p, _c_int, _c_p,
                                                 _c_p, _c_p, _c_int, _c_int,
                                                 _c_int, _c_int, _c_int, _c_flt,
                                                 _c_p, _c_p, _c_p, _c_p, _c_p,
                                                 _c_sz, _c_p]),
    "prism_a2v_bridge_workspace_bytes": (_c_sz, [_c_int] * 6),
    "prism_a2v_bridge": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                  _c_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_int, _c_int, _c_flt, _c_p, _c_p, _c_sz,
                                  _c_p]),
    "prism_sparse_attn_bwd_workspace_bytes": (_c_sz, [_c_int] * 4),
    "prism_sparse_attn_bwd": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                       _c_int, _c_p, _c_p, _c_p, _c_int,
                                       _c_int, _c_int, _c_int, _c_int, _c_flt,
                                       _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
}

_LIB = None


class PrismError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libprism.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m dynamic_block_sparse_shape_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise PrismError(st, name, lib().prism_last_error().decode())
    return st


# ------------------------------------------------------------ raw C names
def prism_last_error() -> str:
    return lib().prism_last_error().decode()


def prism_version() -> int:
    return lib().prism_version()


def prism_profile_enable(on: int) -> int:
    return _call("prism_profile_enable", int(on))


def prism_profile_reset() -> None:
    lib().prism_profile_reset()


def prism_profile_count() -> int:
    return lib().prism_profile_count()


def prism_profile_name(i: int) -> str:
    return lib().prism_profile_name(i).decode()


def prism_profile_ms(i: int) -> float:
    return lib().prism_profile_ms(i)


def kernel_times():
    """[(kernel name, ms)] of the launches recorded since the last reset."""
    return [(prism_profile_name(i), prism_profile_ms(i))
            for i in range(prism_profile_count())]


def prism_shape_table(out_ptr) -> int:
    return lib().prism_shape_table(out_ptr)


def prism_zone_shapes_workspace_bytes(B, T, H, W, C, zt, zh, zw) -> int:
    return lib().prism_zone_shapes_workspace_bytes(B, T, H, W, C, zt, zh, zw)


def prism_sparse_attn_fwd_workspace_bytes(B, Hh, N, d) -> int:
    return lib().prism_sparse_attn_fwd_workspace_bytes(B, Hh, N, d)


def prism_sparse_attn_bwd_workspace_bytes(B, Hh, N, d) -> int:
    return lib().prism_sparse_attn_bwd_workspace_bytes(B, Hh, N, d)


def prism_zone_shapes(feat, a2v_res, dtype, B, T, H, W, C, zone_t, zone_h,
                      zone_w, lambda_a2v, fixed_shape, zone_shape, perm,
                      inv_perm, zone_stats, workspace, workspace_bytes, stream):
    return _call("prism_zone_shapes", feat, a2v_res, dtype, B, T, H, W, C,
                 zone_t, zone_h, zone_w, lambda_a2v, fixed_shape, zone_shape,
                 perm, inv_perm, zone_stats, workspace, workspace_bytes, stream)


def prism_zone_shapes_noalloc(feat, a2v_res, dtype, B, T, H, W, C, zone_t,
                              zone_h, zone_w, lambda_a2v, fixed_shape,
                              zone_shape, perm, inv_perm, zone_stats, stream):
    return _call("prism_zone_shapes_noalloc", feat, a2v_res, dtype, B, T, H, W,
                 C, zone_t, zone_h, zone_w, lambda_a2v, fixed_shape,
                 zone_shape, perm, inv_perm, zone_stats, stream)


def prism_pool_blocks(q, k, dtype, perm, B, Hh, N, d, q_mean, k_mean, proxy,
                      stream):
    return _call("prism_pool_blocks", q, k, dtype, perm, B, Hh, N, d, q_mean,
                 k_mean, proxy, stream)


def prism_route_blocks_workspace_bytes(B, Hh, N, d) -> int:
    return lib().prism_route_blocks_workspace_bytes(B, Hh, N, d)


def prism_route_blocks(q, k, dtype, perm, B, Hh, N, d, top_k, cdf_threshold,
                       q_mean, k_mean, counts, kv_idx, capacity, workspace,
                       workspace_bytes, stream):
    return _call("prism_route_blocks", q, k, dtype, perm, B, Hh, N, d, top_k,
                 cdf_threshold, q_mean, k_mean, counts, kv_idx, capacity,
                 workspace, workspace_bytes, stream)


def prism_select_blocks(proxy, B, Hh, Nb, top_k, cdf_threshold, counts,
                        kv_idx, capacity, stream):
    return _call("prism_select_blocks", proxy, B, Hh, Nb, top_k,
                 cdf_threshold, counts, kv_idx, capacity, stream)


def prism_sparse_attn_fwd(q, k, v, dtype, perm, counts, kv_idx, capacity, B,
                          Hh, N, d, softmax_scale, o, lse, workspace,
                          workspace_bytes, stream):
    return _call("prism_sparse_attn_fwd", q, k, v, dtype, perm, counts,
                 kv_idx, capacity, B, Hh, N, d, softmax_scale, o, lse,
                 workspace, workspace_bytes, stream)


def prism_dropped_terms_workspace_bytes(B, Hh, N, d) -> int:
    return lib().prism_dropped_terms_workspace_bytes(B, Hh, N, d)


def prism_dropped_terms(proxy, q_mean, k_mean, v, dtype, perm, counts, kv_idx,
                        capacity, B, Hh, N, d, drop_lse, drop_v, workspace,
                        workspace_bytes, stream):
    return _call("prism_dropped_terms", proxy, q_mean, k_mean, v, dtype, perm,
                 counts, kv_idx, capacity, B, Hh, N, d, drop_lse, drop_v,
                 workspace, workspace_bytes, stream)


def prism_sparse_attn_fwd_corrected(q, k, v, dtype, perm, counts, kv_idx,
                                    capacity, B, Hh, N, d, softmax_scale,
                                    drop_lse, drop_v, o, lse, workspace,
                                    workspace_bytes, stream):
    return _call("prism_sparse_attn_fwd_corrected", q, k, v, dtype, perm,
                 counts, kv_idx, capacity, B, Hh, N, d, softmax_scale,
                 drop_lse, drop_v, o, lse, workspace, workspace_bytes, stream)


def prism_a2v_bridge_workspace_bytes(B, N, Na, Cv, Ca, heads) -> int:
    return lib().prism_a2v_bridge_workspace_bytes(B, N, Na, Cv, Ca, heads)


def prism_a2v_bridge(x_v, x_a, w_q, w_k, w_v, w_o, pos_v, pos_a, dtype, B, N,
                     Na, Cv, Ca, heads, rope_base, dh, workspace,
                     workspace_bytes, stream):
    return _call("prism_a2v_bridge", x_v, x_a, w_q, w_k, w_v, w_o, pos_v,
                 pos_a, dtype, B, N, Na, Cv, Ca, heads, rope_base, dh,
                 workspace, workspace_bytes, stream)


def prism_sparse_attn_bwd(q, k, v, o, d_o, lse, dtype, perm, counts, kv_idx,
                          capacity, B, Hh, N, d, softmax_scale, dq, dk, dv,
                          workspace, workspace_bytes, stream):
    return _call("prism_sparse_attn_bwd", q, k, v, o, d_o, lse, dtype, perm,
                 counts, kv_idx, capacity, B, Hh, N, d, softmax_scale, dq, dk,
                 dv, workspace, workspace_bytes, stream)


# ---------------------------------------------------------- torch helpers
def shape_table():
    buf = (ctypes.c_int32 * 39)()
    n = lib().prism_shape_table(ctypes.cast(buf, _c_p))
    return [tuple(buf[3 * i:3 * i + 3]) for i in range(n)]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PRISM_BF16
    if t.dtype == torch.float32:
        return PRISM_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    return _torch().cuda.current_stream().cuda_stream


def zone_shapes(feat, a2v, T: int, H: int, W: int, zone=(8, 8, 8),
                lam: float = 1.0, fixed_shape: int = -1, B: Optional[int] = None,
                with_inverse: bool = True, with_stats: bool = True,
                stream=None):
    """Stage 1.  feat/a2v: [B, N, C] device tensors (or None with a fixed
    shape).  Returns (zone_shape [B,nZ] i32, perm [B,N] i32, inv_perm or None,
    zone_stats [B,nZ,6] f64 or None)."""
    torch = _torch()
    dev = feat.device if feat is not None else torch.device("cuda")
    if feat is not None:
        B, N, C = feat.shape
        dt = _dtype_code(feat)
    else:
        B = 1 if B is None else B
        N, C, dt = T * H * W, 1, PRISM_BF16
    nZ = (-(-T // zone[0])) * (-(-H // zone[1])) * (-(-W // zone[2]))
    zs = torch.empty((B, nZ), dtype=torch.int32, device=dev)
    perm = torch.empty((B, T * H * W), dtype=torch.int32, device=dev)
    inv = torch.empty_like(perm) if with_inverse else None
    stats = (torch.empty((B, nZ, 6), dtype=torch.float64, device=dev)
             if (with_stats and fixed_shape < 0) else None)
    ws_bytes = 0
    ws = None
    if fixed_shape < 0:
        ws_bytes = prism_zone_shapes_workspace_bytes(B, T, H, W, C, *zone)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    prism_zone_shapes(_ptr(feat), _ptr(a2v), dt, B, T, H, W, C, zone[0],
                      zone[1], zone[2], float(lam), int(fixed_shape),
                      _ptr(zs), _ptr(perm), _ptr(inv), _ptr(stats), _ptr(ws),
                      ws_bytes, _stream(stream))
    return zs, perm, inv, stats


def pool_blocks(q, k, perm, stream=None):
    """Stage 2.  q, k: [B, Hh, N, d].  Returns (q_mean, k_mean, proxy)."""
    torch = _torch()
    B, Hh, N, d = q.shape
    Nb = N // 64
    qm = torch.empty((B, Hh, Nb, d), dtype=torch.float64, device=q.device)
    km = torch.empty_like(qm)
    proxy = torch.empty((B, Hh, Nb, Nb), dtype=torch.float64, device=q.device)
    prism_pool_blocks(_ptr(q), _ptr(k), _dtype_code(q), _ptr(perm), B, Hh, N,
                      d, _ptr(qm), _ptr(km), _ptr(proxy), _stream(stream))
    return qm, km, proxy


def select_blocks(proxy, top_k: int, cdf_threshold: float = 0.20,
                  capacity: Optional[int] = None, stream=None):
    """Stage 3.  proxy: [B, Hh, Nb, Nb] fp64.  Returns (counts, kv_idx)."""
    torch = _torch()
    B, Hh, Nb, _ = proxy.shape
    cap = Nb if capacity is None else capacity
    counts = torch.empty((B, Hh, Nb), dtype=torch.int32, device=proxy.device)
    kv_idx = torch.empty((B, Hh, Nb, cap), dtype=torch.int32,
                         device=proxy.device)
    prism_select_blocks(_ptr(proxy), B, Hh, Nb, int(top_k),
                        float(cdf_threshold), _ptr(counts), _ptr(kv_idx), cap,
                        _stream(stream))
    return counts, kv_idx


def route_blocks(q, k, perm, top_k: int, cdf_threshold: float = 0.20,
                 capacity: Optional[int] = None, stream=None):
    """Stages 2-3 fused, without the proxy matrix.  q, k: [B, Hh, N, d].
    Returns (q_mean, k_mean, counts, kv_idx)."""
    torch = _torch()
    B, Hh, N, d = q.shape
    Nb = N // 64
    cap = Nb if capacity is None else capacity
    qm = torch.empty((B, Hh, Nb, d), dtype=torch.float64, device=q.device)
    km = torch.empty_like(qm)
    counts = torch.empty((B, Hh, Nb), dtype=torch.int32, device=q.device)
    kv_idx = torch.empty((B, Hh, Nb, cap), dtype=torch.int32, device=q.device)
    need = prism_route_blocks_workspace_bytes(B, Hh, N, d)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    prism_route_blocks(_ptr(q), _ptr(k), _dtype_code(q), _ptr(perm), B, Hh, N,
                       d, int(top_k), float(cdf_threshold), _ptr(qm), _ptr(km),
                       _ptr(counts), _ptr(kv_idx), cap, _ptr(ws), need,
                       _stream(stream))
    return qm, km, counts, kv_idx


def sparse_attn_fwd(q, k, v, perm, counts, kv_idx,
                    softmax_scale: Optional[float] = None, workspace=None,
                    stream=None):
    """Stage 4 forward.  Returns (o [B,Hh,N,d] q.dtype, lse [B,Hh,N] f32)."""
    torch = _torch()
    B, Hh, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hh, N), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = prism_sparse_attn_fwd_workspace_bytes(B, Hh, N, d)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    scale = -1.0 if softmax_scale is None else float(softmax_scale)
    prism_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q),
                          _ptr(perm), _ptr(counts), _ptr(kv_idx),
                          kv_idx.shape[-1], B, Hh, N, d, scale, _ptr(o),
                          _ptr(lse), _ptr(workspace), workspace.numel(),
                          _stream(stream))
    return o, lse


def sparse_attn_bwd(q, k, v, o, d_o, lse, perm, counts, kv_idx,
                    softmax_scale: Optional[float] = None, workspace=None,
                    stream=None):
    """Stage 4 backward.  Returns fp32 (dq, dk, dv) [B, Hh, N, d]."""
    torch = _torch()
    B, Hh, N, d = q.shape
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    need = prism_sparse_attn_bwd_workspace_bytes(B, Hh, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    scale = -1.0 if softmax_scale is None else float(softmax_scale)
    prism_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o),
                          _ptr(lse), _dtype_code(q), _ptr(perm), _ptr(counts),
                          _ptr(kv_idx), kv_idx.shape[-1], B, Hh, N, d, scale,
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                          workspace.numel(), _stream(stream))
    return dq, dk, dv


def dropped_terms(proxy, q_mean, k_mean, v, perm, counts, kv_idx,
                  workspace=None, stream=None):
    """Stand-in of the unselected blocks (forward-only variant).  Returns
    (drop_lse [B,Hh,Nb] f32, drop_v [B,Hh,Nb,d] f32)."""
    torch = _torch()
    B, Hh, N, d = v.shape
    Nb = N // 64
    drop_lse = torch.empty((B, Hh, Nb), dtype=torch.float32, device=v.device)
    drop_v = torch.empty((B, Hh, Nb, d), dtype=torch.float32, device=v.device)
    if workspace is None:
        need = prism_dropped_terms_workspace_bytes(B, Hh, N, d)
        workspace = torch.empty(need, dtype=torch.uint8, device=v.device)
    prism_dropped_terms(_ptr(proxy), _ptr(q_mean), _ptr(k_mean), _ptr(v),
                        _dtype_code(v), _ptr(perm), _ptr(counts), _ptr(kv_idx),
                        kv_idx.shape[-1], B, Hh, N, d, _ptr(drop_lse),
                        _ptr(drop_v), _ptr(workspace), workspace.numel(),
                        _stream(stream))
    return drop_lse, drop_v


def sparse_attn_fwd_corrected(q, k, v, perm, counts, kv_idx, drop_lse, drop_v,
                              softmax_scale: Optional[float] = None,
                              workspace=None, stream=None):
    """Stage 4 forward with the stand-in of the unselected blocks in the same
    softmax.  Returns (o [B,Hh,N,d] q.dtype, lse [B,Hh,N] f32)."""
    torch = _torch()
    B, Hh, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hh, N), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = prism_sparse_attn_fwd_workspace_bytes(B, Hh, N, d)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    scale = -1.0 if softmax_scale is None else float(softmax_scale)
    prism_sparse_attn_fwd_corrected(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q),
                                    _ptr(perm), _ptr(counts), _ptr(kv_idx),
                                    kv_idx.shape[-1], B, Hh, N, d, scale,
                                    _ptr(drop_lse), _ptr(drop_v), _ptr(o),
                                    _ptr(lse), _ptr(workspace),
                                    workspace.numel(), _stream(stream))
    return o, lse


def a2v_bridge(x_v, x_a, w_q, w_k, w_v, w_o, heads: int, pos_v=None,
               pos_a=None, rope_base: float = 10000.0, workspace=None,
               stream=None):
    """Unscaled a2v bridge residual.  x_v [B, N, Cv], x_a [B, Na, Ca],
    weights [out, in], all bf16; pos_v [B, N] / pos_a [B, Na] fp32 or None.
    Returns dh [B, N, Cv] bf16."""
    torch = _torch()
    B, N, Cv = x_v.shape
    _, Na, Ca = x_a.shape
    dh = torch.empty_like(x_v)
    if workspace is None:
        need = prism_a2v_bridge_workspace_bytes(B, N, Na, Cv, Ca, heads)
        workspace = torch.empty(need, dtype=torch.uint8, device=x_v.device)
    prism_a2v_bridge(_ptr(x_v), _ptr(x_a), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                     _ptr(w_o), _ptr(pos_v), _ptr(pos_a), _dtype_code(x_v), B,
                     N, Na, Cv, Ca, heads, float(rope_base), _ptr(dh),
                     _ptr(workspace), workspace.numel(), _stream(stream))
    return dh
