"""The C ABI library loads, exports every declared entry point, and rejects
invalid arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import dynamic_block_sparse_shape_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prism.h")

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = P.lib()
    names = _declared()
    assert len(names) == 24, names
    for n in names:
        assert hasattr(L, n), n
    # the Python binding carries the same names
    for n in names:
        assert hasattr(P, n), n


def test_shape_table():
    tbl = P.shape_table()
    assert len(tbl) == 13
    assert tbl[0] == (4, 4, 4) and (8, 2, 4) in tbl and (2, 4, 8) in tbl
    assert all(t * h * w == 64 for t, h, w in tbl)
    assert P.lib().prism_shape_table(None) == 13
    assert P.prism_version() >= 100


def test_workspace_queries():
    n = P.prism_zone_shapes_workspace_bytes(1, 20, 90, 160, 3072, 8, 8, 8)
    # 720 zones x 96 fp32 slices x 3 doubles + one double per token
    assert n >= 720 * 96 * 3 * 8 + 288000 * 8
    assert P.prism_zone_shapes_workspace_bytes(1, 20, 90, 161, 3072, 8, 8, 8) == 0
    nb = 4500
    m = P.prism_sparse_attn_bwd_workspace_bytes(1, 24, 288000, 128)
    assert m >= 24 * 288000 * 4 + 24 * nb * ((nb + 31) // 32) * 4
    assert P.prism_sparse_attn_bwd_workspace_bytes(1, 24, 288000, 96) == 0
    f = P.prism_sparse_attn_fwd_workspace_bytes(1, 24, 288000, 128)
    # two list bitmaps (columns, rows) and the pairing
    assert f >= 2 * 24 * nb * ((nb + 31) // 32) * 4 + 24 * ((nb + 1) // 2) * 8
    assert P.prism_sparse_attn_fwd_workspace_bytes(1, 24, 288000, 96) == 0
    assert m >= f


def _expect(status, fn, *args, **kw):
    with pytest.raises(P.PrismError) as ei:
        fn(*args, **kw)
    assert ei.value.status == status, str(ei.value)
    assert P.prism_last_error() != ""


def test_zone_shapes_noalloc_rejections():
    """The allocation-free stage-1 call checks its arguments like
    prism_zone_shapes and refuses calls whose scratch exceeds the library's
    fixed array, all before any HIP call."""
    base = dict(feat=FAKE, a2v_res=FAKE, dtype=1, B=1, T=20, H=90, W=160,
                C=3072, zone_t=8, zone_h=8, zone_w=8, lambda_a2v=1.0,
                fixed_shape=-1, zone_shape=FAKE, perm=FAKE, inv_perm=None,
                zone_stats=None, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return P.prism_zone_shapes_noalloc(*a.values())

    limit = 32 << 20
    need = P.prism_zone_shapes_workspace_bytes(8, 20, 90, 160, 3072, 8, 8, 8)
    assert need > limit
    _expect(4, call, B=8)                         # scratch above the limit
    _expect(2, call, W=161)                       # N % 64 != 0
    _expect(1, call, feat=None)
    _expect(1, call, dtype=7)
    _expect(1, call, perm=FAKE + 2)               # misaligned
    assert P.prism_zone_shapes_workspace_bytes(1, 20, 90, 160, 3072, 8, 8,
                                               8) <= limit


def test_zone_shapes_rejections():
    zs = dict(feat=FAKE, a2v_res=FAKE, dtype=1, B=1, T=20, H=68, W=120, C=3072,
              zone_t=8, zone_h=8, zone_w=8, lambda_a2v=1.0, fixed_shape=-1,
              zone_shape=FAKE, perm=FAKE, inv_perm=None, zone_stats=None,
              workspace=FAKE, workspace_bytes=1 << 40, stream=None)

    def call(**kw):
        a = dict(zs)
        a.update(kw)
        return P.prism_zone_shapes(*a.values())

    _expect(2, call, W=121)                       # N % 64 != 0
    _expect(1, call, feat=None)                   # dynamic needs features
    _expect(1, call, perm=None)
    _expect(1, call, dtype=7)
    _expect(1, call, B=0)
    _expect(1, call, fixed_shape=13)
    _expect(2, call, fixed_shape=5, T=20)         # (8,2,4) vs T-remainder 4
    _expect(3, call, zone_t=16)
    _expect(3, call, C=3070)
    _expect(4, call, workspace_bytes=16)
    _expect(4, call, workspace=None)
    _expect(1, call, lambda_a2v=-1.0)
    # a grid whose remainder zone admits no shape: 4 x 1 x 8 remainder
    _expect(2, call, T=4, H=9, W=64, fixed_shape=-1)


def test_pool_select_rejections():
    _expect(3, P.prism_pool_blocks, FAKE, FAKE, 1, FAKE, 1, 2, 256, 96, FAKE,
            FAKE, FAKE, None)
    _expect(2, P.prism_pool_blocks, FAKE, FAKE, 1, FAKE, 1, 2, 250, 64, FAKE,
            FAKE, FAKE, None)
    _expect(1, P.prism_pool_blocks, None, FAKE, 1, FAKE, 1, 2, 256, 64, FAKE,
            FAKE, FAKE, None)
    _expect(3, P.prism_pool_blocks, FAKE, FAKE, 1, FAKE, 1, 1, 64 * 8193, 64,
            FAKE, FAKE, FAKE, None)
    _expect(1, P.prism_select_blocks, FAKE, 1, 2, 4, -1, 0.2, FAKE, FAKE, 4,
            None)
    _expect(1, P.prism_select_blocks, FAKE, 1, 2, 4, 1, 1.5, FAKE, FAKE, 4,
            None)
    _expect(1, P.prism_select_blocks, FAKE, 1, 2, 4, 1, float("nan"), FAKE,
            FAKE, 4, None)
    _expect(2, P.prism_select_blocks, FAKE, 1, 2, 4, 1, 0.2, FAKE, FAKE, 3,
            None)
    _expect(3, P.prism_select_blocks, FAKE, 1, 1, 8193, 1, 0.2, FAKE, FAKE,
            8193, None)
    _expect(1, P.prism_select_blocks, FAKE, 1, 2, 4, 1, 0.2, None, FAKE, 4,
            None)


def test_attention_rejections():
    base = [FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 4, 1, 2, 256, 128, -1.0,
            FAKE, FAKE, None, 0, None]
    _expect(3, P.prism_sparse_attn_fwd, *(base[:11] + [80] + base[12:]))
    _expect(2, P.prism_sparse_attn_fwd, *(base[:7] + [3] + base[8:]))
    _expect(1, P.prism_sparse_attn_fwd, *([None] + base[1:]))
    _expect(1, P.prism_sparse_attn_fwd, *(base[:13] + [None] + base[14:]))
    _expect(1, P.prism_sparse_attn_fwd, *(base[:3] + [2] + base[4:]))
    _expect(1, P.prism_sparse_attn_fwd, *(base[:12] + [float("inf")] + base[13:]))
    # more than 8192 blocks per head is not supported
    big = base[:10] + [64 * 8193] + base[11:]
    big[7] = 8193
    _expect(3, P.prism_sparse_attn_fwd, *big)
    # the bf16 path needs its workspace (list bitmaps and the block pairing)
    _expect(4, P.prism_sparse_attn_fwd, *base)
    _expect(4, P.prism_sparse_attn_fwd, *(base[:15] + [FAKE, 16] + base[17:]))
    bwd = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 4, 1, 2,
           256, 128, -1.0, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    _expect(4, P.prism_sparse_attn_bwd, *(bwd[:20] + [8] + bwd[21:]))
    _expect(4, P.prism_sparse_attn_bwd, *(bwd[:19] + [None] + bwd[20:]))
    _expect(1, P.prism_sparse_attn_bwd, *(bwd[:4] + [None] + bwd[5:]))
    _expect(3, P.prism_sparse_attn_bwd, *(bwd[:14] + [32] + bwd[15:]))
    bigb = bwd[:13] + [64 * 8193] + bwd[14:]
    bigb[10] = 8193
    _expect(3, P.prism_sparse_attn_bwd, *bigb)


def test_misaligned_pointers_rejected():
    """Tensors are accessed with 16-byte vectors: misaligned pointers are
    refused before any HIP call."""
    zs = dict(feat=FAKE + 8, a2v_res=FAKE, dtype=1, B=1, T=20, H=68, W=120,
              C=3072, zone_t=8, zone_h=8, zone_w=8, lambda_a2v=1.0,
              fixed_shape=-1, zone_shape=FAKE, perm=FAKE, inv_perm=None,
              zone_stats=None, workspace=FAKE, workspace_bytes=1 << 40,
              stream=None)
    _expect(1, P.prism_zone_shapes, *zs.values())
    zs.update(feat=FAKE, perm=FAKE + 2)
    _expect(1, P.prism_zone_shapes, *zs.values())
    _expect(1, P.prism_pool_blocks, FAKE + 4, FAKE, 1, FAKE, 1, 2, 256, 64,
            FAKE, FAKE, FAKE, None)
    _expect(1, P.prism_pool_blocks, FAKE, FAKE, 1, FAKE, 1, 2, 256, 64,
            FAKE, FAKE, FAKE + 8, None)
    _expect(1, P.prism_select_blocks, FAKE, 1, 2, 4, 1, 0.2, FAKE + 2, FAKE,
            4, None)
    base = [FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 4, 1, 2, 256, 128, -1.0,
            FAKE, FAKE, None, 0, None]
    _expect(1, P.prism_sparse_attn_fwd, *([FAKE + 8] + base[1:]))
    _expect(1, P.prism_sparse_attn_fwd, *(base[:13] + [FAKE + 8] + base[14:]))
    bwd = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 4, 1, 2,
           256, 128, -1.0, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    _expect(1, P.prism_sparse_attn_bwd, *(bwd[:16] + [FAKE + 4] + bwd[17:]))
    _expect(1, P.prism_sparse_attn_bwd, *(bwd[:19] + [FAKE + 8] + bwd[20:]))


def test_dropped_terms_rejections():
    """The forward-only variant with the stand-in of the unselected blocks:
    the same host-side checks as the attention calls."""
    nb = 4500
    w = P.prism_dropped_terms_workspace_bytes(1, 24, 288000, 128)
    # block means of v (fp32) and two list bitmaps
    assert w >= 24 * nb * 128 * 4 + 2 * 24 * nb * ((nb + 31) // 32) * 4
    assert P.prism_dropped_terms_workspace_bytes(1, 24, 288000, 96) == 0
    dt = [FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 4, 1, 2, 256, 128,
          FAKE, FAKE, FAKE, 1 << 30, None]
    _expect(3, P.prism_dropped_terms, *(dt[:12] + [96] + dt[13:]))
    _expect(2, P.prism_dropped_terms, *(dt[:11] + [250] + dt[12:]))
    _expect(2, P.prism_dropped_terms, *(dt[:8] + [3] + dt[9:]))
    _expect(1, P.prism_dropped_terms, *([None] + dt[1:]))
    _expect(1, P.prism_dropped_terms, *(dt[:14] + [None] + dt[15:]))
    _expect(1, P.prism_dropped_terms, *(dt[:4] + [5] + dt[5:]))
    _expect(1, P.prism_dropped_terms, *(dt[:14] + [FAKE + 4] + dt[15:]))
    _expect(4, P.prism_dropped_terms, *(dt[:15] + [None] + dt[16:]))
    _expect(4, P.prism_dropped_terms, *(dt[:16] + [64] + dt[17:]))
    big = dt[:11] + [64 * 8193] + dt[12:]
    big[8] = 8193
    _expect(3, P.prism_dropped_terms, *big)
    fc = [FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 4, 1, 2, 256, 128, -1.0,
          FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    _expect(1, P.prism_sparse_attn_fwd_corrected, *(fc[:13] + [None] + fc[14:]))
    _expect(1, P.prism_sparse_attn_fwd_corrected, *(fc[:14] + [None] + fc[15:]))
    _expect(1, P.prism_sparse_attn_fwd_corrected, *(fc[:14] + [FAKE + 4] + fc[15:]))
    _expect(3, P.prism_sparse_attn_fwd_corrected, *(fc[:11] + [80] + fc[12:]))
    _expect(4, P.prism_sparse_attn_fwd_corrected, *(fc[:18] + [16] + fc[19:]))
    _expect(4, P.prism_sparse_attn_fwd_corrected, *(fc[:17] + [None] + fc[18:]))
