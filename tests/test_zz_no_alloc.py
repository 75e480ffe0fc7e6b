"""The allocation-free stage-1 entry point (prism_zone_shapes_noalloc)
against prism_zone_shapes: bit-identical zone shapes, permutation, inverse
permutation and zone statistics, on two calls in a row whose second input is
smaller (the library's scratch array keeps the first call's contents), plus a
fixed-shape call.  All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_shape_amd as P
from synth import CONFIGS, make_inputs
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _case(T, H, W, C, B, seed):
    cfg = dict(CONFIGS[2])
    cfg.update(T=T, H=H, W=W, C=C, B=B, Hh=1, seed=seed, name="noalloc")
    x = make_inputs(cfg)
    return to_dev(x.feat), to_dev(x.a2v)


def _outputs(B, T, H, W):
    nZ = -(-T // 8) * -(-H // 8) * -(-W // 8)
    dev = torch.device("cuda")
    return (torch.full((B, nZ), -5, dtype=torch.int32, device=dev),
            torch.full((B, T * H * W), -5, dtype=torch.int32, device=dev),
            torch.full((B, T * H * W), -5, dtype=torch.int32, device=dev),
            torch.full((B, nZ, 6), float("nan"), dtype=torch.float64, device=dev))


def _run(feat, a2v, B, T, H, W, C, fixed, noalloc, lam=1.0):
    zs, perm, inv, st = _outputs(B, T, H, W)
    sh = torch.cuda.current_stream().cuda_stream
    fp = feat.data_ptr() if feat is not None else None
    ap = a2v.data_ptr() if a2v is not None else None
    stats = st.data_ptr() if fixed < 0 else None
    if noalloc:
        P.prism_zone_shapes_noalloc(fp, ap, P.PRISM_BF16, B, T, H, W, C, 8, 8,
                                    8, lam, fixed, zs.data_ptr(),
                                    perm.data_ptr(), inv.data_ptr(), stats, sh)
    else:
        need = P.prism_zone_shapes_workspace_bytes(B, T, H, W, C, 8, 8, 8)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        P.prism_zone_shapes(fp, ap, P.PRISM_BF16, B, T, H, W, C, 8, 8, 8, lam,
                            fixed, zs.data_ptr(), perm.data_ptr(),
                            inv.data_ptr(), stats, ws.data_ptr(), need, sh)
    torch.cuda.synchronize()
    return zs, perm, inv, (st if fixed < 0 else None)


def _same(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        assert torch.equal(x, y)


def test_noalloc_matches_workspace_entry_point():
    calls = [(20, 36, 48, 1024, 2, 501), (8, 16, 16, 256, 1, 502)]
    for T, H, W, C, B, seed in calls:
        print("noalloc call", (T, H, W), C, B, flush=True)
        need = P.prism_zone_shapes_workspace_bytes(B, T, H, W, C, 8, 8, 8)
        assert 0 < need <= 32 << 20          # within the fixed scratch
        feat, a2v = _case(T, H, W, C, B, seed)
        ref = _run(feat, a2v, B, T, H, W, C, -1, noalloc=False)
        got = _run(feat, a2v, B, T, H, W, C, -1, noalloc=True)
        _same(got, ref)
        # no audio term, another lambda
        _same(_run(feat, None, B, T, H, W, C, -1, noalloc=True, lam=0.5),
              _run(feat, None, B, T, H, W, C, -1, noalloc=False, lam=0.5))
        if B == 2:                          # the larger grid: 90 zones
            assert len(set(ref[0].cpu().numpy().ravel().tolist())) >= 3
    # a fixed shape needs no scratch
    _same(_run(None, None, 1, 4, 8, 8, 8, 1, noalloc=True),
          _run(None, None, 1, 4, 8, 8, 8, 1, noalloc=False))
