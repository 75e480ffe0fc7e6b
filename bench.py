#!/usr/bin/env python3
"""Benchmark of the whole dynamic block-shape sparse-attention path on one GPU.

One step = one pass of every stage over one batch of the 2K-grid training
workload (grid 20x90x160 = 288,000 tokens, 24 heads, head_dim 128, bf16,
8x8x8 macro-zones choosing among 13 shapes, top-k 8, cdf_threshold 0.20):

  1. zone shapes + permutation   (video features + a2v residual, C = 3072)
  2. block pooling + fp64 proxy softmax
  3. hybrid top-k / CDF selection
  4. sparse attention forward, then backward (dO ~ N(0, 1))

Inputs are generated on the host from fixed seeds, copied to the GPU, and are
resident in HBM before the timed region; every output and workspace buffer is
allocated once up front.  The JSON line reports the effective sparse-attention
TFLOP/s (algorithmic forward + backward FLOPs on the selected blocks per
second of the whole step), per-stage and per-kernel times (HIP events), the
roofline of the dominant kernel and the fp64 oracle timed on a bounded sample
on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("effective sparse-attn TFLOP/s fwd+bwd @2K grid; selection GB/s; "
          "MFMA % of peak")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP64_TFLOPS = 78.6       # MI355X fp64 (vector and matrix)
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 (vector and matrix)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
BLOCK = 64


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=5,
                    help="workload id in synth.CONFIGS (default: 2K training)")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of host time for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 1 GiB device copy (reference dispatch "
                         "for HBM byte counters)")
    return ap.parse_args()


# Matrix products each backward kernel executes per selected pair, in units
# of 64*64*d FLOP (one 64x64xd product is 2 units): dK/dV recomputes S and dP
# and forms dV, dK (8); dQ recomputes S and dP and forms dQ (6).  The
# algorithmic backward is 10 units per pair (S, dP, dV, dQ, dK, each once),
# so each kernel is credited its executed share of those 10.
BWD_UNITS = 10
BWD_EXEC_UNITS = {"dkdv_bf16": 8, "dq_bf16": 6}


def kernel_work(name, w):
    """(kind, algorithmic amount per launch) of one library kernel.

    kind "mfma": bf16 FLOPs; "fp64": fp64 FLOPs; "fp32": fp32 MFMA FLOPs;
    "hbm": bytes.  The forward counts 4*64^2*d FLOP per selected pair; the
    backward 10*64^2*d per pair, split between dK/dV and dQ in proportion to
    the products each executes (BWD_EXEC_UNITS).
    """
    B, Hh, N, d, Nb, C, sc = (w["B"], w["Hh"], w["N"], w["d"], w["Nb"],
                              w["C"], w["sigma_c"])
    pair = BLOCK * BLOCK * d                    # one 64x64xd product = 2*pair
    esz = 2
    exec_total = sum(BWD_EXEC_UNITS.values())
    table = {
        "attn_fwd_bf16": ("mfma", 4 * pair * sc),
        "dkdv_bf16": ("mfma", BWD_UNITS * BWD_EXEC_UNITS["dkdv_bf16"]
                      / exec_total * pair * sc),
        "dq_bf16": ("mfma", BWD_UNITS * BWD_EXEC_UNITS["dq_bf16"]
                    / exec_total * pair * sc),
        "proxy_logits": ("fp64", 2 * B * Hh * Nb * Nb * d),
        "select_rows": ("hbm", 8 * B * Hh * Nb * Nb + 4 * sc + 4 * B * Hh * Nb),
        "row_softmax": ("hbm", 16 * B * Hh * Nb * Nb),
        "pool_blocks": ("hbm", 2 * B * Hh * N * d * esz + 2 * B * Hh * Nb * d * 8
                        + 4 * B * N * Hh),
        "zone_feat_dev": ("hbm", B * N * C * esz),
        "token_rms": ("hbm", B * N * C * esz + 8 * B * N),
        "bwd_delta": ("hbm", 2 * B * Hh * N * d * esz + 4 * B * Hh * N),
        "bitmap_build": ("hbm", 4 * sc + 4 * B * Hh * Nb),
        "bitmap_transpose": ("hbm", 8 * B * Hh * ((Nb + 31) // 32) * Nb),
        "pair_weights": ("hbm", 4 * B * Hh * ((Nb + 31) // 32) * Nb
                         + 4 * 32 * B * Hh * Nb),
        # forward variant with the stand-in of the unselected blocks
        "pool_values": ("hbm", B * Hh * N * d * esz + 4 * B * Hh * Nb * d
                        + 4 * B * Hh * N),
        "dropped_terms": ("fp32", 2 * B * Hh * Nb * Nb * d),
    }
    return table.get(name, (None, 0))


def counts_histogram(counts, Nb, bins=10):
    """Histogram of the per-row block counts c_i (1 <= c_i <= Nb): `bins`
    equal-width bins over [1, max c_i], as {"edges": [...], "rows": [...]}."""
    import numpy as np
    top = int(min(Nb, counts.max()))
    edges = np.linspace(1, top + 1, bins + 1)
    rows, _ = np.histogram(counts.reshape(-1), bins=edges)
    return {"edges": [int(round(e)) for e in edges], "rows": [int(r) for r in rows]}


def source_sha(kernel_file):
    with open(os.path.join(ROOT, "dynamic_block_sparse_shape_amd", "csrc",
                           kernel_file), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


KERNEL_FILE = {"attn_fwd_bf16": "attn_fwd.hip", "dkdv_bf16": "attn_bwd.hip",
               "dq_bf16": "attn_bwd.hip", "proxy_logits": "pool_proxy.hip",
               "select_rows": "select.hip", "row_softmax": "pool_proxy.hip",
               "pool_blocks": "pool_proxy.hip",
               "zone_feat_dev": "zone_shapes.hip", "token_rms": "zone_shapes.hip"}


def measured_traffic(kernel, workload_name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current source of the kernel (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload_name}.json")
    if not os.path.exists(path) or kernel not in KERNEL_FILE:
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(KERNEL_FILE[kernel]):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------- oracle
def cpu_baseline(x, w, counts_host, perm_host, budget_s):
    """The fp64 oracle on a bounded sample of the same workload, scaled to
    the whole step.  Returns the cpu_baseline record."""
    import numpy as np
    from oracle import prism_oracle as po
    from synth import bf16_bits_to_f32
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1

    def widen(a):
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    cfg = x.cfg
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    zones = po.zone_tiling(T, H, W)
    if x.feat is not None:
        # stage 1: a few full zones
        F = x.feat[0].reshape(T, H, W, -1)
        A = x.a2v[0].reshape(T, H, W, -1)
        nz = min(6, len(zones))
        t0 = time.perf_counter()
        for (o, e) in zones[:nz]:
            sl = (slice(o[0], o[0] + e[0]), slice(o[1], o[1] + e[1]),
                  slice(o[2], o[2] + e[2]))
            st = po.zone_statistics(widen(F[sl]), widen(A[sl]))
            po.choose_shape(st, e)
        t_stage1 = (time.perf_counter() - t0) / nz * len(zones) * w["B"]
        s1 = f"stage 1 on {nz} of {len(zones)} zones"
    else:
        # fixed shape: stage 1 is the permutation alone
        t0 = time.perf_counter()
        po.block_permutation(T, H, W, zones, [cfg["fixed_shape"]] * len(zones))
        t_stage1 = (time.perf_counter() - t0) * w["B"]
        s1 = "stage 1 (fixed-shape permutation) in full"
    # stages 2-3: one whole head
    perm = perm_host[0]
    q0, k0 = widen(x.q[0, 0]), widen(x.k[0, 0])
    t0 = time.perf_counter()
    route = po.route_head(q0, k0, perm, cfg["top_k"], cfg["cdf_threshold"])
    t_route = (time.perf_counter() - t0) * w["B"] * w["Hh"]
    # stage 4: forward + backward of sampled query blocks of head 0 (one call
    # each, as the oracle would run the whole head)
    v0, do0 = widen(x.v[0, 0]), widen(x.do[0, 0])
    rng = np.random.default_rng(0)
    used = min(16, w["Nb"])
    sample = sorted(rng.choice(w["Nb"], size=used, replace=False).tolist())
    pairs = int(sum(int(route["counts"][i]) for i in sample))
    t0 = time.perf_counter()
    po.sparse_attn_fwd(q0, k0, v0, perm, route["lists"], query_blocks=sample)
    po.sparse_attn_bwd(q0, k0, v0, do0, perm, route["lists"],
                       query_blocks=sample)
    t_att = time.perf_counter() - t0
    t_att_full = t_att / max(pairs, 1) * w["sigma_c"]
    total = t_stage1 + t_route + t_att_full
    flops = 14 * BLOCK * BLOCK * w["d"] * w["sigma_c"]
    return {
        "value": flops / total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle: {s1}, "
                   f"stages 2-3 on 1 of {w['Hh']} heads, attention fwd+bwd on "
                   f"{used} query blocks ({pairs} selected pairs) of head 0; "
                   f"extrapolated to the whole step: {total:.1f} s"),
        "seconds_per_step_extrapolated": total,
        "stage_seconds_extrapolated": {"zone_shapes": t_stage1,
                                       "pool_proxy_select": t_route,
                                       "attention_fwd_bwd": t_att_full},
    }


# ------------------------------------------------ forward variant (timed apart)
def bench_dropped_variant(P, args, w, t, dt_code, fwd_plain_ms, stream):
    """The forward variant that keeps a pooled stand-in of the unselected
    blocks in the softmax: prism_dropped_terms + prism_sparse_attn_fwd_corrected
    on the same inputs and routing as the steps, timed after them (it is not
    part of a training step).  Returns the per-call and per-kernel times and
    the roofline of the dropped_terms kernel."""
    import numpy as np
    import torch
    B, Hh, N, d, Nb = w["B"], w["Hh"], w["N"], w["d"], w["Nb"]
    dev = t["q"].device
    sh = stream.cuda_stream
    dl = torch.empty((B, Hh, Nb), dtype=torch.float32, device=dev)
    dv = torch.empty((B, Hh, Nb, d), dtype=torch.float32, device=dev)
    wsd = torch.empty(P.prism_dropped_terms_workspace_bytes(B, Hh, N, d),
                      dtype=torch.uint8, device=dev)
    oc = torch.empty_like(t["q"])
    lc = torch.empty_like(t["lse"])
    p = {n: x.data_ptr() for n, x in t.items()}

    def once(ev=None):
        if ev:
            ev[0].record(stream)
        P.prism_dropped_terms(p["proxy"], p["qm"], p["km"], p["v"], dt_code,
                              p["perm"], p["counts"], p["kv_idx"], Nb, B, Hh,
                              N, d, dl.data_ptr(), dv.data_ptr(),
                              wsd.data_ptr(), wsd.numel(), sh)
        if ev:
            ev[1].record(stream)
        P.prism_sparse_attn_fwd_corrected(
            p["q"], p["k"], p["v"], dt_code, p["perm"], p["counts"],
            p["kv_idx"], Nb, B, Hh, N, d, -1.0, dl.data_ptr(), dv.data_ptr(),
            oc.data_ptr(), lc.data_ptr(), p["wsf"], t["wsf"].numel(), sh)
        if ev:
            ev[2].record(stream)

    once()
    torch.cuda.synchronize()
    reps = max(1, min(args.steps, 3))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(reps)]
    P.prism_profile_enable(1)
    P.prism_profile_reset()
    for r in range(reps):
        once(evs[r])
    torch.cuda.synchronize()
    kt = P.kernel_times()
    P.prism_profile_enable(0)
    per = {}
    for name, ms in kt:
        per.setdefault(name, []).append(ms)
    kernels = {n: {"avg_ms": float(np.mean(v)), "launches": len(v) / reps}
               for n, v in per.items()}
    fl = kernel_work("dropped_terms", w)[1]
    dt_ms = kernels["dropped_terms"]["avg_ms"]
    bytes_ = 8 * B * Hh * Nb * Nb + B * Hh * Nb * ((Nb + 31) // 32) * 4 \
        + 2 * 4 * B * Hh * Nb * d + 4 * B * Hh * Nb
    roof = {"kernel": "dropped_terms", "avg_launch_ms": dt_ms,
            "fp32_tflops": fl / (dt_ms * 1e-3) / 1e12,
            "frac_of_fp32_peak": fl / (dt_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
            "gbs": bytes_ / (dt_ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": bytes_ / (dt_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "algorithmic_flops": fl, "algorithmic_bytes": bytes_}
    return {
        "dropped_terms_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
        "fwd_corrected_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
        "fwd_plain_ms": fwd_plain_ms,
        "dropped_lse_finite_rows": int(torch.isfinite(dl).sum().item()),
        "kernels": kernels,
        "dropped_terms_roofline": roof,
    }


# ------------------------------------------- fused routing (timed apart)
def bench_fused_routing(P, args, w, t, dt_code, cfg, unfused_ms, stream):
    """prism_route_blocks (pooling, proxy scores and selection without the
    [B, Hh, Nb, Nb] proxy matrix) on the same inputs and permutation as the
    steps, timed after them; counts compared with the steps' unfused ones."""
    import numpy as np
    import torch
    B, Hh, N, d, Nb = w["B"], w["Hh"], w["N"], w["d"], w["Nb"]
    dev = t["q"].device
    sh = stream.cuda_stream
    qm = torch.empty((B, Hh, Nb, d), dtype=torch.float64, device=dev)
    km = torch.empty_like(qm)
    counts = torch.empty((B, Hh, Nb), dtype=torch.int32, device=dev)
    kv = torch.empty((B, Hh, Nb, Nb), dtype=torch.int32, device=dev)
    need = P.prism_route_blocks_workspace_bytes(B, Hh, N, d)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def once():
        P.prism_route_blocks(t["q"].data_ptr(), t["k"].data_ptr(), dt_code,
                             t["perm"].data_ptr(), B, Hh, N, d, cfg["top_k"],
                             cfg["cdf_threshold"], qm.data_ptr(), km.data_ptr(),
                             counts.data_ptr(), kv.data_ptr(), Nb, ws.data_ptr(),
                             need, sh)

    once()
    torch.cuda.synchronize()
    reps = max(1, min(args.steps, 5))
    P.prism_profile_enable(1)
    P.prism_profile_reset()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        once()
    ev[1].record(stream)
    torch.cuda.synchronize()
    kt = P.kernel_times()
    P.prism_profile_enable(0)
    per = {}
    for name, ms in kt:
        per.setdefault(name, []).append(ms)
    kernels = {n: {"avg_ms": float(np.mean(v)), "launches": len(v) / reps}
               for n, v in per.items()}
    flops = 2 * B * Hh * Nb * Nb * d
    rr = kernels["route_rows"]["avg_ms"]
    # the kbar re-layout is part of the fused call's time (kernels: pooling,
    # kbar_pairs, route_rows)
    same = int((counts == t["counts"]).sum().item())
    return {
        "ms": ev[0].elapsed_time(ev[1]) / reps,
        "unfused_ms": unfused_ms,
        "kernels": kernels,
        "route_rows_fp64_tflops": flops / (rr * 1e-3) / 1e12,
        "route_rows_frac_of_fp64_peak": flops / (rr * 1e-3) / 1e12 / PEAK_FP64_TFLOPS,
        "proxy_matrix_bytes_avoided": 8 * B * Hh * Nb * Nb,
        "hbm_footprint_bytes": 16 * B * Hh * Nb * d + need,
        "unfused_hbm_footprint_bytes": 16 * B * Hh * Nb * d + 8 * B * Hh * Nb * Nb,
        "rows_with_unfused_count": same,
        "rows": B * Hh * Nb,
    }


# ------------------------------------------- a2v bridge (timed apart)
def bench_bridge(P, args, x, w, stream):
    """prism_a2v_bridge on the workload's video features (its hidden states)
    and random-weight audio inputs: the producer of stage 1's residual,
    timed after the steps (it belongs to the bridge layer, not the sparse
    attention step)."""
    import numpy as np
    import torch
    from synth import make_bridge_inputs
    cfg = x.cfg
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    B, N, C = w["B"], w["N"], w["C"]
    heads, Ca = 24, 1536
    br = make_bridge_inputs(T, H, W, B=B, Cv=C, Ca=Ca, heads=heads, seed=2500)
    Na = br.x_a.shape[1]
    dev = torch.device("cuda", 0)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    xv = x.dev_feat
    xa, wq, wk, wv, wo, pv, pa = (up(a) for a in (br.x_a, br.w_q, br.w_k, br.w_v,
                                                  br.w_o, br.pos_v, br.pos_a))
    dh = torch.empty_like(xv)
    need = P.prism_a2v_bridge_workspace_bytes(B, N, Na, C, Ca, heads)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    sh = stream.cuda_stream

    def once():
        P.prism_a2v_bridge(xv.data_ptr(), xa.data_ptr(), wq.data_ptr(),
                           wk.data_ptr(), wv.data_ptr(), wo.data_ptr(),
                           pv.data_ptr(), pa.data_ptr(), P.PRISM_BF16, B, N, Na,
                           C, Ca, heads, 10000.0, dh.data_ptr(), ws.data_ptr(),
                           need, sh)

    once()
    torch.cuda.synchronize()
    reps = max(1, min(args.steps, 5))
    P.prism_profile_enable(1)
    P.prism_profile_reset()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        once()
    ev[1].record(stream)
    torch.cuda.synchronize()
    kt = P.kernel_times()
    P.prism_profile_enable(0)
    D = 128 * heads
    # launch order per call: q, k, v projections, attention, output projection
    work = [2 * B * N * C * D, 2 * B * Na * Ca * D, 2 * B * Na * Ca * D,
            4 * B * N * Na * D, 2 * B * N * D * C]
    names = ["q_proj", "k_proj", "v_proj", "attention", "out_proj"]
    per = {n: [] for n in names}
    for i, (_, ms) in enumerate(kt):
        per[names[i % 5]].append(ms)
    launches = {}
    for n, fl in zip(names, work):
        ms = float(np.mean(per[n]))
        launches[n] = {"avg_ms": ms, "tflops": fl / (ms * 1e-3) / 1e12,
                       "frac_of_bf16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    total_ms = ev[0].elapsed_time(ev[1]) / reps
    return {"ms": total_ms, "audio_tokens": Na, "heads": heads,
            "video_width": C, "audio_width": Ca,
            "tflops": sum(work) / (total_ms * 1e-3) / 1e12,
            "frac_of_bf16_peak": sum(work) / (total_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "launches": launches}


# ------------------------------------------------------------------ main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; "
                          "--gpus above 1 is not supported"}))
        sys.exit(2)

    import numpy as np
    import torch

    import dynamic_block_sparse_shape_amd as P
    from synth import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    t0 = time.perf_counter()
    x = make_inputs(args.workload, with_grad=True)
    _log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    B, Hh, d = cfg["B"], cfg["Hh"], cfg["d"]
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    N = T * H * W
    Nb = N // BLOCK
    C = cfg.get("C", 0)
    dyn = cfg["dynamic"]
    bf16 = cfg["dtype"] == "bf16"
    dt_code = P.PRISM_BF16 if bf16 else P.PRISM_FP32

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v, do = up(x.q), up(x.k), up(x.v), up(x.do)
    feat = up(x.feat) if dyn else None
    a2v = up(x.a2v) if dyn else None
    zone = (8, 8, 8)
    nZ = math.ceil(T / 8) * math.ceil(H / 8) * math.ceil(W / 8)
    zs = torch.empty((B, nZ), dtype=torch.int32, device=dev)
    perm = torch.empty((B, N), dtype=torch.int32, device=dev)
    ws1_bytes = P.prism_zone_shapes_workspace_bytes(B, T, H, W, max(C, 8), *zone)
    ws1 = torch.empty(max(ws1_bytes, 1), dtype=torch.uint8, device=dev)
    qm = torch.empty((B, Hh, Nb, d), dtype=torch.float64, device=dev)
    km = torch.empty_like(qm)
    proxy = torch.empty((B, Hh, Nb, Nb), dtype=torch.float64, device=dev)
    counts = torch.empty((B, Hh, Nb), dtype=torch.int32, device=dev)
    kv_idx = torch.empty((B, Hh, Nb, Nb), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hh, N), dtype=torch.float32, device=dev)
    dq = torch.empty((B, Hh, N, d), dtype=torch.float32, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    wsb_bytes = P.prism_sparse_attn_bwd_workspace_bytes(B, Hh, N, d)
    wsb = torch.empty(wsb_bytes, dtype=torch.uint8, device=dev)
    wsf = torch.empty(P.prism_sparse_attn_fwd_workspace_bytes(B, Hh, N, d),
                      dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def ptr(t):
        return None if t is None else t.data_ptr()

    stage_names = ["zone_shapes", "pool_proxy", "select", "attn_fwd", "attn_bwd"]

    def step(events=None):
        def mark(i):
            if events is not None:
                events[i].record(stream)
        mark(0)
        P.prism_zone_shapes(ptr(feat), ptr(a2v), dt_code, B, T, H, W, max(C, 8),
                            *zone, 1.0, -1 if dyn else cfg["fixed_shape"],
                            ptr(zs), ptr(perm), None, None, ptr(ws1), ws1.numel(),
                            sh)
        mark(1)
        P.prism_pool_blocks(ptr(q), ptr(k), dt_code, ptr(perm), B, Hh, N, d,
                            ptr(qm), ptr(km), ptr(proxy), sh)
        mark(2)
        P.prism_select_blocks(ptr(proxy), B, Hh, Nb, cfg["top_k"],
                              cfg["cdf_threshold"], ptr(counts), ptr(kv_idx), Nb,
                              sh)
        mark(3)
        P.prism_sparse_attn_fwd(ptr(q), ptr(k), ptr(v), dt_code, ptr(perm),
                                ptr(counts), ptr(kv_idx), Nb, B, Hh, N, d, -1.0,
                                ptr(o), ptr(lse), ptr(wsf), wsf.numel(), sh)
        mark(4)
        P.prism_sparse_attn_bwd(ptr(q), ptr(k), ptr(v), ptr(o), ptr(do), ptr(lse),
                                dt_code, ptr(perm), ptr(counts), ptr(kv_idx), Nb,
                                B, Hh, N, d, -1.0, ptr(dq), ptr(dk), ptr(dv),
                                ptr(wsb), wsb.numel(), sh)
        mark(5)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        _log("copy calibration: 3 x 1 GiB device copies done")

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        _log(f"warmup step {i + 1}/{args.warmup} done")
    counts_host = counts.cpu().numpy()
    sigma_c = int(counts_host.astype(np.int64).sum())

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)]
           for _ in range(args.steps)]
    P.prism_profile_enable(1)
    P.prism_profile_reset()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    kt = P.kernel_times()
    P.prism_profile_enable(0)
    _log(f"timed {args.steps} steps in {t_total:.3f} s")

    stage_ms = {n: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1])
                                  for s in range(args.steps)]))
                for i, n in enumerate(stage_names)}
    ms_per_step = t_total * 1e3 / args.steps
    per_kernel = {}
    for name, ms in kt:
        per_kernel.setdefault(name, []).append(ms)
    w = dict(B=B, Hh=Hh, N=N, d=d, Nb=Nb, C=C, sigma_c=sigma_c)
    kernels = {}
    for name, lst in per_kernel.items():
        launches = len(lst) / args.steps
        avg = float(np.mean(lst))
        kind, amount = kernel_work(name, w)
        rec = {"avg_ms": avg, "launches_per_step": launches}
        if kind == "mfma":
            rec["tflops"] = amount / (avg * 1e-3) / 1e12
            rec["frac_of_bf16_peak"] = rec["tflops"] / PEAK_BF16_TFLOPS
            if name in BWD_EXEC_UNITS:
                # products the kernel actually runs (recomputed S, dP included)
                ex = BWD_EXEC_UNITS[name] * BLOCK * BLOCK * d * sigma_c
                rec["executed_mfma_tflops"] = ex / (avg * 1e-3) / 1e12
                rec["executed_frac_of_bf16_peak"] = (
                    rec["executed_mfma_tflops"] / PEAK_BF16_TFLOPS)
        elif kind == "fp64":
            rec["tflops_fp64"] = amount / (avg * 1e-3) / 1e12
            rec["frac_of_fp64_peak"] = rec["tflops_fp64"] / PEAK_FP64_TFLOPS
        elif kind == "hbm":
            rec["gbs"] = amount / (avg * 1e-3) / 1e9
            rec["frac_of_hbm_peak"] = rec["gbs"] / PEAK_HBM_GBS
        kernels[name] = rec

    pair = BLOCK * BLOCK * d
    flops_fwd = 4 * pair * sigma_c
    flops_bwd = 10 * pair * sigma_c
    value = (flops_fwd + flops_bwd) / (ms_per_step * 1e-3) / 1e12
    sel_bytes = 8 * B * Hh * Nb * Nb + 4 * sigma_c + 4 * B * Hh * Nb
    sel_ms = kernels.get("select_rows", {}).get("avg_ms", stage_ms["select"])

    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] * kernels[n]["launches_per_step"])
    kind, amount = kernel_work(dom, w)
    dom_ms = kernels[dom]["avg_ms"]
    if kind == "mfma":
        roof = {"bound": "mfma", "achieved": amount / (dom_ms * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    elif kind == "fp64":
        roof = {"bound": "alu", "achieved": amount / (dom_ms * 1e-3) / 1e12,
                "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": amount / (dom_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom, cfg["name"])
    roof["kernel"] = dom
    roof["avg_launch_ms"] = dom_ms
    roof["algorithmic_per_launch"] = amount
    if dom in BWD_EXEC_UNITS:
        roof["algorithmic_rule"] = (
            f"backward 10*64^2*d FLOP per selected pair, {dom} credited "
            f"{BWD_EXEC_UNITS[dom]}/{sum(BWD_EXEC_UNITS.values())} of it")

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "grid_thw": [T, H, W], "tokens": N,
                   "batch": B, "heads": Hh, "head_dim": d, "zone": list(zone),
                   "dynamic_shapes": dyn, "feature_dim": C,
                   "top_k": cfg["top_k"], "cdf_threshold": cfg["cdf_threshold"],
                   "passes": "zone_shapes+pool_proxy+select+attn_fwd+attn_bwd"},
        "roofline": roof,
        "selection_gbs": sel_bytes / (sel_ms * 1e-3) / 1e9,
        "attn_fwd_tflops": kernels.get("attn_fwd_bf16", {}).get("tflops"),
        "attn_fwd_bwd_tflops_stage4": (flops_fwd + flops_bwd) /
        ((stage_ms["attn_fwd"] + stage_ms["attn_bwd"]) * 1e-3) / 1e12,
        "attn_bwd_tflops": flops_bwd / (stage_ms["attn_bwd"] * 1e-3) / 1e12,
        "attn_bwd_frac_of_bf16_peak": flops_bwd / (stage_ms["attn_bwd"] * 1e-3)
        / 1e12 / PEAK_BF16_TFLOPS,
        "mfma_frac": {n: r.get("frac_of_bf16_peak") for n, r in kernels.items()
                      if "frac_of_bf16_peak" in r},
        "density": sigma_c / (B * Hh * Nb * Nb),
        "sigma_c": sigma_c,
        "counts_mean": float(counts_host.mean()),
        "counts_max": int(counts_host.max()),
        "counts_hist": counts_histogram(counts_host, Nb),
        "stage_ms": stage_ms,
        "kernels": kernels,
    }
    out["variants"] = {"fwd_with_dropped_stand_in": bench_dropped_variant(
        P, args, w, dict(q=q, k=k, v=v, perm=perm, qm=qm, km=km, proxy=proxy,
                         counts=counts, kv_idx=kv_idx, wsf=wsf, lse=lse),
        dt_code, stage_ms["attn_fwd"], stream)}
    _log("variant: forward with the stand-in done")
    out["variants"]["fused_routing"] = bench_fused_routing(
        P, args, w, dict(q=q, k=k, perm=perm, counts=counts), dt_code, cfg,
        stage_ms["pool_proxy"] + stage_ms["select"], stream)
    _log("variant: fused routing done")
    if dyn and bf16:
        x.dev_feat = feat
        out["variants"]["a2v_bridge"] = bench_bridge(P, args, x, w, stream)
        _log("variant: a2v bridge done")
    if not args.no_cpu_baseline:
        perm_host = perm.cpu().numpy()
        t0 = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(x, w, counts_host, perm_host,
                                           args.cpu_budget)
        _log(f"cpu baseline took {time.perf_counter() - t0:.1f} s")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
