"""Benchmark of the MXFP8 x MXFP4 MoE expert layer on one MI355X.

A step is one full layer call (route, quant, permute, FC1 + SiTU + requant,
FC2 + combine) over one batch of synthetic input already resident in HBM.
Default workload: the decode batch (T = 8 tokens, H = 7168, I = 3584,
896 experts, top-16).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_T8]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

import synth

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_FP8_PEAK_TFLOPS = 5000.0  # dense MXFP8-rate scaled MFMA (f8 x f4 issues at this rate)

WORKLOADS = synth.WORKLOADS


# The pages' own latency for the checkpoint-true "ep_mixed" runner workload
# (FlashInfer CUTLASS MXFP8 x MXFP4, SiTU(4, 25), RTX PRO 6000D / SM120;
# page 1, "Phase 4 算子性能与 Profiler 归因", "五轮交错 A/B" table): local batch M
# -> median ms.  Another machine's figure: context for vs_baseline.
PAGES_EP_MIXED_MS = {128: 0.926, 512: 1.782, 2048: 4.355, 8192: 16.167}

# Sources of the FC kernels: a traffic figure is valid only for their code.
FC_SOURCES = ("common.h", "fc_common.h", "tiled.h", "fc.hip", "fc_prefill.hip")


def _code_text(src):
    """Source text without comments and blank space, so that a counter
    record stays valid across edits that change no code."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def fc_source_sha():
    h = hashlib.sha256()
    for name in FC_SOURCES:
        with open(os.path.join(ROOT, "mxfp8_mxfp4_experts_amd", "csrc", name)) as f:
            h.update(_code_text(f.read()).encode())
    return h.hexdigest()


def _traffic(workload):
    """HBM bytes per FC1 launch from committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel's reading), if they
    were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "fc1_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        rec = d.get(workload)
        if rec and rec.get("source_sha256") == fc_source_sha():
            return rec["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None
    return None


def copy_calibration():
    """A plain device copy of known size (1 GiB read + 1 GiB written), three
    times: the reference reading for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def cpu_baseline(cfg, act, weights_dev, topk_idx, topk_w, min_s=10.0):
    """The oracle, as it stands, on a bounded sample: the workload's tokens
    from the first, one at a time, each evaluated route by route, until at
    least min_s seconds have passed or the tokens run out.  Returns tokens/s,
    threads used, seconds and tokens."""
    import oracle
    from threadpoolctl import threadpool_info

    def weight_fn(e):
        return tuple(weights_dev[k][e].cpu().numpy() for k in ("w13", "w13_s", "w2", "w2_s"))

    t0 = time.perf_counter()
    n = 0
    while n < cfg.T and (n == 0 or time.perf_counter() - t0 < min_s):
        oracle.oracle_tokens([n], act["x_bf16"], topk_idx, topk_w, weight_fn, top_k=cfg.K,
                             expert_offset=cfg.expert_offset, E_local=cfg.E_local)
        n += 1
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return n / dt, threads, dt, n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rounds", type=int, default=1,
                    help="timed rounds of --steps steps each; the step time is their median")
    ap.add_argument("--workload", default="decode_T8", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    import mxfp8_mxfp4_experts_amd as m

    cfg = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()
    if cfg.H == 7168:
        wcfg = synth.custom_config("w", 0, T=1, H=cfg.H, I=cfg.I, E=cfg.E, K=1, E_local=cfg.E)
        w_all = synth.make_expert_weights(wcfg, device=dev)
        sl = slice(cfg.expert_offset, cfg.expert_offset + cfg.E_local)
        w = {k: v[sl] for k, v in w_all.items()}
    elif cfg.routing == "ep_mixed":
        w = synth.make_expert_weights(cfg, device=dev)
    else:
        w = {k: v.to(dev) for k, v in synth.make_expert_weights(cfg, device="cpu").items()}
    act = synth.make_activations(cfg)
    x = torch.from_numpy(act["x_bf16"].astype(np.int16)).to(dev).view(torch.bfloat16)
    # "ep_mixed" workloads take their top-k ids and weights as inputs (the
    # pages' harness does the same); the others route from the logits.
    given = cfg.routing == "ep_mixed"
    logits = None if given else torch.from_numpy(act["logits"]).to(dev)
    bias = None if given else torch.from_numpy(act["bias"]).to(dev)
    layer = m.MoELayer(w["w13"], w["w13_s"], w["w2"], w["w2_s"], top_k=cfg.K, E=cfg.E,
                       expert_offset=cfg.expert_offset, routed_scaling=cfg.routed_scaling,
                       situ_alpha=cfg.situ_alpha, situ_beta=cfg.situ_beta, max_tokens=cfg.T)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f}s workload={args.workload}",
          file=sys.stderr, flush=True)

    B = m._binding
    K, T, H, I, E_local = cfg.K, cfg.T, cfg.H, cfg.I, cfg.E_local
    R = T * K
    idx, tw = layer.topk_idx[:T], layer.topk_w[:T]
    if given:
        idx.copy_(torch.from_numpy(act["topk_idx"]))
        tw.copy_(torch.from_numpy(act["topk_w"]))
    xq, xs = layer.xq[:T], layer.xs[:T]
    sroute, rrow = layer.sorted_route[:R], layer.route_row[:R]
    hq, hs = layer.hq[:R], layer.hs[:R]

    def step(ev=None):
        if given:
            B.moe_quant_mxfp8(x, xq, xs)
            B.moe_permute(idx, cfg.expert_offset, E_local, layer.workspace, layer.expert_offsets,
                          sroute, rrow)
        else:
            B.moe_route_quant_permute(logits, bias, K, cfg.routed_scaling, x, cfg.expert_offset,
                                      E_local, layer.workspace, idx, tw, xq, xs,
                                      layer.expert_offsets, sroute, rrow)
        if ev is not None:
            ev[0].record()
        B.moe_fc1_situ(xq, xs, K, layer.expert_offsets, sroute, layer.w13, layer.w13_s,
                       layer.workspace, cfg.situ_alpha, cfg.situ_beta, hq, hs, tiled=layer.tiled)
        if ev is not None:
            ev[1].record()
        B.moe_fc2_combine(hq, hs, T, K, layer.expert_offsets, sroute, rrow, tw, layer.w2,
                          layer.w2_s, layer.workspace, out, tiled=layer.tiled,
                          mode=layer.combine_mode)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Each round times exactly K steps between two events, bracketed by
    # synchronisations; with several rounds the step time is their median.
    round_ms, fc1_times, wall = [], [], 0.0
    for _ in range(args.rounds):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(args.steps):
            step(evs[i])
        stop.record()
        torch.cuda.synchronize()
        wall += time.perf_counter() - t0
        round_ms.append(start.elapsed_time(stop) / args.steps)
        fc1_times += [a.elapsed_time(b) for a, b in evs]
    ms_per_step = float(np.median(round_ms))
    fc1_ms = float(np.mean(fc1_times))

    # The timed calls must compute what the layer computes.
    ref = layer(x, logits, bias, topk_idx=idx.clone() if given else None,
                topk_w=tw.clone() if given else None)
    if not torch.equal(ref.view(torch.int16), out.view(torch.int16)):
        print("[bench] timed path disagrees with MoELayer", file=sys.stderr, flush=True)
        sys.exit(1)

    # Algorithmic work of this batch.
    offs = layer.expert_offsets.cpu().numpy()
    n_kept = int(offs[-1])
    D = int(np.count_nonzero(np.diff(offs)))
    rr = rrow.cpu().numpy().reshape(T, K)
    tokens_used = int(np.count_nonzero((rr >= 0).any(1)))
    w13_bytes = 2 * I * H * (1 / 2 + 1 / 32)
    fc1_bytes = D * w13_bytes + tokens_used * H * (1 + 1 / 32) + n_kept * I * (1 + 1 / 32)
    fc1_flops = 2.0 * n_kept * 2 * I * H
    layer_bytes = (D * H * I * 1.59375 + 2 * T * H + (0 if given else 4 * T * cfg.E)
                   + 2 * 1.03125 * T * H
                   + 2 * 1.03125 * n_kept * I + 2 * T * H)
    layer_flops = n_kept * 6.0 * H * I
    traffic = _traffic(args.workload)
    # The binding roof is the one with the longer ideal time at MI355X's
    # published peaks (bytes / 8 TB/s against flops / 5 PFLOP/s).
    t_hbm = fc1_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = fc1_flops / (MFMA_FP8_PEAK_TFLOPS * 1e12)
    mfma_frac = fc1_flops / (fc1_ms * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS
    hbm_frac = fc1_bytes / (fc1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    if t_mfma > t_hbm:
        ach = fc1_flops / (fc1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_FP8_PEAK_TFLOPS, 4),
                "traffic": traffic}
    else:
        ach = fc1_bytes / (fc1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
    roof.update({"kernel": "fc1_situ", "kernel_ms": round(fc1_ms, 5),
                 "algorithmic_bytes": int(fc1_bytes), "algorithmic_flops": fc1_flops,
                 "hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4)})

    res = {
        "metric": "MoE-layer tokens/s",
        "value": round(T / (ms_per_step * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(T / (ms_per_step * 1e-3) / (T / (PAGES_EP_MIXED_MS[T] * 1e-3)), 4)
                        if given and T in PAGES_EP_MIXED_MS else None),
        "dtype": "e4m3xe2m1_f32acc",
        "data": "synthetic (seeded; x~N(0,1) bf16, weights N(0,0.02) -> MXFP4"
                + ("; top-k ids/weights given: 8 local + 8 remote slots per token)" if given
                   else "; router logits N(0,1), bias per workload)"),
        "config": {"workload": f"kimi_k3_moe_{args.workload}", "T": T, "H": H, "I": I,
                   "E": cfg.E, "top_k": K, "E_local": E_local,
                   "expert_offset": cfg.expert_offset, "routing": cfg.routing,
                   "experts_touched": D,
                   "routed_rows": n_kept},
        "layer": {"hbm_frac": round(layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(layer_flops / (ms_per_step * 1e-3) / 1e12
                                     / MFMA_FP8_PEAK_TFLOPS, 4),
                  "tflops": round(layer_flops / (ms_per_step * 1e-3) / 1e12, 2),
                  "gbs": round(layer_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                  "wall_s_timed": round(wall, 3)},
        "roofline": roof,
    }
    if args.rounds > 1:
        res["rounds"] = {"n": args.rounds, "ms_per_step": [round(v, 5) for v in round_ms],
                         "max_over_min": round(max(round_ms) / min(round_ms), 4)}
    if not args.no_cpu_baseline:
        rid = idx.cpu().numpy()
        rw = tw.cpu().numpy()
        tps, threads, dt, n_tok = cpu_baseline(cfg, act, w, rid, rw)
        res["cpu_baseline"] = {"value": round(tps, 4), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the first {n_tok} tokens of the same workload "
                                         f"({K} routes each), {dt:.1f}s, oracle route-by-route "
                                         f"float64"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
