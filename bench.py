#!/usr/bin/env python3
"""Benchmark of one MoE FFN layer step on one MI355X.

A step is the whole hot path on one batch already resident in HBM:
moe_route -> moe_permute -> moe_grouped_ffn (gate/up half, down half with the
combine) [-> moe_combine for large batches].  Default workload: the decode
layer (T=64 tokens, top-8 of 128 experts, H=4096, I=1536, bf16), which is
weight-load bound; ``--config prefill`` times the 6000-token prefill layer
(matrix-core bound).

Prints ONE JSON line.  ``roofline`` covers the dominant kernel (the gate/up
grouped GEMM): its algorithmic bytes (decode) or FLOPs (prefill) per launch
over its average duration, measured with HIP events on the stream the library
launches on.  ``cpu_baseline`` is the CPU oracle timed on this host on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + % bf16 MFMA peak (prefill) / % HBM BW (decode)"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix cores
WORKLOADS = {
    "decode": "decode MoE layer: T=64 tokens x top-8 of E=128 experts (512 assignments), H=4096, SwiGLU I=1536, bf16",
    "prefill": "prefill MoE layer: T=6000 tokens x top-8 of E=128 experts, H=4096, SwiGLU I=1536, bf16",
    "skew": "skewed prefill MoE layer: T=6000, top-8 of 128, logit bias 2*ln Zipf(1.2), H=4096, I=1536, bf16",
    "ep_share": "EP=4 share: T=8192 routed over 128 experts, local experts 0-31, fp8 e4m3 weights, H=4096, I=1536",
    "prefill_mx": "W8A8 MXFP8 prefill MoE layer: T=6000 tokens x top-8 of E=128 experts, H=4096, SwiGLU I=1536",
    "decode_mx": "W8A8 MXFP8 decode MoE layer: T=64 tokens x top-8 of E=128 experts, H=4096, SwiGLU I=1536",
    "decode_shared": "decode MoE layer (T=64, top-8 of 128, H=4096, I=1536, bf16) plus one shared expert (I_s=1536)",
    "prefill_shared": "prefill MoE layer (T=6000, top-8 of 128, H=4096, I=1536, bf16) plus one shared expert "
                      "(I_s=1536)",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU time budget of the oracle sample")
    ap.add_argument("--flush-steps", type=int, default=20,
                    help="extra steps, each after writing a 1 GiB scratch buffer (cold L2 and Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--router", default="packed", choices=["packed", "as-stored"],
                    help="decode-sized batches: read the router weight in the layout of moe_pack_router (exact "
                         "fp32, packed once before timing; routing is bit-identical)")
    ap.add_argument("--weights", default="packed", choices=["packed", "row-major"],
                    help="layout of the resident bf16/fp8 expert weights (packed once with moe_pack_weights "
                         "before timing; MXFP8 and fp32 weights are always row-major)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def measured_traffic(kernel, workload, weights):
    """HBM bytes per launch from a committed counter summary, or None when there is none, it was taken
    with the other weight layout, or the kernel's sources changed since the counters were taken (the
    summary records their SHA-256)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    try:
        h = hashlib.sha256()
        for src in fields["kernel_sources"].split():
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != fields["source_sha256"] or fields.get("weights", "row-major") != weights:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def copy_calibration():
    """A plain copy of known size: the profiler's FETCH_SIZE / WRITE_SIZE for it calibrate those counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def cpu_baseline(inp, cfg, seconds):
    """The oracle as it stands on a bounded sample of the same workload: whole-layer passes (route,
    permute, token-major SwiGLU FFN + combine) over consecutive 64-token chunks of the batch, wrapping
    around, until ``seconds`` of wall time have been spent (at least one chunk)."""
    from oracle import oracle as O
    chunk = min(64, cfg.T)
    done = 0
    stage = {"route": 0.0, "permute": 0.0, "ffn_combine": 0.0}
    t0 = time.perf_counter()
    while True:
        lo = done % cfg.T
        sl = slice(lo, min(lo + chunk, cfg.T))
        x = np.ascontiguousarray(inp["x"][sl])
        ta = time.perf_counter()
        ids, w, _ = O.route(x, inp["w_router"], inp["bias"], cfg.k)
        tb = time.perf_counter()
        O.permute(ids, w, cfg.lo, cfg.hi)
        tc = time.perf_counter()
        if cfg.wdt == "mxfp8":
            O.layer_tokens_mx(np.arange(x.shape[0]), x, ids, w, cfg.lo, cfg.hi, inp["w_gate_up"], inp["s_gate_up"],
                              inp["w_down"], inp["s_down"])
        else:
            O.layer_tokens(np.arange(x.shape[0]), x, ids, w, cfg.lo, cfg.hi, inp["w_gate_up"], inp["w_down"],
                           inp["s_gate_up"], inp["s_down"], round_h=cfg.act != "f32")
        if cfg.I_s > 0:
            O.shared_tokens(np.arange(x.shape[0]), x, inp["ws_gate_up"], inp["ws_down"], inp["ss_gate_up"],
                            inp["ss_down"], round_h=cfg.act != "f32")
        td = time.perf_counter()
        stage["route"] += tb - ta
        stage["permute"] += tc - tb
        stage["ffn_combine"] += td - tc
        done += x.shape[0]
        dt = td - t0
        if dt >= seconds:
            break
    return {"value": done / dt, "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{done} tokens in {chunk}-token chunks of the same {cfg.T}-token batch (wrapping around), "
                      f"whole layer per chunk (route, permute, token-major SwiGLU FFN + combine"
                      f"{' + shared expert' if cfg.I_s > 0 else ''}), {dt:.1f} s",
            "stage_tokens_per_s": {k: round(done / v, 1) if v > 0 else None for k, v in stage.items()}}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the layer has no multi-GPU path here.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from expert_routed_grouped_amd import accounting as A
    from expert_routed_grouped_amd import layer as L
    from expert_routed_grouped_amd import moe, synth

    cfg = synth.CONFIGS[args.config]
    print(f"[bench] generating {args.config} inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(cfg)
    dev = L.to_device(inp)
    if args.weights == "packed":
        L.pack_weights(dev)  # one-time layout change of the resident weights, like loading them
    packed = bool(dev.get("packed", False))
    bufs = L.LayerBuffers(cfg)
    if bufs.rd_ws is not None and args.router == "packed":
        L.pack_router(dev)  # one-time layout change of the resident router weight
    wrp = dev.get("w_router_packed") if bufs.rd_ws is not None else None
    stream = torch.cuda.current_stream()
    p = bufs.perm
    mx = cfg.wdt == "mxfp8"
    if mx:  # activations quantised on the fly into these, h lives in the MX workspace
        xq = torch.empty((cfg.T, cfg.H), dtype=torch.uint8, device="cuda")
        xs = torch.empty((cfg.T, cfg.H // 32), dtype=torch.uint8, device="cuda")
        bufs.workspace = torch.empty(moe.moe_ffn_mx_workspace_size(bufs.R_cap, cfg.I), dtype=torch.uint8,
                                     device="cuda")

    def ffn_half(phase, outs, common):
        if mx:
            moe.moe_grouped_ffn_mx(xq, xs, p["offsets"], p["row_token"], p["row_w"], cfg.T, bufs.R_cap,
                                   dev["w_gate_up"], dev["s_gate_up"], dev["w_down"], dev["s_down"], phase=phase,
                                   packed=packed, **outs, **common)
        else:
            moe.moe_grouped_ffn(dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, bufs.R_cap,
                                dev["w_gate_up"], dev["w_down"], dev["s_gate_up"], dev["s_down"], phase=phase,
                                packed=packed, **outs, **common)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if bufs.rd_ws is not None:  # decode: route + dispatch (+ zeroing of y) in one launch
            moe.moe_route_dispatch(dev["x"], dev["w_router"] if wrp is None else wrp, dev["bias"], cfg.k, cfg.E,
                                   cfg.lo, cfg.hi, bufs.rd_ws, bufs.topk_ids, bufs.topk_w, p,
                                   y_zero=bufs.y if bufs.fused else None, router_packed=wrp is not None,
                                   stream=stream)
        else:
            moe.moe_route(dev["x"], dev["w_router"], dev["bias"], cfg.k, bufs.topk_ids, bufs.topk_w, stream=stream)
            moe.moe_permute(bufs.topk_ids, bufs.topk_w, cfg.E, cfg.lo, cfg.hi, out=p, stream=stream)
        if mx:
            moe.moe_quantize_mx(dev["x"], xq, xs, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        common = dict(workspace=bufs.workspace, gather=True, stream=stream)
        outs = (dict(y=bufs.y, zero_y=bufs.rd_ws is None) if bufs.fused else dict(y_perm=bufs.y_perm, zero_y=False))
        ffn_half("gate_up", outs, common)
        if ev is not None:
            ev[2].record(stream)
        ffn_half("down", outs, common)
        if not bufs.fused:
            moe.moe_combine(bufs.y_perm, p["token_row"], bufs.topk_w, y=bufs.y, stream=stream)
        if bufs.shared_ws is not None:
            shared()
        if ev is not None:
            ev[3].record(stream)

    def shared():
        moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], bufs.y, dev.get("ss_gate_up"),
                              dev.get("ss_down"), workspace=bufs.shared_ws, packed=packed, stream=stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    layer_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    route_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    gu_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    down_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])

    shared_ms = None
    if bufs.shared_ws is not None:  # the shared expert alone, on the same stream
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in sev:
            a.record(stream)
            shared()
            b.record(stream)
        torch.cuda.synchronize()
        shared_ms = float(np.mean([a.elapsed_time(b) for a, b in sev]))

    flushed = None
    if args.flush_steps > 0:
        # each step after a 1 GiB write: the weights come from HBM, as when other layers ran in between
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        fl_ms = []
        for _ in range(args.flush_steps):
            scratch.fill_(0x5A)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            step(e)
            torch.cuda.synchronize()
            fl_ms.append(e[0].elapsed_time(e[3]))
        del scratch
        fl = np.array(fl_ms)
        flushed = {"steps": args.flush_steps, "ms_p50": round(float(np.median(fl)), 4),
                   "ms_p10": round(float(np.percentile(fl, 10)), 4), "ms_p90": round(float(np.percentile(fl, 90)), 4),
                   "tokens_per_s_p50": round(cfg.T / (float(np.median(fl)) * 1e-3), 1)}

    counts = p["counts"].cpu().numpy().astype(np.int64)
    R = int(counts.sum())
    U = int((counts > 0).sum())
    H, I, T = cfg.H, cfg.I, cfg.T
    # MXFP8 tensors carry one E8M0 scale byte per 32 codes
    wbytes = {"bf16": 2, "fp8": 1, "f32": 4, "mxfp8": 1 + 1 / 32}[cfg.wdt]
    abytes = 4 if cfg.act == "f32" else 2
    gu_abytes = 1 + 1 / 32 if mx else abytes   # x codes read, h codes written
    scale_gu = 4 * 2 * I if cfg.wdt == "fp8" else 0
    # gate/up half, algorithmic: each active expert's gate/up weights once, x read once, h written once
    gu_bytes = int(U * (2 * I * H * wbytes + scale_gu) + T * H * gu_abytes + R * I * gu_abytes)
    gu_flops = 4 * R * H * I
    layer_flops = A.useful_flops(R, H, I) + A.router_flops(T, H, cfg.E)
    layer_bytes = A.layer_hbm_bytes(counts, T, H, I, cfg.E, abytes,
                                    A.expert_bytes(H, I, wbytes, cfg.wdt == "fp8"), cfg.E * H * abytes)
    if cfg.I_s > 0:  # the shared expert: every token once, its weights once
        layer_flops += A.useful_flops(T, H, cfg.I_s)
        layer_bytes += A.expert_bytes(H, cfg.I_s, wbytes, cfg.wdt == "fp8")
    gu_s = float(np.mean(gu_ms)) * 1e-3
    hbm_bound = args.config.startswith("decode")  # a few rows per expert: the weight stream bounds the kernel
    if hbm_bound:
        achieved = gu_bytes / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        achieved = gu_flops / gu_s / 1e12
        peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None}
    streaming = bufs.R_cap <= 48 * cfg.E_loc
    kernel = (("ffn_mx_stream_kernel" if streaming else "ffn_mx_kernel") if mx else
              ("ffn_stream_kernel" if streaming else
               ("ffn_dma_kernel" if cfg.wdt == "bf16" else "ffn_big_kernel")))
    roof["traffic"] = measured_traffic(kernel, args.config, "packed" if packed else "row-major")
    # rows the grouped GEMM actually multiplies, by the tiling of the kernel in use
    padded = (A.padded_rows(counts, 64) if kernel == "ffn_stream_kernel" else
              A.padded_rows(counts, 32 if bufs.R_cap <= 16 * cfg.E_loc else 64) if kernel == "ffn_mx_stream_kernel" else
              (A.split_padded_rows(counts, 256, 64) if kernel == "ffn_dma_kernel" else
               (A.split_padded_rows(counts, 192, 64) if kernel == "ffn_mx_kernel" else A.padded_rows(counts, 256))))
    roof.update({"kernel": f"{kernel} (gate/up + SwiGLU half, one launch)", "avg_ms": round(float(np.mean(gu_ms)), 4),
                 "algorithmic_per_launch": gu_bytes if hbm_bound else gu_flops})
    layer_s = ms_per_step * 1e-3
    res = {
        "metric": METRIC,
        "value": round(T / layer_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-weights/bf16", "mxfp8": "mxfp8 (e4m3 + e8m0 block scales)"}.get(cfg.wdt,
                                                                                                            "f32"),
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "T": T, "H": H, "E": cfg.E, "k": cfg.k, "I": I,
                   "local_experts": [cfg.lo, cfg.hi], "parallelism": "none (one GPU)",
                   "combine": "fused atomic epilogue" if bufs.fused else "per-row outputs + moe_combine",
                   "dispatch": "route + dispatch in one launch" if bufs.rd_ws is not None else "moe_route + moe_permute",
                   "weights": "packed 32x64 blocks (moe_pack_weights, once before timing)" if packed else "row-major",
                   "router_weight": ("fp32 [H/4, E, 4] (moe_pack_router, once before timing)" if wrp is not None
                                     else "as stored")},
        "roofline": roof,
        "layer": {"ms_p50": round(float(np.median(layer_ms)), 4), "ms_p10": round(float(np.percentile(layer_ms, 10)), 4),
                  "ms_p90": round(float(np.percentile(layer_ms, 90)), 4),
                  "route_permute_ms": round(float(np.mean(route_ms)), 4), "gate_up_ms": round(float(np.mean(gu_ms)), 4),
                  "down_combine_ms": round(float(np.mean(down_ms)), 4),
                  "shared_expert_ms": None if shared_ms is None else round(shared_ms, 4),
                  "hbm_bytes": int(layer_bytes), "hbm_frac": round(layer_bytes / layer_s / 1e9 / PEAK_HBM_GBS, 4),
                  "flops": int(layer_flops),
                  "mfma_frac": round(layer_flops / layer_s / 1e12 / (PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS), 4)},
        "flushed_caches": flushed,
        "routing": {"assignments": R, "active_experts": U, "max_rows": int(counts.max()),
                    "padded_rows": padded, "padded_over_R": round(padded / R, 4) if R else None,
                    "skew": round(float(counts.max() / (R / max(len(counts), 1))), 3) if R else None},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
