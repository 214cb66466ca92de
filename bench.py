#!/usr/bin/env python3
"""Benchmark of one MoE FFN layer step on one MI355X.

A step is the whole hot path on one batch already resident in HBM: routing
(router GEMM, top-k, renormalised gates), the grouping of assignments by
expert, the SwiGLU grouped GEMMs (gate/up, then down with the combine) and,
for large batches, the standalone combine.

The default run measures both halves of the headline metric in one process:

* ``decode`` (the headline ``value``): T=64 tokens x top-8 of 128 experts,
  H=4096, I=1536, bf16 -- weight-load bound, reported against HBM bandwidth.
  Each of the K timed steps follows a 1 GiB write and a 1 GiB read of other
  buffers, which evict the L2s and the Infinity Cache (the weights of a real
  model come from HBM, other layers ran in between); the warm back-to-back rate
  and the rate after the write alone are reported beside it.
* ``prefill`` (the ``prefill`` object): T=6000 tokens, same layer -- matrix-core
  bound, reported against the bf16 MFMA peak, for the gate/up kernel and for
  the whole layer.

``--config NAME`` measures one workload alone (the other workloads are parity
and reporting cases: skew, ep_share, prefill_mx, decode_mx, decode_shared,
prefill_shared).

Prints ONE JSON line.  ``roofline`` covers the dominant kernel of the headline
workload: its algorithmic bytes (decode) or FLOPs (prefill) per launch over its
average duration, measured with HIP events on the stream the library launches
on.  ``cpu_baseline`` is the CPU oracle timed on this host on a bounded sample
of the headline workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + % bf16 MFMA peak (prefill) / % HBM BW (decode)"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix cores
FLUSH_BYTES = 1 << 30       # written before each flushed step: more than the L2s and the Infinity Cache hold
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
    ap.add_argument("--config", default="default", choices=["default"] + sorted(WORKLOADS),
                    help="default: decode (headline) and prefill in one run; otherwise one workload")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU time budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="time warm back-to-back steps only (no cache-flushing write before each step)")
    ap.add_argument("--router", default="packed", choices=["packed", "as-stored"],
                    help="decode-sized batches: read the router weight in the layout of moe_pack_router (exact "
                         "fp32, packed once before timing; routing is bit-identical)")
    ap.add_argument("--weights", default="packed", choices=["packed", "row-major"],
                    help="layout of the resident bf16/fp8 expert weights (packed once with moe_pack_weights "
                         "before timing)")
    ap.add_argument("--shared-after", action="store_true",
                    help="decode with a shared expert: run it after the routed FFN on the same stream instead of "
                         "on a second stream beside the router")
    ap.add_argument("--one-launch", action="store_true",
                    help="decode batches: the whole layer as one launch (moe_decode_layer) instead of route + "
                         "dispatch, gate/up, down (three launches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


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
    return {"value": round(done / dt, 2), "unit": "tokens/s", "cores": O.num_threads(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{done} tokens of the {cfg.name} workload in {chunk}-token chunks of its {cfg.T}-token batch "
                      f"(wrapping around), whole layer per chunk (route, permute, token-major SwiGLU FFN + combine"
                      f"{' + shared expert' if cfg.I_s > 0 else ''}), {dt:.1f} s",
            "stage_tokens_per_s": {k: round(done / v, 1) if v > 0 else None for k, v in stage.items()}}


def stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": round(float(a.mean()), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p50": round(float(np.median(a)), 4), "p90": round(float(np.percentile(a, 90)), 4)}


class Workload:
    """One workload's resident inputs, buffers and the step as a list of phases (each a few library
    calls on one stream), so that HIP events between phases time each kernel group."""

    def __init__(self, name, args):
        import torch
        from expert_routed_grouped_amd import layer as L
        from expert_routed_grouped_amd import moe, synth
        self.name = name
        cfg = self.cfg = synth.CONFIGS[name]
        say(f"generating {name} inputs")
        self.inp = synth.make_inputs(cfg)
        dev = self.dev = L.to_device(self.inp)
        if args.weights == "packed":
            L.pack_weights(dev)  # one-time layout change of the resident weights, like loading them
        self.packed = bool(dev.get("packed", False))
        bufs = self.bufs = L.LayerBuffers(cfg, use_decode_layer=args.one_launch,
                                          shared_beside_router=not args.shared_after)
        self.one_launch = bufs.dec_ws is not None
        decode_router = bufs.rd_ws is not None or self.one_launch
        if decode_router and args.router == "packed":
            L.pack_router(dev)  # one-time layout change of the resident router weight
        self.wrp = dev.get("w_router_packed") if decode_router else None
        self.stream = torch.cuda.current_stream()
        self.mx = cfg.wdt == "mxfp8"
        if self.mx:  # activations quantised on the fly into these, h lives in the MX workspace
            self.xq = torch.empty((cfg.T, cfg.H), dtype=torch.uint8, device="cuda")
            self.xs = torch.empty((cfg.T, cfg.H // 32), dtype=torch.uint8, device="cuda")
            bufs.workspace = torch.empty(moe.moe_ffn_mx_workspace_size(bufs.R_cap, cfg.I), dtype=torch.uint8,
                                         device="cuda")
        self.moe = moe
        if self.one_launch:  # the whole layer in one kernel (then the shared expert, if any)
            self.phases = [("layer_kernel", self.decode_layer)]
            if bufs.shared_ws is not None:
                self.phases.append(("shared_expert", self.shared))
        else:
            self.phases = [("route", self.route), ("gate_up", lambda: self.ffn_half("gate_up")),
                           ("down", self.down)]

    def decode_layer(self):
        moe, cfg, bufs, dev = self.moe, self.cfg, self.bufs, self.dev
        moe.moe_decode_layer(dev["x"], dev["w_router"] if self.wrp is None else self.wrp, dev["bias"], cfg.k, cfg.E,
                             cfg.lo, cfg.hi, dev["w_gate_up"], dev["w_down"], dev["s_gate_up"], dev["s_down"],
                             bufs.dec_ws, bufs.topk_ids, bufs.topk_w, bufs.perm, bufs.y,
                             router_packed=self.wrp is not None, packed=self.packed, stream=self.stream)

    def route(self):
        moe, cfg, bufs, dev, p, s = self.moe, self.cfg, self.bufs, self.dev, self.bufs.perm, self.stream
        if bufs.side is not None:  # decode with a shared expert: it zeroes y and runs beside the router
            side_stream, side_done = bufs.side
            side_stream.wait_stream(s)
            self.moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], bufs.y, dev.get("ss_gate_up"),
                                       dev.get("ss_down"), workspace=bufs.shared_ws, zero_y=True,
                                       packed=self.packed, stream=side_stream)
            side_done.record(side_stream)
        if bufs.rd_ws is not None:  # decode: route + dispatch (+ zeroing of y) in one launch
            moe.moe_route_dispatch(dev["x"], dev["w_router"] if self.wrp is None else self.wrp, dev["bias"], cfg.k,
                                   cfg.E, cfg.lo, cfg.hi, bufs.rd_ws, bufs.topk_ids, bufs.topk_w, p,
                                   y_zero=bufs.y if (bufs.fused and bufs.side is None) else None,
                                   router_packed=self.wrp is not None, stream=s)
        else:
            moe.moe_route(dev["x"], dev["w_router"], dev["bias"], cfg.k, bufs.topk_ids, bufs.topk_w, stream=s)
            moe.moe_permute(bufs.topk_ids, bufs.topk_w, cfg.E, cfg.lo, cfg.hi, out=p, stream=s)
        if self.mx:
            moe.moe_quantize_mx(dev["x"], self.xq, self.xs, stream=s)

    def ffn_half(self, phase):
        moe, cfg, bufs, dev, p = self.moe, self.cfg, self.bufs, self.dev, self.bufs.perm
        common = dict(workspace=bufs.workspace, gather=True, stream=self.stream, phase=phase, packed=self.packed)
        outs = (dict(y=bufs.y, zero_y=bufs.rd_ws is None) if bufs.fused else dict(y_perm=bufs.y_perm, zero_y=False))
        if self.mx:
            moe.moe_grouped_ffn_mx(self.xq, self.xs, p["offsets"], p["row_token"], p["row_w"], cfg.T, bufs.R_cap,
                                   dev["w_gate_up"], dev["s_gate_up"], dev["w_down"], dev["s_down"], **outs, **common)
        else:
            moe.moe_grouped_ffn(dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, bufs.R_cap,
                                dev["w_gate_up"], dev["w_down"], dev["s_gate_up"], dev["s_down"], **outs, **common)

    def down(self):
        if self.bufs.side is not None:  # the shared expert on the side stream zeroed y and added to it
            self.stream.wait_event(self.bufs.side[1])
        self.ffn_half("down")
        if not self.bufs.fused:
            self.moe.moe_combine(self.bufs.y_perm, self.bufs.perm["token_row"], self.bufs.topk_w, y=self.bufs.y,
                                 stream=self.stream)
        if self.bufs.shared_ws is not None and self.bufs.side is None:
            self.shared()

    def shared(self):
        dev = self.dev
        self.moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], self.bufs.y, dev.get("ss_gate_up"),
                                   dev.get("ss_down"), workspace=self.bufs.shared_ws, packed=self.packed,
                                   stream=self.stream)

    def step(self, ev=None):
        if ev is not None:
            ev[0].record(self.stream)
        for i, (_, fn) in enumerate(self.phases):
            fn()
            if ev is not None:
                ev[i + 1].record(self.stream)


def measure(wl: Workload, args):
    """W warm-up steps; K timed steps each after a cache-flushing write (HIP events around the step);
    K warm back-to-back steps (HIP events, and the wall clock between two synchronisations)."""
    import torch
    from expert_routed_grouped_amd import accounting as A
    cfg, bufs = wl.cfg, wl.bufs
    T, H, I = cfg.T, cfg.H, cfg.I
    nph = len(wl.phases)
    say(f"{wl.name}: warmup {args.warmup}")
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)]

    def phase_ms(evs):
        return {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
                for i, (name, _) in enumerate(wl.phases)}

    flushed = flushed_w = None
    if not args.no_flush:
        # Before each flushed step 1 GiB is written and another 1 GiB read: the L2s and the Infinity
        # Cache then hold none of the layer's data, and no dirty lines either.  After the write alone
        # they hold ~290 MB of dirty lines whose write-back the next kernel pays for (measured on the
        # decode layer: +59 us in its first kernel, nothing elsewhere); that cost belongs to the flush,
        # not to the layer, so it is reported beside the headline rather than in it.
        scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        other = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        total = torch.zeros((), dtype=torch.float32, device="cuda")

        def flushed_steps(n, read):
            evs = [events() for _ in range(n)]
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            for i in range(n):
                scratch.fill_(0x5A)
                if read:
                    torch.sum(other, dim=0, out=total)
                wl.step(evs[i])
                torch.cuda.synchronize()
            w1 = time.perf_counter()
            return {"ms": stats([e[0].elapsed_time(e[nph]) for e in evs]),
                    "phase_ms": {k: round(v, 4) for k, v in phase_ms(evs).items()},
                    "wall_ms_per_step_incl_flush_and_sync": round((w1 - w0) * 1e3 / n, 4)}

        say(f"{wl.name}: timing {args.steps} steps, each after a {FLUSH_BYTES >> 20} MiB write and a "
            f"{FLUSH_BYTES >> 20} MiB read of other buffers")
        flushed = dict(flushed_steps(args.steps, True), flush="1 GiB written, then another 1 GiB read")
        nw = min(args.steps, 20)
        say(f"{wl.name}: timing {nw} steps, each after the 1 GiB write alone")
        flushed_w = dict(flushed_steps(nw, False), flush="1 GiB written (dirty lines left to write back)")
        del scratch, other, total

    say(f"{wl.name}: timing {args.steps} warm back-to-back steps")
    wevs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        wl.step(wevs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    warm_wall = (t1 - t0) * 1e3 / args.steps
    warm = {"ms_per_step_wall": round(warm_wall, 4), "ms": stats([e[0].elapsed_time(e[nph]) for e in wevs]),
            "phase_ms": {k: round(v, 4) for k, v in phase_ms(wevs).items()}}

    shared_ms = None
    if bufs.shared_ws is not None:  # the shared expert alone, on the same stream
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in sev:
            a.record(wl.stream)
            wl.shared()
            b.record(wl.stream)
        torch.cuda.synchronize()
        shared_ms = round(float(np.mean([a.elapsed_time(b) for a, b in sev])), 4)

    counts = bufs.perm["counts"].cpu().numpy().astype(np.int64)
    R = int(counts.sum())
    U = int((counts > 0).sum())
    mx = wl.mx
    # MXFP8 tensors carry one E8M0 scale byte per 32 codes
    wbytes = {"bf16": 2, "fp8": 1, "f32": 4, "mxfp8": 1 + 1 / 32}[cfg.wdt]
    abytes = 4 if cfg.act == "f32" else 2
    gu_abytes = 1 + 1 / 32 if mx else abytes   # x codes read, h codes written
    scale_gu = 4 * 2 * I if cfg.wdt == "fp8" else 0
    # gate/up half, algorithmic: each active expert's gate/up weights once, x read once, h written once
    gu_bytes = int(U * (2 * I * H * wbytes + scale_gu) + T * H * gu_abytes + R * I * gu_abytes)
    gu_flops = 4 * R * H * I
    layer_flops = A.useful_flops(R, H, I) + A.router_flops(T, H, cfg.E)
    # the router weight as the timed step reads it: the moe_pack_router copy is exact fp32
    router_bytes = cfg.E * H * (4 if wl.wrp is not None else abytes)
    layer_bytes = A.layer_hbm_bytes(counts, T, H, I, cfg.E, abytes, A.expert_bytes(H, I, wbytes, cfg.wdt == "fp8"),
                                    router_bytes)
    if cfg.I_s > 0:  # the shared expert: every token once, its weights once
        layer_flops += A.useful_flops(T, H, cfg.I_s)
        layer_bytes += A.expert_bytes(H, cfg.I_s, wbytes, cfg.wdt == "fp8")
    # headline timing: the flushed steps (weights from HBM), else the warm ones
    fw_s = flushed_w["ms"]["mean"] * 1e-3 if flushed_w else None
    step_ms = flushed["ms"]["mean"] if flushed else warm["ms"]["mean"]
    hbm_bound = wl.name.startswith("decode")  # a few rows per expert: the weight stream bounds the kernel
    peak_mfma = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    timing = "cache-flushed steps" if flushed else "warm steps"
    weights = "packed" if wl.packed else "row-major"
    if wl.one_launch:
        # the dominant kernel is the whole routed layer: its algorithmic bytes are the layer's minus
        # the shared expert's (a separate launch)
        k_ms = (flushed or warm)["phase_ms"]["layer_kernel"]
        k_bytes = int(layer_bytes - (A.expert_bytes(H, cfg.I_s, wbytes, cfg.wdt == "fp8") if cfg.I_s > 0 else 0))
        achieved = k_bytes / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic("decode_layer_kernel", wl.name, weights),
                "kernel": "decode_layer_kernel (routing, grouping, gate/up, down + combine: one launch)",
                "avg_ms": round(k_ms, 4), "algorithmic_per_launch": k_bytes, "timing": timing}
        padded = A.padded_rows(counts, 64)
    else:
        gu_ms = (flushed or warm)["phase_ms"]["gate_up"]
        gu_s = gu_ms * 1e-3
        if hbm_bound:
            achieved = gu_bytes / gu_s / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4)}
        else:
            achieved = gu_flops / gu_s / 1e12
            roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_mfma, "unit": "TFLOP/s",
                    "frac": round(achieved / peak_mfma, 4)}
        streaming = bufs.R_cap <= 48 * cfg.E_loc
        kernel = (("ffn_mx_stream_kernel" if streaming else "ffn_mx_kernel") if mx else
                  ("ffn_stream_kernel" if streaming else
                   "ffn_dma_kernel"))
        roof["traffic"] = measured_traffic(kernel, wl.name, weights)
        # rows the grouped GEMM actually multiplies, by the tiling of the kernel in use
        padded = (A.padded_rows(counts, 64) if kernel == "ffn_stream_kernel" else
                  A.padded_rows(counts, 32 if bufs.R_cap <= 16 * cfg.E_loc else 64)
                  if kernel == "ffn_mx_stream_kernel" else
                  (A.split_padded_rows(counts, 256, 64) if kernel == "ffn_dma_kernel" else
                   (A.split_padded_rows(counts, 192, 64) if kernel == "ffn_mx_kernel" else A.padded_rows(counts, 256))))
        roof.update({"kernel": f"{kernel}<0> (gate/up + SwiGLU half, one launch)", "avg_ms": round(gu_ms, 4),
                     "algorithmic_per_launch": gu_bytes if hbm_bound else gu_flops, "timing": timing})
    layer_s = step_ms * 1e-3
    warm_s = warm["ms"]["mean"] * 1e-3
    return {
        "workload": WORKLOADS[wl.name], "name": wl.name, "T": T, "H": H, "E": cfg.E, "k": cfg.k, "I": I,
        "local_experts": [cfg.lo, cfg.hi],
        "tokens_per_s": round(T / layer_s, 1), "ms_per_step": round(step_ms, 4),
        "timing": ("mean of K steps, each after writing 1 GiB and reading another 1 GiB (caches hold none of the "
                   "layer's data), HIP events around the step" if flushed else
                   "mean of K warm back-to-back steps, HIP events"),
        "flushed": flushed, "flushed_write_only": flushed_w, "warm": dict(warm, tokens_per_s=round(T / warm_s, 1)),
        "roofline": roof,
        "layer": {"hbm_bytes": int(layer_bytes), "hbm_frac": round(layer_bytes / layer_s / 1e9 / PEAK_HBM_GBS, 4),
                  "hbm_frac_warm": round(layer_bytes / warm_s / 1e9 / PEAK_HBM_GBS, 4),
                  "hbm_frac_flushed_write_only": (round(layer_bytes / fw_s / 1e9 / PEAK_HBM_GBS, 4) if fw_s
                                                  else None),
                  "router_weight_bytes": int(router_bytes), "flops": int(layer_flops),
                  "mfma_frac": round(layer_flops / layer_s / 1e12 / peak_mfma, 4),
                  "mfma_frac_warm": round(layer_flops / warm_s / 1e12 / peak_mfma, 4),
                  "shared_expert_ms": shared_ms},
        "config": {"combine": "fused atomic epilogue" if bufs.fused else "per-row outputs + moe_combine",
                   "dispatch": ("the whole layer in one launch (moe_decode_layer)" if wl.one_launch else
                                "route + dispatch in one launch" if bufs.rd_ws is not None else
                                "moe_route + moe_permute"),
                   "weights": "packed 32x64 blocks (moe_pack_weights, once before timing)" if wl.packed else "row-major",
                   "router_weight": ("fp32 [H/4, E, 4] (moe_pack_router, once before timing)" if wl.wrp is not None
                                     else "as stored")},
        "routing": {"assignments": R, "active_experts": U, "max_rows": int(counts.max()),
                    "padded_rows": padded, "padded_over_R": round(padded / R, 4) if R else None,
                    "skew": round(float(counts.max() / (R / max(len(counts), 1))), 3) if R else None},
        "dtype": {"bf16": "bf16", "fp8": "fp8-weights/bf16", "mxfp8": "mxfp8 (e4m3 + e8m0 block scales)"}.get(
            cfg.wdt, "f32"),
    }


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

    head_name = "decode" if args.config == "default" else args.config
    head = Workload(head_name, args)
    h = measure(head, args)
    cpu = None
    if not args.no_cpu_baseline:
        say("cpu baseline (oracle)")
        cpu = cpu_baseline(head.inp, head.cfg, args.cpu_seconds)
    pre = one = None
    if args.config == "default":
        del head
        torch.cuda.empty_cache()
        # the same decode layer as one launch (moe_decode_layer), reported beside the headline
        one_args = argparse.Namespace(**dict(vars(args), one_launch=True))
        one_wl = Workload("decode", one_args)
        o = measure(one_wl, one_args)
        del one_wl
        torch.cuda.empty_cache()
        one = {k: o[k] for k in ("tokens_per_s", "ms_per_step", "timing", "roofline", "warm", "flushed",
                                 "flushed_write_only", "config")}
        one["layer_hbm_frac"] = o["layer"]["hbm_frac"]
        pre_wl = Workload("prefill", args)
        p = measure(pre_wl, args)
        del pre_wl
        pre = {k: p[k] for k in ("workload", "tokens_per_s", "ms_per_step", "timing", "roofline", "layer", "warm",
                                 "flushed", "flushed_write_only", "routing", "config")}
        pre["roofline_layer"] = {"bound": "mfma", "achieved": round(p["layer"]["flops"] / p["ms_per_step"] / 1e9, 1),
                                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": p["layer"]["mfma_frac"],
                                 "flops_per_step": p["layer"]["flops"]}
    res = {
        "metric": METRIC,
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic",
        "config": dict({"workload": h["workload"], "T": h["T"], "H": h["H"], "E": h["E"], "k": h["k"], "I": h["I"],
                        "local_experts": h["local_experts"], "parallelism": "none (one GPU)"}, **h["config"]),
        "timing": h["timing"],
        "layer_fractions": {f"{h['name']}_layer_hbm_frac": h["layer"]["hbm_frac"],
                            f"{h['name']}_layer_mfma_frac": h["layer"]["mfma_frac"]},
        "roofline": h["roofline"],
        "layer": h["layer"],
        "warm": h["warm"],
        "flushed": h["flushed"],
        "flushed_write_only": h["flushed_write_only"],
        "routing": h["routing"],
    }
    if pre is not None:
        res["layer_fractions"] = {"decode_layer_hbm_frac": h["layer"]["hbm_frac"],
                                  "decode_layer_hbm_frac_warm": h["layer"]["hbm_frac_warm"],
                                  "decode_layer_hbm_frac_flushed_write_only": h["layer"]["hbm_frac_flushed_write_only"],
                                  "prefill_layer_mfma_frac": pre["layer"]["mfma_frac"],
                                  "prefill_gate_up_kernel_mfma_frac": pre["roofline"]["frac"]}
        res["prefill"] = pre
        res["decode_one_launch"] = one
    res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
