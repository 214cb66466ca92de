"""One MoE FFN layer call = the four library calls in order, on one stream (a decode-sized
batch with a shared expert runs the shared expert on a second stream beside the router).

Host logic only: buffer allocation, choosing between the fused (atomic) combine
and the per-row outputs + ``moe_combine`` path, and moving synthetic numpy
inputs to the device.  All arithmetic runs in the library's kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import moe

# Above this many (row x hidden) outputs the fused epilogue's fp32 atomics cost more
# than writing per-row outputs and reducing them with moe_combine (measured on MI355X:
# ~0.33 T atomic adds/s against ~6-7 TB/s of streaming stores).
FUSED_COMBINE_MAX_ELEMS = 16 * 1024 * 1024


def to_device(inputs: dict, device="cuda") -> dict:
    """numpy synthetic inputs (bf16 as uint16 bits, fp8 as uint8 codes) -> device tensors."""
    def t(a, kind):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if kind == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).to(device)

    cfg = inputs["cfg"]
    out = {"cfg": cfg}
    out["x"] = t(inputs["x"], cfg.act)
    out["w_router"] = t(inputs["w_router"], cfg.act)
    out["bias"] = t(inputs.get("bias"), "f32")
    if "w_gate_up" in inputs:
        out["w_gate_up"] = t(inputs["w_gate_up"], cfg.wdt)
        out["w_down"] = t(inputs["w_down"], cfg.wdt)
        out["s_gate_up"] = t(inputs.get("s_gate_up"), "f32")
        out["s_down"] = t(inputs.get("s_down"), "f32")
    if "ws_gate_up" in inputs:  # shared expert
        out["ws_gate_up"] = t(inputs["ws_gate_up"], cfg.wdt)
        out["ws_down"] = t(inputs["ws_down"], cfg.wdt)
        out["ss_gate_up"] = t(inputs.get("ss_gate_up"), "f32")
        out["ss_down"] = t(inputs.get("ss_down"), "f32")
    return out


def pack_weights(dev: dict) -> dict:
    """Replace the bf16 / fp8 expert weights (MXFP8: their codes) of ``dev`` (routed and shared) by
    copies in the packed block layout (``moe_pack_weights``); later calls pass ``packed=True``.
    fp32 weights and MX scales stay row-major.  Done once, outside any timed region, like loading
    the weights."""
    if dev["cfg"].wdt not in ("bf16", "fp8", "mxfp8") or dev.get("packed"):
        return dev
    for key in ("w_gate_up", "w_down", "ws_gate_up", "ws_down"):
        if dev.get(key) is not None:
            dev[key] = moe.moe_pack_weights(dev[key])
    dev["packed"] = True
    return dev


def pack_router(dev: dict) -> dict:
    """Add the router weight in the layout of moe_pack_router (exact fp32, [H/4, E, 4]) as
    ``dev["w_router_packed"]``; decode-sized batches (moe_route_dispatch) then read it.  Done once,
    like loading the weights; routing is bit-identical."""
    w = dev["w_router"]
    if w.shape[1] % 4 == 0 and (dev.get("w_router_packed") is None or not _router_pack_current(dev)):
        dev["w_router_packed"] = moe.moe_pack_router(w)
        dev["w_router_packed_src"] = (w.data_ptr(), w._version)
    return dev


def _router_pack_current(dev: dict) -> bool:
    """True while ``w_router_packed`` was made from the present ``w_router`` tensor, unmodified since
    (same storage, same in-place version counter)."""
    w = dev["w_router"]
    return dev.get("w_router_packed_src") == (w.data_ptr(), w._version)


class LayerBuffers:
    """Device buffers of one layer shape, reused across calls."""

    def __init__(self, cfg, device="cuda", fused: Optional[bool] = None, use_route_dispatch: bool = True,
                 use_decode_layer: bool = False, shared_beside_router: bool = True):
        T, k, El, H, I = cfg.T, cfg.k, cfg.E_loc, cfg.H, cfg.I
        self.cfg = cfg
        self.R_cap = T * min(k, El)
        self.fused = (self.R_cap * H <= FUSED_COMBINE_MAX_ELEMS) if fused is None else fused
        d = dict(device=device)
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, **d)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, **d)
        self.perm = dict(counts=torch.empty(El, dtype=torch.int32, **d),
                         offsets=torch.empty(El + 1, dtype=torch.int32, **d),
                         row_token=torch.empty(max(self.R_cap, 1), dtype=torch.int32, **d),
                         row_w=torch.empty(max(self.R_cap, 1), dtype=torch.float32, **d),
                         token_row=torch.empty((T, k), dtype=torch.int32, **d),
                         workspace=torch.empty(max(moe.moe_permute_workspace_size(T, k, El), 256), dtype=torch.uint8,
                                               **d))
        adt = moe.MOE_F32 if cfg.act == "f32" else moe.MOE_BF16
        self.workspace = torch.empty(moe.moe_ffn_workspace_size(self.R_cap, El, H, I, adt), dtype=torch.uint8, **d)
        self.y = torch.empty((T, H), dtype=torch.float32, **d)
        self.y_perm = None if self.fused else torch.empty((max(self.R_cap, 1), H), dtype=torch.float32, **d)
        self.shared_ws = (torch.empty(moe.moe_shared_workspace_size(T, cfg.I_s, adt), dtype=torch.uint8, **d)
                          if cfg.I_s > 0 else None)
        # use_decode_layer: decode batches (T <= 64) run the whole layer in one launch
        # (moe_decode_layer; its workspace starts zeroed).  Off by default: on MI355X the one-launch
        # kernel measured 1.03 ms for the 64-token layer against 0.86 ms for route + dispatch, gate/up
        # and down as three launches
        dec = (use_decode_layer and self.fused and 1 <= T <= 64 and cfg.act == "bf16" and cfg.wdt in ("bf16", "fp8")
               and cfg.E <= 256 and H % 64 == 0 and I % 64 == 0 and H <= 16384)
        self.dec_ws = moe.moe_decode_layer_workspace(T, k, El, I, device) if dec else None
        # otherwise decode-sized batches route and dispatch in one launch (its ticket workspace starts zeroed)
        fits = 1 <= T <= 512 and T * k <= 8192 and cfg.E <= 256 and H % 8 == 0 and H <= 16384
        self.rd_ws = (moe.moe_route_dispatch_workspace(device) if (fits and use_route_dispatch and not dec)
                      else None)
        # a decode-sized batch with a shared expert: the shared expert (which zeroes y, then adds to it)
        # runs on a second stream while the latency-bound router leaves HBM idle; the routed down
        # projection waits for it before its own fp32 adds into y
        self.side = None
        if shared_beside_router and self.rd_ws is not None and self.fused and self.shared_ws is not None:
            self.side = (torch.cuda.Stream(device=device), torch.cuda.Event())


def run_layer(dev: dict, bufs: LayerBuffers, stream=None) -> torch.Tensor:
    """route -> permute -> grouped FFN (-> combine) (-> shared expert), or for decode-sized batches
    moe_decode_layer (-> shared expert).  Returns y [T,H] fp32."""
    cfg = bufs.cfg
    p = bufs.perm
    packed = bool(dev.get("packed", False))
    wp = dev.get("w_router_packed")
    if wp is not None and not _router_pack_current(dev):  # w_router replaced or edited: pack again
        wp = pack_router(dev)["w_router_packed"]
    if bufs.dec_ws is not None:  # the whole layer in one launch
        moe.moe_decode_layer(dev["x"], dev["w_router"] if wp is None else wp, dev["bias"], cfg.k, cfg.E, cfg.lo, cfg.hi,
                             dev["w_gate_up"], dev["w_down"], dev.get("s_gate_up"), dev.get("s_down"), bufs.dec_ws,
                             bufs.topk_ids, bufs.topk_w, p, bufs.y, router_packed=wp is not None, packed=packed,
                             stream=stream)
        if bufs.shared_ws is not None:
            moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], bufs.y, dev.get("ss_gate_up"),
                                  dev.get("ss_down"), workspace=bufs.shared_ws, packed=packed, stream=stream)
        return bufs.y
    if bufs.side is not None:  # shared expert beside the router, routed halves after it
        main = stream if stream is not None else torch.cuda.current_stream()
        side_stream, side_done = bufs.side
        side_stream.wait_stream(main)
        moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], bufs.y, dev.get("ss_gate_up"),
                              dev.get("ss_down"), workspace=bufs.shared_ws, zero_y=True, packed=packed,
                              stream=side_stream)
        side_done.record(side_stream)
        moe.moe_route_dispatch(dev["x"], dev["w_router"] if wp is None else wp, dev["bias"], cfg.k, cfg.E, cfg.lo,
                               cfg.hi, bufs.rd_ws, bufs.topk_ids, bufs.topk_w, p, y_zero=None,
                               router_packed=wp is not None, stream=main)
        ffn = dict(workspace=bufs.workspace, gather=True, packed=packed, stream=main)
        moe.moe_grouped_ffn(dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, bufs.R_cap,
                            dev["w_gate_up"], dev["w_down"], dev.get("s_gate_up"), dev.get("s_down"),
                            y=bufs.y, zero_y=False, phase="gate_up", **ffn)
        main.wait_event(side_done)
        moe.moe_grouped_ffn(dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, bufs.R_cap,
                            dev["w_gate_up"], dev["w_down"], dev.get("s_gate_up"), dev.get("s_down"),
                            y=bufs.y, zero_y=False, phase="down", **ffn)
        return bufs.y
    if bufs.rd_ws is not None:  # one launch: route, dispatch and (fused combine) the zeroing of y
        moe.moe_route_dispatch(dev["x"], dev["w_router"] if wp is None else wp, dev["bias"], cfg.k, cfg.E, cfg.lo,
                               cfg.hi, bufs.rd_ws, bufs.topk_ids, bufs.topk_w, p,
                               y_zero=bufs.y if bufs.fused else None, router_packed=wp is not None, stream=stream)
    else:
        moe.moe_route(dev["x"], dev["w_router"], dev["bias"], cfg.k, bufs.topk_ids, bufs.topk_w, stream=stream)
        moe.moe_permute(bufs.topk_ids, bufs.topk_w, cfg.E, cfg.lo, cfg.hi, out=p, stream=stream)
    if bufs.fused:
        moe.moe_grouped_ffn(dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, bufs.R_cap,
                            dev["w_gate_up"], dev["w_down"], dev.get("s_gate_up"), dev.get("s_down"),
                            y=bufs.y, workspace=bufs.workspace, gather=True, zero_y=bufs.rd_ws is None,
                            packed=packed, stream=stream)
    else:
        moe.moe_grouped_ffn(dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, bufs.R_cap,
                            dev["w_gate_up"], dev["w_down"], dev.get("s_gate_up"), dev.get("s_down"),
                            y_perm=bufs.y_perm, workspace=bufs.workspace, gather=True, packed=packed, stream=stream)
        moe.moe_combine(bufs.y_perm, p["token_row"], bufs.topk_w, y=bufs.y, stream=stream)
    if bufs.shared_ws is not None:
        moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], bufs.y, dev.get("ss_gate_up"),
                              dev.get("ss_down"), workspace=bufs.shared_ws, packed=packed, stream=stream)
    return bufs.y
