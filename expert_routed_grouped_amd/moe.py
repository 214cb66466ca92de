"""Thin ctypes binding of ``libmoe.so`` (declared in ``include/moe.h``).

Argument marshalling only: torch tensors in, raw device pointers and sizes to
the C ABI, every step runs in the library's HIP kernels on the tensor's
current stream.  There is no fallback: without the built library every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP8, MOE_F32_ROUTER_PACKED = 0, 1, 2, 3, 4
MOE_FFN_GATHER, MOE_FFN_ZERO_Y, MOE_FFN_ONLY_GATE_UP, MOE_FFN_ONLY_DOWN = 1, 2, 4, 8
MOE_FFN_PACKED_WEIGHTS = 16
STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_DTYPE", -4: "MOE_ERR_WORKSPACE",
          -5: "MOE_ERR_HIP", -6: "MOE_ERR_ALIGN"}

# Every symbol moe.h declares (checked by the CPU test suite).
EXPORTS = ("moe_version", "moe_status_str", "moe_route", "moe_permute", "moe_permute_workspace_size",
           "moe_ffn_workspace_size", "moe_grouped_ffn", "moe_combine", "moe_quantize_mx", "moe_ffn_mx_workspace_size",
           "moe_grouped_ffn_mx", "moe_shared_workspace_size", "moe_shared_expert", "moe_route_dispatch_workspace_size",
           "moe_route_dispatch", "moe_pack_weights", "moe_pack_router", "moe_grouped_ffn_noalloc",
           "moe_decode_layer_workspace_size", "moe_decode_layer", "moe_workspace_size")
MOE_OP_PERMUTE, MOE_OP_GROUPED_FFN, MOE_OP_GROUPED_FFN_F32, MOE_OP_GROUPED_FFN_MX = 0, 1, 2, 3
MOE_OP_ROUTE_DISPATCH, MOE_OP_DECODE_LAYER, MOE_OP_SHARED_EXPERT, MOE_OP_SHARED_EXPERT_F32 = 4, 5, 6, 7
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m expert_routed_grouped_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_version.restype = I
        L.moe_version.argtypes = []
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [I]
        L.moe_route.restype = I
        L.moe_route.argtypes = [P, I, P, I, P, I, I, I, I, P, P, P]
        L.moe_permute.restype = I
        L.moe_permute.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P, P, I, I, P, P, Z, P]
        L.moe_permute_workspace_size.restype = Z
        L.moe_permute_workspace_size.argtypes = [I, I, I]
        L.moe_ffn_workspace_size.restype = Z
        L.moe_ffn_workspace_size.argtypes = [I, I, I, I, I]
        L.moe_grouped_ffn.restype = I
        L.moe_grouped_ffn.argtypes = [P, I, P, P, P, I, I, I, I, I, P, P, I, P, P, P, P, P, Z, ctypes.c_uint, P]
        L.moe_grouped_ffn_noalloc.restype = I
        L.moe_grouped_ffn_noalloc.argtypes = [P, I, P, P, P, I, I, I, I, I, P, P, I, P, P, P, P, ctypes.c_uint, P]
        L.moe_workspace_size.restype = Z
        L.moe_workspace_size.argtypes = [I, I, I, I, I, I]
        L.moe_decode_layer_workspace_size.restype = Z
        L.moe_decode_layer_workspace_size.argtypes = [I, I, I, I]
        L.moe_decode_layer.restype = I
        L.moe_decode_layer.argtypes = [P, I, P, I, P, I, I, I, I, I, I, I, P, P, I, P, P, P, P, P, P, P, P, P, P, P,
                                       Z, ctypes.c_uint, P]
        L.moe_combine.restype = I
        L.moe_combine.argtypes = [P, P, P, I, I, I, P, P]
        L.moe_quantize_mx.restype = I
        L.moe_quantize_mx.argtypes = [P, I, I, I, P, P, P]
        L.moe_ffn_mx_workspace_size.restype = Z
        L.moe_ffn_mx_workspace_size.argtypes = [I, I]
        L.moe_grouped_ffn_mx.restype = I
        L.moe_grouped_ffn_mx.argtypes = [P, P, P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, Z, ctypes.c_uint, P]
        L.moe_shared_workspace_size.restype = Z
        L.moe_shared_workspace_size.argtypes = [I, I, I]
        L.moe_shared_expert.restype = I
        L.moe_shared_expert.argtypes = [P, I, I, I, I, P, P, I, P, P, P, P, Z, ctypes.c_uint, P]
        L.moe_route_dispatch_workspace_size.restype = Z
        L.moe_route_dispatch_workspace_size.argtypes = []
        L.moe_route_dispatch.restype = I
        L.moe_route_dispatch.argtypes = [P, I, P, I, P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]
        L.moe_pack_weights.restype = I
        L.moe_pack_weights.argtypes = [P, I, I, I, I, P, P]
        L.moe_pack_router.restype = I
        L.moe_pack_router.argtypes = [P, I, I, I, P, P]
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise MoEError(fn, status, lib().moe_status_str(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    if not t.is_cuda:  # every array of the ABI is device memory; a host pointer would fault the GPU
        raise ValueError("tensors passed to the MoE library must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def moe_version() -> int:
    return lib().moe_version()


def moe_route(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor], k: int,
              topk_ids: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None, stream=None):
    """Router logits (canonical fp32 FMA chain), top-k, renormalised gates -> (topk_ids, topk_w)."""
    T, H = x.shape
    E = w_router.shape[0]
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check("moe_route", lib().moe_route(_ptr(x), _dtype(x), _ptr(w_router), _dtype(w_router), _ptr(bias), T, H, E, k,
                                        _ptr(topk_ids), _ptr(topk_w), _stream(stream)))
    return topk_ids, topk_w


def moe_permute(topk_ids: torch.Tensor, topk_w: torch.Tensor, E: int, e_begin: int, e_end: int,
                x: Optional[torch.Tensor] = None, x_perm: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                stream=None) -> dict:
    """Counts, offsets and the stable by-expert grouping of the local assignments.

    Returns dict(counts, offsets, row_token, row_w, token_row[, x_perm]); row
    buffers have R_cap = T*min(k, E_loc) entries, the first offsets[-1] are valid."""
    T, k = topk_ids.shape
    El = e_end - e_begin
    R_cap = T * min(k, El)
    dev = topk_ids.device
    o = dict(out) if out else {}
    o.setdefault("counts", torch.empty(El, dtype=torch.int32, device=dev))
    o.setdefault("offsets", torch.empty(El + 1, dtype=torch.int32, device=dev))
    o.setdefault("row_token", torch.empty(max(R_cap, 1), dtype=torch.int32, device=dev))
    o.setdefault("row_w", torch.empty(max(R_cap, 1), dtype=torch.float32, device=dev))
    o.setdefault("token_row", torch.empty((T, k), dtype=torch.int32, device=dev))
    o.setdefault("workspace", torch.empty(max(moe_permute_workspace_size(T, k, El), 256), dtype=torch.uint8, device=dev))
    H = 0
    xdt = MOE_BF16
    if x is not None:
        H = x.shape[1]
        xdt = _dtype(x)
        if x_perm is None:
            x_perm = torch.empty((max(R_cap, 1), H), dtype=x.dtype, device=dev)
        o["x_perm"] = x_perm
    _check("moe_permute", lib().moe_permute(_ptr(topk_ids), _ptr(topk_w), T, k, E, e_begin, e_end,
                                            _ptr(o["counts"]), _ptr(o["offsets"]), _ptr(o["row_token"]),
                                            _ptr(o["row_w"]), _ptr(o["token_row"]), _ptr(x), xdt, H,
                                            _ptr(x_perm), _ptr(o["workspace"]),
                                            o["workspace"].numel() * o["workspace"].element_size(), _stream(stream)))
    o["R_cap"] = R_cap
    return o


def moe_workspace_size(op: int, T: int, k: int, E_loc: int, H: int, I: int) -> int:
    """Bytes of workspace one call of ``op`` (MOE_OP_*) needs."""
    return int(lib().moe_workspace_size(op, T, k, E_loc, H, I))


def moe_permute_workspace_size(T: int, k: int, E_loc: int) -> int:
    return int(lib().moe_permute_workspace_size(T, k, E_loc))


def moe_ffn_workspace_size(R_cap: int, E_loc: int, H: int, I: int, a_dtype: int) -> int:
    return int(lib().moe_ffn_workspace_size(R_cap, E_loc, H, I, a_dtype))


def moe_grouped_ffn(a: torch.Tensor, offsets: torch.Tensor, row_token: torch.Tensor, row_w: torch.Tensor, T: int,
                    R_cap: int, w_gate_up: torch.Tensor, w_down: torch.Tensor,
                    s_gate_up: Optional[torch.Tensor] = None, s_down: Optional[torch.Tensor] = None,
                    y: Optional[torch.Tensor] = None, y_perm: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, gather: bool = True, zero_y: bool = True,
                    phase: str = "both", packed: bool = False, stream=None):
    """SwiGLU expert FFN over the grouped rows.  With ``y`` the gate-weighted combine is
    fused (y accumulates; zeroed first when ``zero_y``); otherwise writes ``y_perm``.
    ``phase``: "both", "gate_up" or "down" (the two halves, same arguments and workspace).
    ``packed``: both weight tensors come from moe_pack_weights."""
    El, twoI, H = w_gate_up.shape
    I = twoI // 2
    adt = _dtype(a)
    need = moe_ffn_workspace_size(R_cap, El, H, I, adt)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
    flags = (MOE_FFN_GATHER if gather else 0) | (MOE_FFN_ZERO_Y if zero_y else 0)
    flags |= {"both": 0, "gate_up": MOE_FFN_ONLY_GATE_UP, "down": MOE_FFN_ONLY_DOWN}[phase]
    flags |= MOE_FFN_PACKED_WEIGHTS if packed else 0
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _ptr(a), adt, _ptr(offsets), _ptr(row_token), _ptr(row_w), El, T, R_cap, H, I, _ptr(w_gate_up),
        _ptr(w_down), _dtype(w_gate_up), _ptr(s_gate_up), _ptr(s_down), _ptr(y), _ptr(y_perm), _ptr(workspace),
        workspace.numel() * workspace.element_size(), flags, _stream(stream)))
    return y if y is not None else y_perm


def moe_grouped_ffn_noalloc(a: torch.Tensor, offsets: torch.Tensor, row_token: torch.Tensor, row_w: torch.Tensor,
                            T: int, R_cap: int, w_gate_up: torch.Tensor, w_down: torch.Tensor,
                            s_gate_up: Optional[torch.Tensor] = None, s_down: Optional[torch.Tensor] = None,
                            y: Optional[torch.Tensor] = None, y_perm: Optional[torch.Tensor] = None,
                            gather: bool = True, zero_y: bool = True, phase: str = "both", packed: bool = False,
                            stream=None):
    """moe_grouped_ffn with its intermediate in the library's static per-GPU scratch array (no
    workspace argument, nothing allocated by the call).  Calls on one GPU must not overlap."""
    El, twoI, H = w_gate_up.shape
    I = twoI // 2
    flags = (MOE_FFN_GATHER if gather else 0) | (MOE_FFN_ZERO_Y if zero_y else 0)
    flags |= {"both": 0, "gate_up": MOE_FFN_ONLY_GATE_UP, "down": MOE_FFN_ONLY_DOWN}[phase]
    flags |= MOE_FFN_PACKED_WEIGHTS if packed else 0
    _check("moe_grouped_ffn_noalloc", lib().moe_grouped_ffn_noalloc(
        _ptr(a), _dtype(a), _ptr(offsets), _ptr(row_token), _ptr(row_w), El, T, R_cap, H, I, _ptr(w_gate_up),
        _ptr(w_down), _dtype(w_gate_up), _ptr(s_gate_up), _ptr(s_down), _ptr(y), _ptr(y_perm), flags,
        _stream(stream)))
    return y if y is not None else y_perm


def moe_quantize_mx(x: torch.Tensor, codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                    stream=None):
    """MXFP8 quantisation of a [rows, K] fp32/bf16 tensor -> (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    rows, K = x.shape
    if codes is None:
        codes = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    _check("moe_quantize_mx", lib().moe_quantize_mx(_ptr(x), _dtype(x), rows, K, _ptr(codes), _ptr(scales),
                                                    _stream(stream)))
    return codes, scales


def moe_ffn_mx_workspace_size(R_cap: int, I: int) -> int:
    return int(lib().moe_ffn_mx_workspace_size(R_cap, I))


def moe_grouped_ffn_mx(a_codes: torch.Tensor, a_scales: torch.Tensor, offsets: torch.Tensor, row_token: torch.Tensor,
                       row_w: torch.Tensor, T: int, R_cap: int, wgu_codes: torch.Tensor, wgu_scales: torch.Tensor,
                       wd_codes: torch.Tensor, wd_scales: torch.Tensor, y: Optional[torch.Tensor] = None,
                       y_perm: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       gather: bool = True, zero_y: bool = True, phase: str = "both", packed: bool = False,
                       stream=None):
    """W8A8 MXFP8 SwiGLU expert FFN (activations and weights as MX codes + E8M0 scales).  ``packed``:
    the weight codes are in the packed block layout (moe_pack_weights); scales stay row-major."""
    El, twoI, H = wgu_codes.shape
    I = twoI // 2
    need = moe_ffn_mx_workspace_size(R_cap, I)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=a_codes.device)
    flags = (MOE_FFN_GATHER if gather else 0) | (MOE_FFN_ZERO_Y if zero_y else 0)
    flags |= {"both": 0, "gate_up": MOE_FFN_ONLY_GATE_UP, "down": MOE_FFN_ONLY_DOWN}[phase]
    flags |= MOE_FFN_PACKED_WEIGHTS if packed else 0
    _check("moe_grouped_ffn_mx", lib().moe_grouped_ffn_mx(
        _ptr(a_codes), _ptr(a_scales), _ptr(offsets), _ptr(row_token), _ptr(row_w), El, T, R_cap, H, I,
        _ptr(wgu_codes), _ptr(wgu_scales), _ptr(wd_codes), _ptr(wd_scales), _ptr(y), _ptr(y_perm), _ptr(workspace),
        workspace.numel() * workspace.element_size(), flags, _stream(stream)))
    return y if y is not None else y_perm


def moe_combine(y_perm: torch.Tensor, token_row: torch.Tensor, topk_w: torch.Tensor, y: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    T, k = token_row.shape
    H = y_perm.shape[1]
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=y_perm.device)
    _check("moe_combine", lib().moe_combine(_ptr(y_perm), _ptr(token_row), _ptr(topk_w), T, k, H, _ptr(y),
                                            _stream(stream)))
    return y


def moe_shared_workspace_size(T: int, I_s: int, x_dtype: int) -> int:
    return int(lib().moe_shared_workspace_size(T, I_s, x_dtype))


def moe_shared_expert(x: torch.Tensor, w_gate_up: torch.Tensor, w_down: torch.Tensor, y: torch.Tensor,
                      s_gate_up: Optional[torch.Tensor] = None, s_down: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, zero_y: bool = False, packed: bool = False,
                      stream=None):
    """y += shared-expert SwiGLU FFN of x (every token, weight 1); ``zero_y`` zeroes y first;
    ``packed``: both weight tensors come from moe_pack_weights."""
    T, H = x.shape
    I_s = w_gate_up.shape[0] // 2
    xdt = _dtype(x)
    need = moe_shared_workspace_size(T, I_s, xdt)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check("moe_shared_expert", lib().moe_shared_expert(
        _ptr(x), xdt, T, H, I_s, _ptr(w_gate_up), _ptr(w_down), _dtype(w_gate_up), _ptr(s_gate_up), _ptr(s_down),
        _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(),
        (MOE_FFN_ZERO_Y if zero_y else 0) | (MOE_FFN_PACKED_WEIGHTS if packed else 0), _stream(stream)))
    return y


def moe_pack_weights(w: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Weights [E, N, K] (or [N, K], one expert) in the packed block layout, as a tensor of the
    same shape and dtype (pass it with ``packed=True``)."""
    E, N, K = (1, *w.shape) if w.dim() == 2 else w.shape
    if out is None:
        out = torch.empty_like(w)
    if out.shape != w.shape or out.dtype != w.dtype:
        raise ValueError("out must have the shape and dtype of w")
    _check("moe_pack_weights", lib().moe_pack_weights(_ptr(w), _dtype(w), E, N, K, _ptr(out), _stream(stream)))
    return out


def moe_route_dispatch_workspace(device="cuda") -> torch.Tensor:
    """A zeroed workspace for moe_route_dispatch (its ticket counter starts at zero)."""
    return torch.zeros(int(lib().moe_route_dispatch_workspace_size()), dtype=torch.uint8, device=device)


def moe_pack_router(w_router: torch.Tensor, stream=None) -> torch.Tensor:
    """The router weight [E, H] (bf16 or fp32) as exact fp32 in the layout of moe_pack_router,
    [H/4, E, 4]; pass it to moe_route_dispatch with ``router_packed=True``."""
    E, H = w_router.shape
    out = torch.empty((H // 4, E, 4), dtype=torch.float32, device=w_router.device)
    _check("moe_pack_router", lib().moe_pack_router(_ptr(w_router), _dtype(w_router), E, H, _ptr(out),
                                                    _stream(stream)))
    return out


def moe_route_dispatch(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor], k: int, E: int,
                       e_begin: int, e_end: int, workspace: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                       out: dict, y_zero: Optional[torch.Tensor] = None, router_packed: bool = False,
                       stream=None) -> dict:
    """Route + local dispatch of a decode batch in one launch; ``out`` holds counts, offsets,
    row_token, row_w, token_row (as from moe_permute); zeroes ``y_zero`` when given.
    ``router_packed``: ``w_router`` is the fp32 [H/4, E, 4] tensor of moe_pack_router (the C ABI
    cannot see buffer sizes, so the layout is checked here: a raw [E, H] weight passed as packed
    would be read past its end)."""
    T, H = x.shape
    if router_packed:
        if w_router.dtype != torch.float32 or tuple(w_router.shape) != (H // 4, E, 4) or H % 4 != 0:
            raise ValueError(f"router_packed needs the fp32 [H/4, E, 4] = {(H // 4, E, 4)} tensor of moe_pack_router, "
                             f"got {w_router.dtype} {tuple(w_router.shape)}")
    elif tuple(w_router.shape) != (E, H):
        raise ValueError(f"w_router must be [E, H] = {(E, H)}, got {tuple(w_router.shape)}")
    _check("moe_route_dispatch", lib().moe_route_dispatch(
        _ptr(x), _dtype(x), _ptr(w_router), MOE_F32_ROUTER_PACKED if router_packed else _dtype(w_router), _ptr(bias),
        T, H, E, k, e_begin, e_end, _ptr(topk_ids),
        _ptr(topk_w), _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["row_token"]), _ptr(out["row_w"]),
        _ptr(out["token_row"]), _ptr(y_zero), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def moe_decode_layer_workspace(T: int, k: int, E_loc: int, I: int, device="cuda") -> torch.Tensor:
    """A zeroed workspace for moe_decode_layer (its control words must start at zero)."""
    return torch.zeros(int(lib().moe_decode_layer_workspace_size(T, k, E_loc, I)), dtype=torch.uint8, device=device)


def moe_decode_layer(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor], k: int, E: int,
                     e_begin: int, e_end: int, w_gate_up: torch.Tensor, w_down: torch.Tensor,
                     s_gate_up: Optional[torch.Tensor], s_down: Optional[torch.Tensor], workspace: torch.Tensor,
                     topk_ids: torch.Tensor, topk_w: torch.Tensor, out: dict, y: torch.Tensor,
                     router_packed: bool = False, packed: bool = False, stream=None) -> torch.Tensor:
    """The whole decode layer in one launch: routing into ``topk_ids``/``topk_w``, the grouping into
    ``out`` (counts, offsets, row_token, row_w, token_row as from moe_permute) and y [T, H]
    (overwritten).  ``router_packed``: ``w_router`` is the moe_pack_router tensor; ``packed``: the
    expert weights come from moe_pack_weights."""
    T, H = x.shape
    El, twoI, _ = w_gate_up.shape
    if router_packed:
        if w_router.dtype != torch.float32 or tuple(w_router.shape) != (H // 4, E, 4):
            raise ValueError(f"router_packed needs the fp32 [H/4, E, 4] = {(H // 4, E, 4)} tensor of moe_pack_router, "
                             f"got {w_router.dtype} {tuple(w_router.shape)}")
    elif tuple(w_router.shape) != (E, H):
        raise ValueError(f"w_router must be [E, H] = {(E, H)}, got {tuple(w_router.shape)}")
    if El != e_end - e_begin or tuple(w_down.shape) != (El, H, twoI // 2):
        raise ValueError("expert weights must be [E_loc, 2I, H] and [E_loc, H, I]")
    _check("moe_decode_layer", lib().moe_decode_layer(
        _ptr(x), _dtype(x), _ptr(w_router), MOE_F32_ROUTER_PACKED if router_packed else _dtype(w_router), _ptr(bias),
        T, H, E, k, e_begin, e_end, twoI // 2, _ptr(w_gate_up), _ptr(w_down), _dtype(w_gate_up), _ptr(s_gate_up),
        _ptr(s_down), _ptr(topk_ids), _ptr(topk_w), _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["row_token"]),
        _ptr(out["row_w"]), _ptr(out["token_row"]), _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(),
        MOE_FFN_PACKED_WEIGHTS if packed else 0, _stream(stream)))
    return y


def decode_layer_error_word(workspace: torch.Tensor) -> int:
    """The diagnostic word of a moe_decode_layer workspace (nonzero: a wait in the kernel gave up)."""
    return int(workspace[16:20].view(torch.int32).item())
