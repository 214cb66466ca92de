"""Python face of the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only users.  The GPU library never
imports this module and this module imports nothing from the GPU library.

Dtype codes: 0 = fp32, 1 = bf16 (uint16 bit patterns), 2 = fp8 e4m3 (uint8 codes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DT = {"f32": 0, "bf16": 1, "fp8": 2}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc: plain -O2, OpenMP, no fp contraction, no fast-math."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None
_lib_path = None  # None: the library built from moe_oracle.c


def use_library(path):
    """Load the oracle from another build of moe_oracle.c (the pin tests use this to
    check that planted mistakes are caught); ``None`` restores the default."""
    global _lib, _lib_path
    _lib, _lib_path = None, path


def lib():
    global _lib
    if _lib is None:
        if _lib_path is None:
            build()
        L = ctypes.CDLL(_lib_path or LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        L.oracle_router_logits.argtypes = [P, i, P, i, P, i, i, i, P]
        L.oracle_topk.argtypes = [P, i, i, i, P, P]
        L.oracle_topk.restype = i
        L.oracle_route.argtypes = [P, i, P, i, P, i, i, i, i, P, P, P]
        L.oracle_route.restype = i
        L.oracle_permute.argtypes = [P, P, i, i, i, i, P, P, P, P, P]
        L.oracle_permute.restype = i
        L.oracle_layer_tokens.argtypes = [P, i, P, i, P, P, i, i, i, i, i, i, P, P, i, P, P, i, P]
        L.oracle_combine.argtypes = [P, P, P, i, i, i, P]
        L.oracle_num_threads.restype = i
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_mx_scale.restype = ctypes.c_uint8
        L.oracle_mx_scale.argtypes = [ctypes.c_double]
        L.oracle_mx_quantize.argtypes = [P, i, i, i, P, P]
        L.oracle_layer_tokens_mx.argtypes = [P, i, P, i, P, P, i, i, i, i, i, P, P, P, P, P]
        L.oracle_h_mx.argtypes = [P, P, i, P, i, i, i, P, P, P, P]
        L.oracle_shared_tokens.argtypes = [P, i, P, i, i, i, P, P, i, P, P, i, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt_of(a: np.ndarray) -> int:
    return {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.uint8): 2}[a.dtype]


def num_threads() -> int:
    return lib().oracle_num_threads()


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def bf16_round(values) -> np.ndarray:
    v = np.asarray(values, dtype=np.float32).ravel()
    return np.array([lib().oracle_bf16_round(float(f)) for f in v], dtype=np.uint16)


def router_logits(x, w_router, bias=None) -> np.ndarray:
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w_router)
    T, H = x.shape
    E = w.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib().oracle_router_logits(_p(x), _dt_of(x), _p(w), _dt_of(w), _p(b), T, H, E, _p(out))
    return out


def topk(logits, k: int):
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    if lib().oracle_topk(_p(lg), T, E, k, _p(ids), _p(w)) != 0:
        raise ValueError("bad k")
    return ids, w


def route(x, w_router, bias, k: int):
    """Returns (topk_ids [T,k] int32, topk_w [T,k] fp32, logits [T,E] fp32)."""
    lg = router_logits(x, w_router, bias)
    ids, w = topk(lg, k)
    return ids, w, lg


def permute(topk_ids, topk_w, e_begin: int, e_end: int) -> dict:
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, k = ids.shape
    El = e_end - e_begin
    counts = np.empty(El, dtype=np.int32)
    offsets = np.empty(El + 1, dtype=np.int32)
    cap = max(1, T * min(k, max(El, 1)))
    row_token = np.full(cap, -1, dtype=np.int32)
    row_w = np.zeros(cap, dtype=np.float32)
    token_row = np.empty((T, k), dtype=np.int32)
    R = lib().oracle_permute(_p(ids), _p(w), T, k, e_begin, e_end, _p(counts), _p(offsets),
                             _p(row_token), _p(row_w), _p(token_row))
    return dict(counts=counts, offsets=offsets, row_token=row_token[:R], row_w=row_w[:R],
                token_row=token_row, R=R)


def layer_tokens(tokens, x, topk_ids, topk_w, e_begin: int, e_end: int, w_gate_up, w_down,
                 s_gate_up=None, s_down=None, round_h: bool = True) -> np.ndarray:
    """y rows (fp32 [len(tokens), H]) of the listed tokens, token-major."""
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    wgu = np.ascontiguousarray(w_gate_up)
    wd = np.ascontiguousarray(w_down)
    T, H = x.shape
    k = ids.shape[1]
    I = wd.shape[2]
    assert wgu.shape[1:] == (2 * I, H) and wd.shape[1:] == (H, I)
    assert wgu.dtype == wd.dtype
    sgu = None if s_gate_up is None else np.ascontiguousarray(s_gate_up, dtype=np.float32)
    sd = None if s_down is None else np.ascontiguousarray(s_down, dtype=np.float32)
    if _dt_of(wgu) == 2:
        assert sgu is not None and sd is not None
    y = np.empty((len(tok), H), dtype=np.float32)
    lib().oracle_layer_tokens(_p(tok), len(tok), _p(x), _dt_of(x), _p(ids), _p(w), T, H, k, e_begin, e_end, I,
                              _p(wgu), _p(wd), _dt_of(wgu), _p(sgu), _p(sd), 1 if round_h else 0, _p(y))
    return y


def shared_tokens(tokens, x, w_gate_up, w_down, s_gate_up=None, s_down=None, round_h: bool = True) -> np.ndarray:
    """R10: the shared expert's contribution (fp32 [len(tokens), H]) for the listed tokens."""
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    x = np.ascontiguousarray(x)
    wgu = np.ascontiguousarray(w_gate_up)
    wd = np.ascontiguousarray(w_down)
    T, H = x.shape
    I_s = wd.shape[1]
    assert wgu.shape == (2 * I_s, H) and wd.shape == (H, I_s) and wgu.dtype == wd.dtype
    sgu = None if s_gate_up is None else np.ascontiguousarray(s_gate_up, dtype=np.float32)
    sd = None if s_down is None else np.ascontiguousarray(s_down, dtype=np.float32)
    if _dt_of(wgu) == 2:
        assert sgu is not None and sd is not None
    y = np.empty((len(tok), H), dtype=np.float32)
    lib().oracle_shared_tokens(_p(tok), len(tok), _p(x), _dt_of(x), H, I_s, _p(wgu), _p(wd), _dt_of(wgu), _p(sgu),
                               _p(sd), 1 if round_h else 0, _p(y))
    return y


def e4m3_encode(v: float) -> int:
    """R8: nearest e4m3 code (ties to even, saturating at 448, sign kept)."""
    return int(lib().oracle_e4m3_encode(float(v)))


def mx_scale(amax: float) -> int:
    """R8: E8M0 scale byte of a block whose largest magnitude is ``amax``."""
    return int(lib().oracle_mx_scale(float(amax)))


def mx_quantize(x) -> tuple:
    """R8: rows x K (fp32 or bf16 bits) -> (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    x = np.ascontiguousarray(x)
    rows, K = x.shape
    assert K % 32 == 0
    codes = np.empty((rows, K), dtype=np.uint8)
    scales = np.empty((rows, K // 32), dtype=np.uint8)
    lib().oracle_mx_quantize(_p(x), _dt_of(x), rows, K, _p(codes), _p(scales))
    return codes, scales


def mx_dequantize(codes, scales) -> np.ndarray:
    """Exact values of an MX tensor (fp64)."""
    table = np.array([e4m3_value(c) for c in range(256)])
    v = table[np.asarray(codes)]
    return v * np.ldexp(1.0, np.repeat(np.asarray(scales, dtype=np.int64), 32, axis=-1) - 127)


def layer_tokens_mx(tokens, x, topk_ids, topk_w, e_begin: int, e_end: int, wgu_q, wgu_s, wd_q, wd_s) -> np.ndarray:
    """W8A8 MXFP8 layer: y rows (fp32 [len(tokens), H]) of the listed tokens, token-major."""
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    wgu_q, wgu_s = np.ascontiguousarray(wgu_q, dtype=np.uint8), np.ascontiguousarray(wgu_s, dtype=np.uint8)
    wd_q, wd_s = np.ascontiguousarray(wd_q, dtype=np.uint8), np.ascontiguousarray(wd_s, dtype=np.uint8)
    T, H = x.shape
    k = ids.shape[1]
    I = wd_q.shape[2]
    assert wgu_q.shape[1:] == (2 * I, H) and wd_q.shape[1:] == (H, I)
    assert wgu_s.shape[1:] == (2 * I, H // 32) and wd_s.shape[1:] == (H, I // 32)
    y = np.empty((len(tok), H), dtype=np.float32)
    lib().oracle_layer_tokens_mx(_p(tok), len(tok), _p(x), _dt_of(x), _p(ids), _p(w), H, k, e_begin, e_end, I,
                                 _p(wgu_q), _p(wgu_s), _p(wd_q), _p(wd_s), _p(y))
    return y


def h_mx(row_token, row_expert, x, wgu_q, wgu_s) -> tuple:
    """MXFP8 intermediate (codes [R, I], scales [R, I/32]) of assignment rows (token, local expert)."""
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    re_ = np.ascontiguousarray(row_expert, dtype=np.int32)
    x = np.ascontiguousarray(x)
    wgu_q, wgu_s = np.ascontiguousarray(wgu_q, dtype=np.uint8), np.ascontiguousarray(wgu_s, dtype=np.uint8)
    T, H = x.shape
    I = wgu_q.shape[1] // 2
    R = len(rt)
    codes = np.empty((R, I), dtype=np.uint8)
    scales = np.empty((R, I // 32), dtype=np.uint8)
    lib().oracle_h_mx(_p(rt), _p(re_), R, _p(x), _dt_of(x), H, I, _p(wgu_q), _p(wgu_s), _p(codes), _p(scales))
    return codes, scales


def combine(y_perm, token_row, topk_w) -> np.ndarray:
    yp = np.ascontiguousarray(y_perm, dtype=np.float32)
    tr = np.ascontiguousarray(token_row, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, k = tr.shape
    H = yp.shape[1] if yp.ndim == 2 else 0
    y = np.empty((T, H), dtype=np.float32)
    lib().oracle_combine(_p(yp), _p(tr), _p(w), T, k, H, _p(y))
    return y


def layer(inputs: dict, tokens=None, round_h=None):
    """Whole layer for a synthetic-input dict: routing, permutation, y of ``tokens``
    (all tokens when None).  ``round_h`` defaults to True unless activations are fp32."""
    cfg = inputs["cfg"]
    ids, w, lg = route(inputs["x"], inputs["w_router"], inputs.get("bias"), cfg.k)
    perm = permute(ids, w, cfg.lo, cfg.hi)
    if tokens is None:
        tokens = np.arange(cfg.T, dtype=np.int32)
    if round_h is None:
        round_h = cfg.act != "f32"
    y = layer_tokens(tokens, inputs["x"], ids, w, cfg.lo, cfg.hi, inputs["w_gate_up"], inputs["w_down"],
                     inputs.get("s_gate_up"), inputs.get("s_down"), round_h=round_h)
    return dict(topk_ids=ids, topk_w=w, logits=lg, y=y, tokens=np.asarray(tokens, dtype=np.int32), **perm)
