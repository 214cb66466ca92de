"""Seeded synthetic inputs for the MoE FFN layer.

This module only *makes data*: it draws Gaussian tensors, rounds them to their
storage type (bf16 / fp8 e4m3 with a per-output-channel scale) and builds the
Zipf logit bias of the skewed-routing workload.  It holds none of the layer's
arithmetic, so both the GPU path (tests, bench) and the CPU oracle (tests) can
take their inputs from here without sharing any computation.

Workloads (shapes follow the pages):
  * ``tiny``      fp32, T=64, H=256, E=8, top-2, I=128 (inputs N(0,1)/sqrt(fan_in)).
  * ``decode``    T=64 tokens x top-8 of 128 experts = 512 assignments, the
                  decode batch of the AI-infra book, ch. 9, section 9.3.3.
                  Expert shape 3 x 4096 x 1536 (Qwen3-235B-A22B, section 9.3.2).
  * ``prefill``   T=6000, about 6000*8/128 = 375 rows per expert, the prefill
                  shape of "Hosting Qwen on Blackwell", section "Prefillers".
  * ``skew``      prefill + a per-expert logit bias 2*ln(Zipf(1.2) weight of
                  rank e+1), a hot-expert load in the spirit of the book's
                  section 9.4.1 skew examples.
  * ``ep_share``  T=8192, routed over 128 experts but only experts 0..31 are
                  local (one rank of the EP=4 prefill sharding, "Hosting Qwen
                  on Blackwell", sections "Prefillers" and "Expert
                  parallelism"); fp8 e4m3 weights with fp32 per-channel scales.

Storage conventions (arrays are numpy, row-major):
  bf16 values are stored as ``uint16`` bit patterns, fp8 e4m3 as ``uint8``
  codes (OCP E4M3: bias 7, no infinities, 0x7F/0xFF are NaN, max 448).

RNG: numpy PCG64 streams keyed by ``SeedSequence([1000*seed + stream, index])``
with stream 1 = x, 2 = router weight, 3 = gate/up weights, 4 = down weights and
index = the global expert id for expert weights (0 otherwise).  Every expert's
weights can therefore be generated on its own, in any order or in parallel.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = [
    "LayerConfig", "CONFIGS", "make_inputs", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "quantize_e4m3_per_row", "zipf_logit_bias", "gen_x", "gen_router", "gen_expert",
]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    act: str = "bf16"          # 'f32' | 'bf16'  (activations and router weight)
    wdt: str = "bf16"          # 'f32' | 'bf16' | 'fp8' | 'mxfp8' (expert weights)
    e_begin: int = 0
    e_end: Optional[int] = None  # None -> E
    bias: str = "none"         # 'none' | 'zipf'
    zipf_s: float = 1.2
    bias_scale: float = 2.0
    init: str = "fixed"        # 'fixed': x~N(0,1), W~N(0,0.02); 'fan_in': N(0,1)/sqrt(fan_in)
    x_std: float = 1.0
    w_std: float = 0.02
    seed: int = 0
    I_s: int = 0               # intermediate size of the shared expert (0: none)

    @property
    def lo(self) -> int:
        return self.e_begin

    @property
    def hi(self) -> int:
        return self.E if self.e_end is None else self.e_end

    @property
    def E_loc(self) -> int:
        return self.hi - self.lo

    @property
    def R_cap(self) -> int:
        """Upper bound on local assignments: each token has k distinct experts."""
        return self.T * min(self.k, self.E_loc)

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  ``seed`` is the workload number.
CONFIGS = {
    "tiny": LayerConfig("tiny", T=64, H=256, E=8, k=2, I=128, act="f32", wdt="f32", init="fan_in", seed=1),
    "decode": LayerConfig("decode", T=64, H=4096, E=128, k=8, I=1536, seed=2),
    "prefill": LayerConfig("prefill", T=6000, H=4096, E=128, k=8, I=1536, seed=3),
    "skew": LayerConfig("skew", T=6000, H=4096, E=128, k=8, I=1536, bias="zipf", seed=4),
    "ep_share": LayerConfig("ep_share", T=8192, H=4096, E=128, k=8, I=1536, wdt="fp8", e_begin=0, e_end=32, seed=5),
    # W8A8 MXFP8 variant of the prefill layer (weights converted offline, activations on the fly)
    "prefill_mx": LayerConfig("prefill_mx", T=6000, H=4096, E=128, k=8, I=1536, wdt="mxfp8", seed=6),
    "decode_mx": LayerConfig("decode_mx", T=64, H=4096, E=128, k=8, I=1536, wdt="mxfp8", seed=9),
    # the decode and prefill layers with one always-active shared expert of a routed expert's shape
    "decode_shared": LayerConfig("decode_shared", T=64, H=4096, E=128, k=8, I=1536, seed=7, I_s=1536),
    "prefill_shared": LayerConfig("prefill_shared", T=6000, H=4096, E=128, k=8, I=1536, seed=8, I_s=1536),
}


# ----------------------------------------------------------------------------
# Storage-type rounding (data preparation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); returns uint16 bit patterns.

    Inputs must be finite (the generator never makes NaN/Inf)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_table() -> np.ndarray:
    """Values of the 127 non-negative finite e4m3 codes 0x00..0x7E (index = code)."""
    codes = np.arange(0x7F)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3_POS = _e4m3_table()


def _encode_e4m3(v: np.ndarray) -> np.ndarray:
    """float64 -> e4m3 codes, round to nearest (ties to even code), saturating to 448."""
    a = np.minimum(np.abs(v), 448.0)
    idx = np.searchsorted(_E4M3_POS, a)          # first value >= a
    idx = np.clip(idx, 1, len(_E4M3_POS) - 1)
    lo = _E4M3_POS[idx - 1]
    hi = _E4M3_POS[idx]
    dlo = a - lo
    dhi = hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (idx % 2 == 0))
    code = np.where(pick_hi, idx, idx - 1)
    code = np.where(a == 0.0, 0, code)
    sign = np.where(np.signbit(v) & (code != 0), 0x80, 0)
    return (code | sign).astype(np.uint8)


def quantize_e4m3_per_row(w: np.ndarray):
    """Per-output-channel (last axis reduced) fp8 e4m3 quantisation of float32 ``w``.

    scale[n] = max_h |w[n,h]| / 448 (fp32), code = RNE-saturate(w / scale).
    Returns (codes uint8 same shape, scales float32 shape[:-1])."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=-1)
    scale = (amax.astype(np.float64) / 448.0).astype(np.float32)
    scale = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    codes = _encode_e4m3(w.astype(np.float64) / scale[..., None].astype(np.float64))
    return codes, scale


def mx_weights(rng: np.random.Generator, shape: tuple, std: float):
    """A synthetic MXFP8 weight tensor (blocks of 32 along the last axis) with a spread close to
    ``std``: the power of two nearest std/32, times a per-block jitter of 1/2, 1 or 2, is each
    block's E8M0 scale, and its e4m3 codes are the nearest codes of N(0, 32^2) draws divided
    by that jitter.  Returns (codes uint8 shape, scales uint8 shape[:-1] + (K/32,))."""
    K = shape[-1]
    base = 127 + int(np.round(np.log2(std / 32.0)))
    jitter = rng.integers(-1, 2, size=shape[:-1] + (K // 32,))
    v = rng.standard_normal(shape, dtype=np.float32).astype(np.float64) * 32.0
    v = v.reshape(shape[:-1] + (K // 32, 32)) * np.ldexp(1.0, -jitter)[..., None]
    codes = _encode_e4m3(v).reshape(shape)
    return codes, (base + jitter).astype(np.uint8)


def zipf_logit_bias(E: int, s: float = 1.2, scale: float = 2.0) -> np.ndarray:
    """bias[e] = scale * ln(p_{e+1}), p_r = r^-s / sum_{r=1..E} r^-s (fp64, stored fp32)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p = p / p.sum()
    return (scale * np.log(p)).astype(np.float32)


# ----------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------
def _rng(cfg: LayerConfig, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 * cfg.seed + stream, index])))


def _store(a32: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f32":
        return a32.astype(np.float32)
    if dt == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(dt)


def _stds(cfg: LayerConfig):
    if cfg.init == "fan_in":
        return (1.0 / np.sqrt(cfg.H), 1.0 / np.sqrt(cfg.H), 1.0 / np.sqrt(cfg.H), 1.0 / np.sqrt(cfg.I))
    return (cfg.x_std, cfg.w_std, cfg.w_std, cfg.w_std)


def gen_x(cfg: LayerConfig) -> np.ndarray:
    sx = _stds(cfg)[0]
    a = _rng(cfg, 1).standard_normal((cfg.T, cfg.H), dtype=np.float32) * np.float32(sx)
    return _store(a, cfg.act)


def gen_router(cfg: LayerConfig) -> np.ndarray:
    sr = _stds(cfg)[1]
    a = _rng(cfg, 2).standard_normal((cfg.E, cfg.H), dtype=np.float32) * np.float32(sr)
    return _store(a, cfg.act)


def gen_expert(cfg: LayerConfig, e: int):
    """Weights of global expert ``e``: (w_gate_up [2I,H], w_down [H,I], s_gate_up, s_down).

    Rows 0..I-1 of w_gate_up are the gate projection, rows I..2I-1 the up projection.
    Scales are None unless the weight type is fp8."""
    _, _, sgu, sd = _stds(cfg)
    if cfg.wdt == "mxfp8":  # weights arrive already converted: draw codes and block scales directly
        qgu, s_gu = mx_weights(_rng(cfg, 3, e), (2 * cfg.I, cfg.H), sgu)
        qd, s_d = mx_weights(_rng(cfg, 4, e), (cfg.H, cfg.I), sd)
        return qgu, qd, s_gu, s_d
    gu = _rng(cfg, 3, e).standard_normal((2 * cfg.I, cfg.H), dtype=np.float32) * np.float32(sgu)
    dn = _rng(cfg, 4, e).standard_normal((cfg.H, cfg.I), dtype=np.float32) * np.float32(sd)
    if cfg.wdt == "fp8":
        qgu, s_gu = quantize_e4m3_per_row(gu)
        qd, s_d = quantize_e4m3_per_row(dn)
        return qgu, qd, s_gu, s_d
    return _store(gu, cfg.wdt), _store(dn, cfg.wdt), None, None


SHARED_INDEX = 1 << 20  # draw index of the shared expert's weights (routed experts use 0..E-1)


def gen_shared(cfg: LayerConfig):
    """Weights of the shared expert, drawn like a routed expert's with intermediate size I_s:
    (w_gate_up [2 I_s, H], w_down [H, I_s], s_gate_up, s_down)."""
    assert cfg.I_s > 0 and cfg.wdt != "mxfp8"
    return gen_expert(cfg.replace(I=cfg.I_s), SHARED_INDEX)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_inputs(cfg: LayerConfig, experts: Optional[list] = None, with_weights: bool = True) -> dict:
    """All inputs of one layer call.

    ``experts``: global expert ids whose weights to generate (default: every
    local expert).  Weight arrays are indexed by ``e - cfg.lo``; experts not
    requested are left zero (callers that only check a sample of tokens need
    only the experts those tokens use)."""
    out = {"cfg": cfg, "x": gen_x(cfg), "w_router": gen_router(cfg)}
    out["bias"] = zipf_logit_bias(cfg.E, cfg.zipf_s, cfg.bias_scale) if cfg.bias == "zipf" else None
    if not with_weights:
        return out
    wd = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "mxfp8": np.uint8}[cfg.wdt]
    El = cfg.E_loc
    w_gu = np.zeros((El, 2 * cfg.I, cfg.H), dtype=wd)
    w_d = np.zeros((El, cfg.H, cfg.I), dtype=wd)
    s_gu = np.ones((El, 2 * cfg.I), dtype=np.float32) if cfg.wdt == "fp8" else None
    s_d = np.ones((El, cfg.H), dtype=np.float32) if cfg.wdt == "fp8" else None
    if cfg.wdt == "mxfp8":  # E8M0 block scales along the contraction axis
        s_gu = np.zeros((El, 2 * cfg.I, cfg.H // 32), dtype=np.uint8)
        s_d = np.zeros((El, cfg.H, cfg.I // 32), dtype=np.uint8)
    ids = list(range(cfg.lo, cfg.hi)) if experts is None else sorted(set(int(e) for e in experts if cfg.lo <= e < cfg.hi))

    def one(e):
        a, b, sa, sb = gen_expert(cfg, e)
        j = e - cfg.lo
        w_gu[j] = a
        w_d[j] = b
        if sa is not None:
            s_gu[j] = sa
            s_d[j] = sb

    if len(ids) > 2:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, ids))
    else:
        for e in ids:
            one(e)
    out.update(w_gate_up=w_gu, w_down=w_d, s_gate_up=s_gu, s_down=s_d, experts=ids)
    if cfg.I_s > 0:
        a, b, sa, sb = gen_shared(cfg)
        out.update(ws_gate_up=a, ws_down=b, ss_gate_up=sa, ss_down=sb)
    return out
