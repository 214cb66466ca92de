"""GPU: moe_grouped_ffn_noalloc (intermediate in the library's static per-GPU scratch array)
against moe_grouped_ffn (caller workspace) on the same inputs, through the C ABI.

Two calls in a row, the second with a smaller batch (the array keeps the first call's contents):
the per-row outputs must be bit-identical to moe_grouped_ffn's (same kernels, same inputs) and
the fused-combine output within the layer tolerance of it and of the oracle.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from expert_routed_grouped_amd import layer as L
from expert_routed_grouped_amd import moe, synth
from expert_routed_grouped_amd.synth import CONFIGS, LayerConfig

pytestmark = pytest.mark.gpu

Y_TOL = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def routed(cfg):
    inp = synth.make_inputs(cfg)
    dev = L.to_device(inp)
    ids, w, _ = O.route(inp["x"], inp["w_router"], inp["bias"], cfg.k)
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(w).cuda()
    p = moe.moe_permute(ids_d, w_d, cfg.E, cfg.lo, cfg.hi)
    return inp, dev, ids, w, p


def run_both(cfg, dev, p, fused, packed=False):
    """(output of moe_grouped_ffn_noalloc, output of moe_grouped_ffn) on the same routing."""
    args = (dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, p["R_cap"], dev["w_gate_up"], dev["w_down"],
            dev["s_gate_up"], dev["s_down"])
    outs = []
    for fn in (moe.moe_grouped_ffn_noalloc, moe.moe_grouped_ffn):
        if fused:
            out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
            fn(*args, y=out, zero_y=True, gather=True, packed=packed)
        else:
            out = torch.full((max(p["R_cap"], 1), cfg.H), float("nan"), dtype=torch.float32, device="cuda")
            fn(*args, y_perm=out, gather=True, packed=packed)
        torch.cuda.synchronize()
        outs.append(out)
    return outs


def check_close(y, y_ref, what):
    y = y.double().cpu().numpy()
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    err = np.max(np.abs(y - y_ref))
    say(f"  {what}: max|err| = {err:.3e}, RMS = {rms:.3e}")
    assert rms > 0 and err <= Y_TOL * rms


# the decode layer (weight-streaming kernel), then a batch smaller in every dimension whose 60 rows
# per expert take the tile kernels
CALLS = [CONFIGS["decode"], LayerConfig("na_small", T=60, H=512, E=2, k=2, I=256, seed=801, w_std=0.05)]


@pytest.mark.parametrize("fused", [False, True], ids=["per_row", "fused"])
def test_noalloc_matches_workspace_entry_point_twice(fused):
    for n, cfg in enumerate(CALLS):
        inp, dev, ids, w, p = routed(cfg)
        say(f"noalloc call {n + 1}: {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} R_cap={p['R_cap']} "
            f"fused={fused}")
        got, ref = run_both(cfg, dev, p, fused)
        if fused:  # fp32 atomics: the order of a token's k additions is not fixed
            check_close(got, ref.double().cpu().numpy(), f"{cfg.name} vs moe_grouped_ffn")
            y_o = O.layer_tokens(np.arange(cfg.T, dtype=np.int32), inp["x"], ids, w, cfg.lo, cfg.hi, inp["w_gate_up"],
                                 inp["w_down"], inp["s_gate_up"], inp["s_down"])
            check_close(got, y_o, f"{cfg.name} vs oracle")
        else:  # same kernels on the same inputs: every valid per-row output bit for bit
            R = int(p["offsets"][-1])
            assert R > 0
            assert torch.equal(got[:R].view(torch.int32), ref[:R].view(torch.int32))
            y = moe.moe_combine(got, p["token_row"], torch.from_numpy(w).cuda())
            y_o = O.layer_tokens(np.arange(cfg.T, dtype=np.int32), inp["x"], ids, w, cfg.lo, cfg.hi, inp["w_gate_up"],
                                 inp["w_down"], inp["s_gate_up"], inp["s_down"])
            check_close(y, y_o, f"{cfg.name} per-row outputs combined vs oracle")
        del dev
        torch.cuda.empty_cache()


def test_noalloc_halves_and_packed_weights():
    # the two halves as separate calls (h stays in the static array between them), packed weights
    cfg = LayerConfig("na_halves", T=96, H=512, E=16, k=4, I=256, seed=802, w_std=0.05)
    inp, dev, ids, w, p = routed(cfg)
    L.pack_weights(dev)
    args = (dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, p["R_cap"], dev["w_gate_up"], dev["w_down"])
    yp = torch.full((p["R_cap"], cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn_noalloc(*args, y_perm=yp, phase="gate_up", packed=True)
    moe.moe_grouped_ffn_noalloc(*args, y_perm=yp, phase="down", packed=True)
    ref = torch.full_like(yp, float("nan"))
    moe.moe_grouped_ffn(*args, y_perm=ref, packed=True)
    torch.cuda.synchronize()
    R = int(p["offsets"][-1])
    assert torch.equal(yp[:R].view(torch.int32), ref[:R].view(torch.int32))


def test_noalloc_refuses_batches_past_its_scratch():
    # 10923 rows of I = 1536 bf16 values need more than the 32 MiB array: refused, nothing enqueued
    T, H, I, El = 10923, 256, 1536, 1
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    offsets = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    rt = torch.arange(T, dtype=torch.int32, device="cuda")
    rw = torch.ones(T, dtype=torch.float32, device="cuda")
    wgu = torch.zeros((El, 2 * I, H), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((El, H, I), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, H), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoEError) as ex:
        moe.moe_grouped_ffn_noalloc(x, offsets, rt, rw, T, T, wgu, wd, y=y)
    assert ex.value.status == -4
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)  # MOE_FFN_ZERO_Y was not enqueued either
