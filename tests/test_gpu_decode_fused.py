"""GPU: moe_decode_layer (the whole decode layer in one launch) through the C ABI.

Against the four-call path on the same inputs: routing ids and gates bit for bit (moe_route), the
grouping bit for bit (moe_permute), the intermediate h of every routed (token, expert) pair bit for
bit (moe_grouped_ffn's with few rows per expert: same MFMA sequence per row), and y against the
oracle within 1e-2 * RMS.  Every call must leave the control
words of its workspace zero (repeated calls, graph replays) and its diagnostic word zero.
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
CTL_WORDS = 64  # control words before the per-expert completion counts


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def check_close(y, y_ref, what):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    err = np.max(np.abs(y - y_ref))
    say(f"  {what}: max|err| = {err:.3e}, RMS = {rms:.3e}, ratio = {err / rms:.2e}")
    assert rms > 0 and err <= Y_TOL * rms


def decode_buffers(cfg):
    d = dict(device="cuda")
    R_cap = cfg.T * min(cfg.k, cfg.E_loc)
    out = dict(counts=torch.full((cfg.E_loc,), -7, dtype=torch.int32, **d),
               offsets=torch.full((cfg.E_loc + 1,), -7, dtype=torch.int32, **d),
               row_token=torch.full((max(R_cap, 1),), -7, dtype=torch.int32, **d),
               row_w=torch.full((max(R_cap, 1),), -7.0, dtype=torch.float32, **d),
               token_row=torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, **d))
    ids = torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, **d)
    w = torch.full((cfg.T, cfg.k), -7.0, dtype=torch.float32, **d)
    y = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, **d)
    return out, ids, w, y, R_cap


def run_decode(dev, cfg, ws, router="as-stored", packed=False):
    out, ids, w, y, R_cap = decode_buffers(cfg)
    wr = dev["w_router_packed"] if router == "packed" else dev["w_router"]
    moe.moe_decode_layer(dev["x"], wr, dev["bias"], cfg.k, cfg.E, cfg.lo, cfg.hi, dev["w_gate_up"], dev["w_down"],
                         dev["s_gate_up"], dev["s_down"], ws, ids, w, out, y, router_packed=router == "packed",
                         packed=packed)
    torch.cuda.synchronize()
    return out, ids, w, y, R_cap


def check_workspace_clean(ws, El):
    ctl = ws[:4 * (CTL_WORDS + El)].view(torch.int32).cpu().numpy()
    assert ctl[4] == 0, f"a wait inside the kernel gave up (error bits {ctl[4]:#x})"
    assert not ctl[:4].any() and not ctl[CTL_WORDS:].any(), "control words not reset"


def check_h(h, h_ref, same_kernel):
    """h against moe_grouped_ffn's.  With few rows per expert moe_grouped_ffn runs the weight-streaming
    kernel, whose per-row MFMA sequence the one-launch kernel shares: bit for bit.  With many it runs
    the tile kernel, which sums the contraction in another order: the fp32 G and U differ in their
    last bits, so a bf16 h may round the other way (one bf16 step), and where G or U cancel the
    absolute fp32 noise can move a small h by more; checked: few values differ, each within one bf16
    step of the larger magnitude or 1e-3 of h's RMS."""
    if same_kernel:
        assert torch.equal(h, h_ref)
        return
    a = (h.int().cpu().numpy().astype(np.uint32) & 0xFFFF) << 16
    b = (h_ref.int().cpu().numpy().astype(np.uint32) & 0xFFFF) << 16
    fa, fb = a.view(np.float32).astype(np.float64), b.view(np.float32).astype(np.float64)
    diff = fa != fb
    bound = np.maximum(2.0 ** -7 * np.maximum(np.abs(fa), np.abs(fb)), 1e-3 * np.sqrt(np.mean(fb ** 2)))
    say(f"  h: {int(diff.sum())} of {diff.size} bf16 values differ (tile kernel sums in another order), largest "
        f"difference {np.max(np.abs(fa - fb) / bound):.3f} x the bound")
    assert diff.mean() < 0.01 and np.all(np.abs(fa - fb) <= bound)


def h_rows(ws, cfg, perm):
    """The dense h [E_loc, T, I] of the workspace, gathered to the grouped rows (expert, token of row)."""
    El, T, I = cfg.E_loc, cfg.T, cfg.I
    off = -(-4 * (CTL_WORDS + El) // 256) * 256
    h = ws[off:off + 2 * El * T * I].view(torch.int16).view(El * T, I)
    counts = perm["counts"].long()
    R = int(counts.sum())
    expert = torch.repeat_interleave(torch.arange(El, device=h.device), counts)
    return h[expert * T + perm["row_token"][:R].long()]


CASES = [
    CONFIGS["decode"],
    LayerConfig("dl_t1", T=1, H=256, E=16, k=4, I=128, seed=701),
    LayerConfig("dl_t32", T=32, H=512, E=32, k=4, I=192, seed=702, w_std=0.05),      # one 32-row block
    LayerConfig("dl_t33", T=33, H=512, E=8, k=2, I=256, seed=703, w_std=0.05),       # two blocks, ragged
    LayerConfig("dl_local", T=64, H=512, E=40, k=6, I=128, e_begin=5, e_end=29, seed=704, w_std=0.05),
    LayerConfig("dl_e200", T=48, H=256, E=200, k=8, I=64, seed=705, w_std=0.05),     # four router waves
    LayerConfig("dl_e21", T=50, H=320, E=21, k=5, I=320, seed=706, w_std=0.05),      # H, I not multiples of 128
    LayerConfig("dl_zipf", T=64, H=256, E=64, k=8, I=128, bias="zipf", seed=707, w_std=0.05),  # hot experts
    # every token on 4 of 4 experts (64 rows each: a full tile in the down projection)
    LayerConfig("dl_k_eq_e", T=64, H=256, E=4, k=4, I=128, seed=708, w_std=0.05),
    LayerConfig("dl_fp8", T=64, H=512, E=16, k=4, I=256, wdt="fp8", seed=710),
    LayerConfig("dl_fp8_local", T=60, H=256, E=32, k=8, I=128, wdt="fp8", e_begin=0, e_end=8, seed=711),
]
VARIANTS = [("as-stored", False), ("packed", True)]


@pytest.mark.parametrize("router,packed", VARIANTS, ids=["stored", "packed"])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_decode_layer_matches_four_calls_and_oracle(cfg, router, packed):
    inp = synth.make_inputs(cfg)
    dev = L.to_device(inp)
    if packed:
        L.pack_weights(dev)
    if router == "packed":
        L.pack_router(dev)
    El = cfg.E_loc
    ws = moe.moe_decode_layer_workspace(cfg.T, cfg.k, El, cfg.I)
    say(f"decode layer {cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} local [{cfg.lo},{cfg.hi}) "
        f"w={cfg.wdt} router={router} packed={packed}")
    # the four-call path on the same device inputs
    ids_r, w_r = moe.moe_route(dev["x"], dev["w_router"], dev["bias"], cfg.k)
    p_r = moe.moe_permute(ids_r, w_r, cfg.E, cfg.lo, cfg.hi)
    ffn_ws = torch.empty(moe.moe_ffn_workspace_size(p_r["R_cap"], El, cfg.H, cfg.I, moe.MOE_BF16), dtype=torch.uint8,
                         device="cuda")
    y_r = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(dev["x"], p_r["offsets"], p_r["row_token"], p_r["row_w"], cfg.T, p_r["R_cap"],
                        dev["w_gate_up"], dev["w_down"], dev["s_gate_up"], dev["s_down"], y=y_r, workspace=ffn_ws,
                        packed=packed)
    torch.cuda.synchronize()
    R = int(p_r["offsets"][-1])
    y_o = O.layer_tokens(np.arange(cfg.T, dtype=np.int32), inp["x"], ids_r.cpu().numpy(), w_r.cpu().numpy(), cfg.lo,
                         cfg.hi, inp["w_gate_up"], inp["w_down"], inp["s_gate_up"], inp["s_down"])
    for call in range(3):  # the control words must come back to zero after every call
        out, ids, w, y, R_cap = run_decode(dev, cfg, ws, router, packed)
        assert torch.equal(ids, ids_r) and torch.equal(w.view(torch.int32), w_r.view(torch.int32))
        for key in ("counts", "offsets"):
            assert torch.equal(out[key], p_r[key]), key
        assert torch.equal(out["row_token"][:R], p_r["row_token"][:R])
        assert torch.equal(out["row_w"][:R].view(torch.int32), p_r["row_w"][:R].view(torch.int32))
        assert torch.equal(out["token_row"], p_r["token_row"])
        check_h(h_rows(ws, cfg, p_r), ffn_ws[:2 * R * cfg.I].view(torch.int16).view(R, cfg.I),
                same_kernel=p_r["R_cap"] <= 48 * El)
        check_workspace_clean(ws, El)
        check_close(y.cpu().numpy(), y_o, f"{cfg.name} call {call} vs oracle")
        check_close(y.cpu().numpy(), y_r.cpu().numpy(), f"{cfg.name} call {call} vs moe_grouped_ffn")


def test_decode_layer_then_smaller_batch_same_workspace():
    # one workspace sized for the larger batch serves a smaller one next (fewer experts, fewer tokens)
    big = LayerConfig("dl_big", T=64, H=256, E=32, k=4, I=128, seed=712, w_std=0.05)
    small = LayerConfig("dl_small", T=5, H=256, E=32, k=4, I=128, e_begin=3, e_end=17, seed=713, w_std=0.05)
    ws = moe.moe_decode_layer_workspace(big.T, big.k, big.E_loc, big.I)
    for cfg in (big, small, big):
        inp = synth.make_inputs(cfg)
        dev = L.to_device(inp)
        out, ids, w, y, _ = run_decode(dev, cfg, ws)
        ids_o, w_o, _ = O.route(inp["x"], inp["w_router"], inp["bias"], cfg.k)
        assert np.array_equal(ids.cpu().numpy(), ids_o)
        y_o = O.layer_tokens(np.arange(cfg.T, dtype=np.int32), inp["x"], ids_o, w_o, cfg.lo, cfg.hi, inp["w_gate_up"],
                             inp["w_down"], inp["s_gate_up"], inp["s_down"])
        check_close(y.cpu().numpy(), y_o, cfg.name)
        check_workspace_clean(ws, big.E_loc)


def test_decode_layer_empty_batch_zeroes_counts():
    cfg = LayerConfig("dl_empty", T=0, H=256, E=16, k=4, I=128, seed=714)
    ws = moe.moe_decode_layer_workspace(1, cfg.k, cfg.E_loc, cfg.I)
    out, ids, w, y, _ = decode_buffers(cfg)
    x = torch.zeros((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((cfg.E, cfg.H), dtype=torch.bfloat16, device="cuda")
    wgu = torch.zeros((cfg.E, 2 * cfg.I, cfg.H), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((cfg.E, cfg.H, cfg.I), dtype=torch.bfloat16, device="cuda")
    moe.moe_decode_layer(x, wr, None, cfg.k, cfg.E, 0, cfg.E, wgu, wd, None, None, ws, ids, w, out, y)
    torch.cuda.synchronize()
    assert torch.all(out["counts"] == 0) and torch.all(out["offsets"] == 0)


@pytest.mark.parametrize("packed", [False, True], ids=["stored", "packed"])
def test_decode_layer_graph_replay(packed):
    # the layer captured once in a HIP graph (one kernel, no memset: the workspace comes back zero by
    # itself) and replayed with eager work in between; every replay against the oracle
    cfg = LayerConfig("dl_graph", T=64, H=512, E=32, k=4, I=256, seed=715, w_std=0.05)
    inp = synth.make_inputs(cfg)
    dev = L.to_device(inp)
    if packed:
        L.pack_weights(dev)
        L.pack_router(dev)
    bufs = L.LayerBuffers(cfg, fused=True, use_decode_layer=True)
    assert bufs.dec_ws is not None
    r = O.layer(inp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L.run_layer(dev, bufs, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        L.run_layer(dev, bufs, stream=s)
    for rep in range(4):
        bufs.y.fill_(float("nan"))
        bufs.topk_ids.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bufs.topk_ids.cpu().numpy(), r["topk_ids"]), f"replay {rep}"
        check_close(bufs.y.cpu().numpy(), r["y"], f"graph replay {rep} packed={packed}")
        check_workspace_clean(bufs.dec_ws, cfg.E_loc)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        del junk
