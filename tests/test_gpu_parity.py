"""GPU parity: every entry point of the HIP library against the CPU oracle.

Routing ids, counts, offsets, the permutation and x_perm must match bit for
bit; gates within 1e-6; layer outputs within max|err| <= 1e-2 * RMS(oracle).
Small shapes and the full workload shapes (decode, prefill, skewed prefill, EP
share, MXFP8, shared expert), the latter in the launch configuration the
benchmark times, are compared element by element on every token.
"""
import functools
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from expert_routed_grouped_amd import layer as L
from expert_routed_grouped_amd import moe, synth
from expert_routed_grouped_amd.synth import CONFIGS, LayerConfig, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

GATE_TOL = 1e-6
Y_TOL = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=None)
def host_inputs(cfg: LayerConfig):
    return synth.make_inputs(cfg)


@functools.lru_cache(maxsize=None)
def oracle_routing(cfg: LayerConfig):
    inp = host_inputs(cfg)
    ids, w, _ = O.route(inp["x"], inp["w_router"], inp["bias"], cfg.k)
    return ids, w


def check_y(y_gpu, y_ref, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    err = np.max(np.abs(y_gpu - y_ref)) if y_ref.size else 0.0
    say(f"  {what} max|err| = {err:.3e}, RMS = {rms:.3e}, ratio = {err / max(rms, 1e-30):.2e}")
    assert rms > 0
    assert err <= Y_TOL * rms


def gpu_route(dev, cfg):
    ids, w = moe.moe_route(dev["x"], dev["w_router"], dev["bias"], cfg.k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def to_dev_routing(ids, w):
    return torch.from_numpy(np.ascontiguousarray(ids)).cuda(), torch.from_numpy(np.ascontiguousarray(w)).cuda()


def gpu_layer(dev, cfg, ids_d, w_d, fused: bool, gather: bool = True):
    """The four calls on the given routing; returns (y, perm dict)."""
    x = dev["x"]
    p = moe.moe_permute(ids_d, w_d, cfg.E, cfg.lo, cfg.hi, x=None if gather else x)
    R_cap = p["R_cap"]
    a = x if gather else p["x_perm"]
    y = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    if fused:
        y.fill_(float("nan"))  # MOE_FFN_ZERO_Y must clear it
        moe.moe_grouped_ffn(a, p["offsets"], p["row_token"], p["row_w"], cfg.T, R_cap, dev["w_gate_up"],
                            dev["w_down"], dev["s_gate_up"], dev["s_down"], y=y, gather=gather, zero_y=True)
    else:
        yp = torch.empty((max(R_cap, 1), cfg.H), dtype=torch.float32, device="cuda")
        moe.moe_grouped_ffn(a, p["offsets"], p["row_token"], p["row_w"], cfg.T, R_cap, dev["w_gate_up"],
                            dev["w_down"], dev["s_gate_up"], dev["s_down"], y_perm=yp, gather=gather)
        moe.moe_combine(yp, p["token_row"], w_d, y=y)
    torch.cuda.synchronize()
    return y.cpu().numpy(), p


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
ROUTE_CASES = [
    CONFIGS["tiny"], CONFIGS["decode"], CONFIGS["prefill"], CONFIGS["skew"], CONFIGS["ep_share"],
    LayerConfig("r_f32_oddH", T=37, H=203, E=5, k=3, I=64, act="f32", wdt="f32", init="fan_in", seed=101),
    LayerConfig("r_E200", T=600, H=512, E=200, k=8, I=64, seed=102),
    LayerConfig("r_E512_k32", T=70, H=256, E=512, k=32, I=64, seed=103, w_std=0.05),
    LayerConfig("r_kE", T=64, H=128, E=16, k=16, I=64, seed=104),
    LayerConfig("r_k1", T=513, H=64, E=64, k=1, I=64, seed=105),
    # 16 tokens per workgroup (at least 512 workgroups), the last one partly empty
    LayerConfig("r_tr4_ragged", T=8195, H=256, E=128, k=8, I=64, seed=106, w_std=0.05),
    # up to 1024 experts: 16 router waves, one and four tokens per workgroup
    LayerConfig("r_E1024", T=70, H=256, E=1024, k=8, I=64, seed=107, w_std=0.05),
    LayerConfig("r_E1000_t600", T=600, H=192, E=1000, k=32, I=64, seed=108, w_std=0.05),
]


@pytest.mark.parametrize("cfg", ROUTE_CASES, ids=lambda c: c.name)
def test_route_matches_oracle(cfg):
    inp = synth.make_inputs(cfg, with_weights=False)
    dev = L.to_device(inp)
    say(f"route {cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    ids, w = gpu_route(dev, cfg)
    ids_o, w_o, _ = O.route(inp["x"], inp["w_router"], inp["bias"], cfg.k)
    assert np.array_equal(ids, ids_o)
    assert np.max(np.abs(w - w_o)) <= GATE_TOL
    # deterministic: a second run gives the same bits
    ids2, w2 = gpu_route(dev, cfg)
    assert np.array_equal(ids2, ids) and np.array_equal(w2.view(np.uint32), w.view(np.uint32))


def test_route_ties_and_zero_router():
    cfg = LayerConfig("ties", T=300, H=256, E=128, k=8, I=64, seed=106)
    inp = synth.make_inputs(cfg, with_weights=False)
    wr = inp["w_router"].copy()
    wr[7] = wr[3]
    wr[100] = wr[3]
    wr[64] = wr[0]
    for w_router in (wr, np.zeros_like(wr)):
        dev = L.to_device(dict(inp, w_router=w_router))
        ids, w = gpu_route(dev, cfg)
        ids_o, w_o, _ = O.route(inp["x"], w_router, None, cfg.k)
        assert np.array_equal(ids, ids_o)
        assert np.max(np.abs(w - w_o)) <= GATE_TOL
    assert np.all(ids == np.arange(8)) and np.all(w == np.float32(0.125))



@pytest.mark.parametrize("T,path", [(40, "route"), (300, "route"), (8200, "route"), (40, "dispatch"),
                                    (300, "dispatch")])
def test_route_ties_every_path(T, path):
    """Exact ties (duplicated router rows, within one 64-expert half and across halves, one of three)
    go to the lower expert index on every router path: one token per workgroup (T <= 256), the
    LDS-staged kernel with 12 and 16 tokens per workgroup, and route + dispatch."""
    cfg = LayerConfig(f"ties{T}", T=T, H=256, E=128, k=8, I=64, seed=108)
    inp = synth.make_inputs(cfg, with_weights=False)
    wr = inp["w_router"].copy()
    wr[7] = wr[3]
    wr[100] = wr[3]
    wr[64] = wr[0]
    wr[127] = wr[126]
    dev = L.to_device(dict(inp, w_router=wr))
    say(f"route ties T={T} via {path}")
    ids_o, w_o, _ = O.route(inp["x"], wr, None, cfg.k)
    if path == "route":
        ids, w = gpu_route(dev, cfg)
    else:
        ws = moe.moe_route_dispatch_workspace()
        out = dict(counts=torch.empty((cfg.E,), dtype=torch.int32, device="cuda"),
                   offsets=torch.empty((cfg.E + 1,), dtype=torch.int32, device="cuda"),
                   row_token=torch.empty((T * cfg.k,), dtype=torch.int32, device="cuda"),
                   row_w=torch.empty((T * cfg.k,), dtype=torch.float32, device="cuda"),
                   token_row=torch.empty((T, cfg.k), dtype=torch.int32, device="cuda"))
        ids_d = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
        w_d = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
        moe.moe_route_dispatch(dev["x"], dev["w_router"], None, cfg.k, cfg.E, 0, cfg.E, ws, ids_d, w_d, out)
        torch.cuda.synchronize()
        ids, w = ids_d.cpu().numpy(), w_d.cpu().numpy()
        p_o = O.permute(ids_o, w_o, 0, cfg.E)
        assert np.array_equal(out["offsets"].cpu().numpy(), p_o["offsets"])
        assert np.array_equal(out["row_token"].cpu().numpy()[:p_o["R"]], p_o["row_token"])
    assert np.array_equal(ids, ids_o)
    assert np.max(np.abs(w - w_o)) <= GATE_TOL
    # the ties really occur: some token selects both members of a duplicated pair, lower index first
    both = [(a, b) for a, b in ((3, 7), (3, 100), (0, 64), (126, 127))
            if np.any(np.isin(ids_o, a).any(1) & np.isin(ids_o, b).any(1))]
    assert both, "no token selected a tied pair"
    for a, b in both:
        rows = np.nonzero(np.isin(ids_o, a).any(1) & np.isin(ids_o, b).any(1))[0]
        pa = np.argmax(ids_o[rows] == a, axis=1)
        pb = np.argmax(ids_o[rows] == b, axis=1)
        assert np.all(pa < pb)


def test_route_empty_batch():
    cfg = LayerConfig("empty", T=0, H=64, E=8, k=2, I=64, seed=107)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    ids, w = moe.moe_route(x, wr, None, 2)
    assert ids.shape == (0, 2)


# ----------------------------------------------------------------------------
# permutation
# ----------------------------------------------------------------------------
def check_permutation(p_gpu, p_or, T, k, x=None, same_gates=True):
    """Integer outputs bit for bit.  row_w is a copy of the gates given to moe_permute:
    bit for bit when those were the oracle's, else within the gate tolerance."""
    R = p_or["R"]
    assert np.array_equal(p_gpu["counts"].cpu().numpy(), p_or["counts"])
    assert np.array_equal(p_gpu["offsets"].cpu().numpy(), p_or["offsets"])
    assert np.array_equal(p_gpu["row_token"][:R].cpu().numpy(), p_or["row_token"])
    rw = p_gpu["row_w"][:R].cpu().numpy()
    if same_gates:
        assert np.array_equal(rw.view(np.uint32), p_or["row_w"].view(np.uint32))
    else:
        assert np.max(np.abs(rw - p_or["row_w"]), initial=0.0) <= GATE_TOL
    assert np.array_equal(p_gpu["token_row"].cpu().numpy(), p_or["token_row"])
    if x is not None:
        xp = p_gpu["x_perm"][:R].cpu()
        ref = x[p_or["row_token"]]
        assert np.array_equal(xp.view(torch.int16).numpy().view(np.uint16) if xp.dtype == torch.bfloat16 else xp.numpy(),
                              ref)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skew", "ep_share"])
def test_permute_matches_oracle(name):
    cfg = CONFIGS[name]
    ids, w = oracle_routing(cfg)
    inp = host_inputs(cfg)
    say(f"permute {name}: T={cfg.T} k={cfg.k} local=[{cfg.lo},{cfg.hi})")
    ids_d, w_d = to_dev_routing(ids, w)
    xd = L.to_device({"cfg": cfg, "x": inp["x"], "w_router": inp["w_router"]})["x"]
    p = moe.moe_permute(ids_d, w_d, cfg.E, cfg.lo, cfg.hi, x=xd)
    torch.cuda.synchronize()
    check_permutation(p, O.permute(ids, w, cfg.lo, cfg.hi), cfg.T, cfg.k, x=inp["x"])
    counts = p["counts"].cpu().numpy()
    if cfg.E_loc == cfg.E:
        assert counts.sum() == cfg.T * cfg.k
    if name == "prefill":
        assert counts.mean() == 375  # 6000 * 8 / 128


def routing_case(kind):
    rng = np.random.default_rng(sum(map(ord, kind)))
    if kind == "one_hot_experts":      # every token picks experts 0..k-1
        T, E, k = 1000, 64, 4
        ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    elif kind == "k_equals_E":
        T, E, k = 300, 8, 8
        ids = np.argsort(rng.random((T, E)), axis=1).astype(np.int32)
    elif kind == "max_experts":
        T, E, k = 2000, 512, 8
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    elif kind == "ragged":
        T, E, k = 333, 128, 7
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    elif kind == "many_tokens":
        T, E, k = 20000, 128, 8
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    else:
        raise ValueError(kind)
    w = rng.random(ids.shape).astype(np.float32)
    return ids, w, E


@pytest.mark.parametrize("kind,lo,hi", [("one_hot_experts", 0, 64), ("one_hot_experts", 2, 3), ("k_equals_E", 0, 8),
                                        ("k_equals_E", 5, 8), ("max_experts", 0, 512), ("max_experts", 100, 356),
                                        ("ragged", 0, 128), ("ragged", 127, 128), ("many_tokens", 0, 128),
                                        ("many_tokens", 32, 64)])
def test_permute_edge_cases(kind, lo, hi):
    ids, w, E = routing_case(kind)
    ids_d, w_d = to_dev_routing(ids, w)
    p = moe.moe_permute(ids_d, w_d, E, lo, hi)
    torch.cuda.synchronize()
    check_permutation(p, O.permute(ids, w, lo, hi), *ids.shape)


def test_permute_empty_batch():
    ids_d = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w_d = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    p = moe.moe_permute(ids_d, w_d, 8, 0, 8)
    torch.cuda.synchronize()
    assert p["counts"].cpu().tolist() == [0] * 8 and p["offsets"].cpu().tolist() == [0] * 9


# ----------------------------------------------------------------------------
# expert FFN + combine, every token against the oracle
# ----------------------------------------------------------------------------
FFN_CASES = [
    # several 128-row tiles per expert with ragged tails; 64-col ragged N tail in the down projection
    LayerConfig("ffn_bf16", T=700, H=320, E=4, k=2, I=192, seed=201, w_std=0.05),
    LayerConfig("ffn_fp8_local", T=700, H=320, E=6, k=3, I=192, wdt="fp8", e_begin=1, e_end=4, seed=202, w_std=0.05),
    # e4m3 tiles with one K step in both halves (H = I = 64: the shortest pipeline, a 64-wide N tail),
    # and one expert of 300 rows over three K steps (two unequal M tiles)
    LayerConfig("ffn_fp8_k64", T=600, H=64, E=4, k=2, I=64, wdt="fp8", seed=211, w_std=0.05),
    LayerConfig("ffn_fp8_single", T=300, H=192, E=1, k=1, I=128, wdt="fp8", seed=212, w_std=0.05),
    LayerConfig("ffn_skew_empty", T=500, H=256, E=32, k=4, I=128, bias="zipf", seed=203, w_std=0.05),
    LayerConfig("ffn_k_eq_E", T=130, H=128, E=4, k=4, I=64, seed=204, w_std=0.05),
    LayerConfig("ffn_single_expert", T=257, H=192, E=1, k=1, I=128, seed=205, w_std=0.05),
    CONFIGS["tiny"],
    LayerConfig("ffn_f32_local", T=200, H=128, E=8, k=2, I=64, act="f32", wdt="f32", e_begin=2, e_end=6,
                init="fan_in", seed=206),
    # few rows per expert: the weight-streaming kernels (column tails in both halves)
    LayerConfig("stream_bf16", T=64, H=320, E=32, k=4, I=192, seed=207, w_std=0.05),
    LayerConfig("stream_fp8_local", T=48, H=256, E=16, k=4, I=128, wdt="fp8", e_begin=4, e_end=12, seed=208,
                w_std=0.05),
    # one hot expert with more than 64 rows: several 64-row tiles and both 32-row blocks
    LayerConfig("stream_hot", T=120, H=256, E=16, k=2, I=128, bias="zipf", seed=209, w_std=0.05),
    # many experts: 1000 routed, 600 of them local (mostly empty experts, a few rows each)
    LayerConfig("many_experts", T=300, H=128, E=1000, k=8, I=64, e_begin=200, e_end=800, seed=210, w_std=0.05),
    # one token; two tokens whose only local assignment is expert 2 (the other slots dropped)
    LayerConfig("ffn_t1", T=1, H=128, E=8, k=3, I=64, seed=213, w_std=0.05),
    LayerConfig("ffn_t2_local", T=2, H=128, E=8, k=2, I=64, e_begin=2, e_end=3, seed=214, w_std=0.05),
]


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "combine"])
@pytest.mark.parametrize("cfg", FFN_CASES, ids=lambda c: c.name)
def test_layer_all_tokens_matches_oracle(cfg, fused):
    inp = host_inputs(cfg)
    dev = L.to_device(inp)
    say(f"layer {cfg.name} fused={fused}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} w={cfg.wdt}")
    ids, w = oracle_routing(cfg)
    ids_g, w_g = gpu_route(dev, cfg)
    assert np.array_equal(ids_g, ids)
    ids_d, w_d = to_dev_routing(ids_g, w_g)
    y, p = gpu_layer(dev, cfg, ids_d, w_d, fused=fused)
    y_o = O.layer_tokens(np.arange(cfg.T), inp["x"], ids, w, cfg.lo, cfg.hi, inp["w_gate_up"], inp["w_down"],
                         inp["s_gate_up"], inp["s_down"], round_h=cfg.act != "f32")
    check_y(y, y_o, cfg.name)
    if cfg.E_loc < cfg.E:
        no_local = ~np.any((ids >= cfg.lo) & (ids < cfg.hi), axis=1)
        assert np.all(y[no_local] == 0)


# Per-expert row counts around the tile sizes of the large-batch kernels (64-row and 256-row
# boundaries, one empty expert): each expert's rows are split into equal M tiles.
TILE_COUNTS = [1, 63, 64, 65, 255, 256, 257, 511, 512, 513, 0, 999, 752, 752]


def constructed_routing(counts, T, k, seed):
    """ids [T,k] with exactly counts[e] assignments of expert e and k distinct experts per token:
    the expert-sorted assignment list is dealt out with stride T (every run is shorter than T)."""
    assert sum(counts) == T * k and max(counts) < T
    flat = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    ids = np.ascontiguousarray(flat.reshape(k, T).T)
    assert all(len(set(r)) == k for r in ids.tolist())
    w = np.random.default_rng(seed).random((T, k)).astype(np.float32)
    return ids, w


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "combine"])
@pytest.mark.parametrize("wdt", ["bf16", "fp8"])
def test_layer_tile_boundaries(wdt, fused):
    cfg = LayerConfig(f"tiles_{wdt}", T=1000, H=320, E=len(TILE_COUNTS), k=5, I=192, wdt=wdt, seed=210,
                      w_std=0.05)
    inp = host_inputs(cfg)
    dev = L.to_device(inp)
    ids, w = constructed_routing(TILE_COUNTS, cfg.T, cfg.k, seed=211)
    say(f"layer {cfg.name} fused={fused}: counts {TILE_COUNTS}")
    ids_d, w_d = to_dev_routing(ids, w)
    y, p = gpu_layer(dev, cfg, ids_d, w_d, fused=fused)
    assert p["counts"].cpu().tolist() == TILE_COUNTS
    y_o = O.layer_tokens(np.arange(cfg.T), inp["x"], ids, w, cfg.lo, cfg.hi, inp["w_gate_up"], inp["w_down"],
                         inp["s_gate_up"], inp["s_down"], round_h=True)
    check_y(y, y_o, cfg.name)


@pytest.mark.parametrize("cfg", [FFN_CASES[0], FFN_CASES[1]], ids=lambda c: c.name)
def test_layer_with_materialised_x_perm(cfg):
    """gather=False: the FFN reads x_perm written by moe_permute instead of gathering x."""
    inp = host_inputs(cfg)
    dev = L.to_device(inp)
    ids, w = oracle_routing(cfg)
    ids_d, w_d = to_dev_routing(ids, w)
    y, _ = gpu_layer(dev, cfg, ids_d, w_d, fused=False, gather=False)
    y_o = O.layer_tokens(np.arange(cfg.T), inp["x"], ids, w, cfg.lo, cfg.hi, inp["w_gate_up"], inp["w_down"],
                         inp["s_gate_up"], inp["s_down"])
    check_y(y, y_o, cfg.name + " x_perm")


def test_combine_matches_oracle_and_is_deterministic():
    rng = np.random.default_rng(5)
    ids, w, E = routing_case("ragged")
    p = O.permute(ids, w, 10, 90)
    yp = rng.standard_normal((max(p["R"], 1), 256)).astype(np.float32)
    y_o = O.combine(yp, p["token_row"], w)
    yp_d = torch.from_numpy(yp).cuda()
    tr_d = torch.from_numpy(p["token_row"]).cuda()
    w_d = torch.from_numpy(w).cuda()
    y1 = moe.moe_combine(yp_d, tr_d, w_d).cpu().numpy()
    y2 = moe.moe_combine(yp_d, tr_d, w_d).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.max(np.abs(y1 - y_o)) <= 1e-6 * np.max(np.abs(y_o))


def test_ffn_empty_batch_zeroes_y():
    cfg = LayerConfig("e", T=4, H=64, E=2, k=1, I=64, seed=1)
    y = torch.full((4, 64), 3.0, device="cuda")
    off = torch.zeros(3, dtype=torch.int32, device="cuda")
    rt = torch.zeros(1, dtype=torch.int32, device="cuda")
    rw = torch.zeros(1, dtype=torch.float32, device="cuda")
    wgu = torch.zeros((2, 128, 64), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_ffn(x, off, rt, rw, 4, 4, wgu, wd, y=y, zero_y=True)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


# ----------------------------------------------------------------------------
# the decode layer under HIP graph capture: every replay against the oracle
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "combine"])
@pytest.mark.parametrize("packed", [False, True], ids=["stored", "packed"])
def test_layer_graph_replay_matches_oracle(fused, packed):
    # every step of the layer is a kernel of the library (zeroing included), so the whole call
    # can be captured once and replayed; eager work runs between the replays.  ``packed``: the
    # expert weights and the router weight in their packed layouts (the benchmark's configuration)
    cfg = LayerConfig("graph", T=64, H=512, E=32, k=4, I=256, seed=601, w_std=0.05)
    inp = host_inputs(cfg)
    dev = L.to_device(inp)
    if packed:
        L.pack_weights(dev)
        L.pack_router(dev)
        assert dev.get("packed") and dev.get("w_router_packed") is not None
    bufs = L.LayerBuffers(cfg, fused=fused)
    r = O.layer(inp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L.run_layer(dev, bufs, stream=s)  # warm-up outside the capture
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
        check_y(bufs.y.cpu().numpy(), r["y"], f"graph replay {rep} fused={fused} packed={packed}")
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between the replays
        torch.cuda.synchronize()
        del junk


@pytest.mark.parametrize("packed", [False, True], ids=["stored", "packed"])
def test_layer_graph_replay_shared_beside_router(packed):
    """A decode batch with a shared expert: the shared expert (which zeroes y) runs on a second stream
    beside the router and the routed down projection waits for it.  Eager, and captured in one graph
    (the second stream forks from and joins the capturing stream), every replay against the oracle."""
    cfg = LayerConfig("graph_shared", T=64, H=512, E=32, k=4, I=256, seed=602, w_std=0.05, I_s=256)
    inp = host_inputs(cfg)
    dev = L.to_device(inp)
    if packed:
        L.pack_weights(dev)
        L.pack_router(dev)
    bufs = L.LayerBuffers(cfg, fused=True)
    assert bufs.side is not None, "a decode batch with a shared expert runs it beside the router"
    r = O.layer(inp)
    r["y"] = r["y"].astype(np.float64) + O.shared_tokens(np.arange(cfg.T), inp["x"], inp["ws_gate_up"],
                                                         inp["ws_down"], inp["ss_gate_up"], inp["ss_down"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L.run_layer(dev, bufs, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    check_y(bufs.y.cpu().numpy(), r["y"], f"eager, shared beside the router, packed={packed}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        L.run_layer(dev, bufs, stream=s)
    for rep in range(4):
        bufs.y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bufs.topk_ids.cpu().numpy(), r["topk_ids"]), f"replay {rep}"
        check_y(bufs.y.cpu().numpy(), r["y"], f"graph replay {rep}, shared beside the router, packed={packed}")
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between the replays
        torch.cuda.synchronize()
        del junk


# ----------------------------------------------------------------------------
# full workload shapes, benchmark launch configuration, every output row
# ----------------------------------------------------------------------------
@functools.lru_cache(maxsize=None)
def oracle_full_y(name):
    """The oracle's y for every token of a full workload (token-major, all host cores), computed
    once per workload and shared by the row-major and packed-weight runs."""
    cfg = CONFIGS[name]
    inp = host_inputs(cfg)
    ids, w = oracle_routing(cfg)
    toks = np.arange(cfg.T, dtype=np.int32)
    say(f"full layer {name}: oracle on all {cfg.T} tokens ({O.num_threads()} threads)")
    y = O.layer_tokens(toks, inp["x"], ids, w, cfg.lo, cfg.hi, inp["w_gate_up"], inp["w_down"], inp["s_gate_up"],
                       inp["s_down"])
    if cfg.I_s > 0:
        y = (y.astype(np.float64) + O.shared_tokens(toks, inp["x"], inp["ws_gate_up"], inp["ws_down"],
                                                     inp["ss_gate_up"], inp["ss_down"])).astype(np.float32)
    return y


FULL_CASES = [(n, False, True) for n in ["decode", "prefill", "skew", "ep_share", "decode_shared", "prefill_shared"]]
FULL_CASES += [(n, True, True) for n in ["decode", "prefill", "skew", "ep_share", "decode_shared", "prefill_shared"]]
# the decode workloads also through the four-call path (route + dispatch launch, grouped FFN)
FULL_CASES += [(n, p, False) for n in ["decode", "decode_shared"] for p in (False, True)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,packed,one_launch", FULL_CASES,
                         ids=[f"{n}{'_packed' if p else ''}{'' if o else '_4calls'}" for n, p, o in FULL_CASES])
def test_full_workload_layer(name, packed, one_launch):
    """The layer as the benchmark launches it (same kernels, grid and tile walk), compared with the
    oracle on every one of the T x H outputs."""
    cfg = CONFIGS[name]
    inp = host_inputs(cfg)
    say(f"full layer {name}: generating / uploading")
    dev = L.to_device(inp)
    if packed:
        L.pack_weights(dev)
    bufs = L.LayerBuffers(cfg, use_decode_layer=one_launch)
    if (bufs.rd_ws is not None or bufs.dec_ws is not None) and packed:
        L.pack_router(dev)
    say(f"full layer {name}: run_layer fused={bufs.fused} R_cap={bufs.R_cap} packed={packed} "
        f"one_launch={bufs.dec_ws is not None}")
    y = L.run_layer(dev, bufs)
    torch.cuda.synchronize()
    ids, w = oracle_routing(cfg)
    assert np.array_equal(bufs.topk_ids.cpu().numpy(), ids)
    assert np.max(np.abs(bufs.topk_w.cpu().numpy() - w)) <= GATE_TOL
    p_or = O.permute(ids, w, cfg.lo, cfg.hi)
    check_permutation(bufs.perm, p_or, cfg.T, cfg.k, same_gates=False)
    y_o = oracle_full_y(name)
    yg = y.cpu().numpy()
    say(f"full layer {name}: comparing all {cfg.T} rows x {cfg.H} columns")
    check_y(yg, y_o, name)
    # a second call reuses the buffers and gives the same routing and (up to atomic order) the same y
    y2 = L.run_layer(dev, bufs).cpu().numpy()
    check_y(y2, y_o, name + " (repeat)")
    del dev, bufs
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# the largest batch the grouped FFN accepts at the workload's H and I
# ----------------------------------------------------------------------------
# R_cap * H = 262136 * 4096 is 32768 elements short of 2^30, the grouped FFN's limit: the per-row
# fp32 outputs end 128 KiB below 4 GiB, h takes 805 MB, so the tile kernels' 32-bit buffer offsets
# and the combine's reads run at the top of their range.
MAX_CFG = LayerConfig("max_rows", T=32767, H=4096, E=128, k=8, I=1536, seed=10)


@pytest.mark.timeout(900)
def test_layer_at_the_size_limit():
    """The layer at the largest T the grouped FFN takes (packed weights, per-row outputs + combine,
    as at prefill): routing and the permutation in full, y on every token that owns one of the
    highest 256 rows of the per-row outputs, the first and last 16 tokens and 64 others."""
    cfg = MAX_CFG
    assert cfg.R_cap * cfg.H < (1 << 30) <= (cfg.T + 1) * cfg.k * cfg.H
    say(f"size limit: generating T={cfg.T} (R_cap={cfg.R_cap})")
    inp = synth.make_inputs(cfg)
    dev = L.to_device(inp)
    L.pack_weights(dev)
    bufs = L.LayerBuffers(cfg)
    assert not bufs.fused, "a batch this size writes per-row outputs and combines them"
    say(f"size limit: run_layer R_cap={bufs.R_cap}, per-row outputs {bufs.R_cap * cfg.H * 4} bytes")
    y = L.run_layer(dev, bufs)
    torch.cuda.synchronize()
    ids, w, _ = O.route(inp["x"], inp["w_router"], inp["bias"], cfg.k)
    assert np.array_equal(bufs.topk_ids.cpu().numpy(), ids)
    assert np.max(np.abs(bufs.topk_w.cpu().numpy() - w)) <= GATE_TOL
    p_or = O.permute(ids, w, cfg.lo, cfg.hi)
    check_permutation(bufs.perm, p_or, cfg.T, cfg.k, same_gates=False)
    R = p_or["R"]
    assert R == cfg.R_cap
    rng = np.random.default_rng(10)
    toks = set(p_or["row_token"][R - 256:].tolist()) | set(range(16)) | set(range(cfg.T - 16, cfg.T))
    toks |= set(rng.choice(cfg.T, 64, replace=False).tolist())
    toks = np.array(sorted(toks), dtype=np.int32)
    say(f"size limit: oracle on {toks.size} tokens")
    y_o = O.layer_tokens(toks, inp["x"], ids, w, cfg.lo, cfg.hi, inp["w_gate_up"], inp["w_down"], inp["s_gate_up"],
                         inp["s_down"])
    check_y(y.cpu().numpy()[toks], y_o, f"size limit, {toks.size} tokens")
    del dev, bufs, y, inp
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# decode route + dispatch in one launch: bit-identical to moe_route + moe_permute
# ----------------------------------------------------------------------------
RD_CASES = [
    CONFIGS["decode"],
    LayerConfig("rd_t1", T=1, H=256, E=16, k=4, I=64, seed=501),
    LayerConfig("rd_max", T=512, H=512, E=128, k=16, I=64, seed=502, w_std=0.05),     # T*k = 8192
    LayerConfig("rd_e256", T=100, H=256, E=256, k=8, I=64, seed=503, w_std=0.05),    # four waves per block
    LayerConfig("rd_e40_local", T=77, H=128, E=40, k=3, I=64, e_begin=5, e_end=30, seed=504),  # one wave
    LayerConfig("rd_f32", T=33, H=64, E=8, k=2, I=64, act="f32", wdt="f32", init="fan_in", seed=505),
    LayerConfig("rd_zipf", T=200, H=256, E=64, k=8, I=64, bias="zipf", seed=506, w_std=0.05),
    # ragged: H = 264 leaves 8 h after the whole rounds of the router's load ring; E, T odd sizes
    LayerConfig("rd_ragged", T=70, H=264, E=21, k=5, I=64, seed=507, w_std=0.05),
]


@pytest.mark.parametrize("cfg", RD_CASES, ids=lambda c: c.name)
def test_route_dispatch_matches_route_then_permute(cfg):
    inp = synth.make_inputs(cfg, with_weights=False)
    dev = L.to_device(inp)
    say(f"route+dispatch {cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} local [{cfg.lo},{cfg.hi})")
    ids, w = moe.moe_route(dev["x"], dev["w_router"], dev["bias"], cfg.k)
    p = moe.moe_permute(ids, w, cfg.E, cfg.lo, cfg.hi)
    torch.cuda.synchronize()
    ids_o, w_o, _ = O.route(inp["x"], inp["w_router"], inp["bias"], cfg.k)
    p_o = O.permute(ids_o, w_o, cfg.lo, cfg.hi)
    R = int(p_o["R"])
    ws = moe.moe_route_dispatch_workspace()
    El = cfg.hi - cfg.lo
    for rep in range(3):  # the ticket counter must come back to zero after every call
        out = dict(counts=torch.full((El,), -7, dtype=torch.int32, device="cuda"),
                   offsets=torch.full((El + 1,), -7, dtype=torch.int32, device="cuda"),
                   row_token=torch.full((max(p["R_cap"], 1),), -7, dtype=torch.int32, device="cuda"),
                   row_w=torch.full((max(p["R_cap"], 1),), -7.0, dtype=torch.float32, device="cuda"),
                   token_row=torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, device="cuda"))
        ids2 = torch.full_like(ids, -7)
        w2 = torch.full_like(w, -7.0)
        y = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_route_dispatch(dev["x"], dev["w_router"], dev["bias"], cfg.k, cfg.E, cfg.lo, cfg.hi, ws, ids2, w2,
                               out, y_zero=y)
        torch.cuda.synchronize()
        assert torch.equal(ids2, ids) and torch.equal(w2.view(torch.int32), w.view(torch.int32))
        assert np.array_equal(ids2.cpu().numpy(), ids_o)
        for key in ("counts", "offsets", "token_row"):
            assert torch.equal(out[key], p[key]), key
        assert torch.equal(out["row_token"][:R], p["row_token"][:R])
        assert torch.equal(out["row_w"][:R].view(torch.int32), p["row_w"][:R].view(torch.int32))
        assert np.array_equal(out["row_token"][:R].cpu().numpy(), p_o["row_token"])
        assert torch.all(y == 0)
        assert torch.all(ws == 0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_pack_router_layout(dt):
    """moe_pack_router: out[(j E + e) 4 + i] = w[e, 4j + i], exact fp32 values."""
    rng = np.random.default_rng(601)
    w = rng.standard_normal((21, 264), dtype=np.float32)
    wt = torch.from_numpy(w).cuda()
    if dt == "bf16":
        wt = wt.to(torch.bfloat16)
    out = moe.moe_pack_router(wt)
    torch.cuda.synchronize()
    ref = wt.float().cpu().numpy().reshape(21, 66, 4).transpose(1, 0, 2)
    assert out.shape == (66, 21, 4) and np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("cfg", RD_CASES, ids=lambda c: c.name)
def test_route_dispatch_packed_router_bit_identical(cfg):
    """moe_route_dispatch on the moe_pack_router layout gives the same routing, gates, grouping and
    zeroing as on the stored router weight (same chains on the same values)."""
    inp = synth.make_inputs(cfg, with_weights=False)
    dev = L.to_device(inp)
    say(f"route+dispatch packed router {cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    El = cfg.hi - cfg.lo
    R_cap = cfg.T * min(cfg.k, El)
    res = []
    for packed in (False, True):
        ws = moe.moe_route_dispatch_workspace()
        out = dict(counts=torch.full((El,), -7, dtype=torch.int32, device="cuda"),
                   offsets=torch.full((El + 1,), -7, dtype=torch.int32, device="cuda"),
                   row_token=torch.full((max(R_cap, 1),), -7, dtype=torch.int32, device="cuda"),
                   row_w=torch.full((max(R_cap, 1),), -7.0, dtype=torch.float32, device="cuda"),
                   token_row=torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, device="cuda"))
        ids = torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, device="cuda")
        w = torch.full((cfg.T, cfg.k), -7.0, dtype=torch.float32, device="cuda")
        y = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
        wr = moe.moe_pack_router(dev["w_router"]) if packed else dev["w_router"]
        moe.moe_route_dispatch(dev["x"], wr, dev["bias"], cfg.k, cfg.E, cfg.lo, cfg.hi, ws, ids, w, out, y_zero=y,
                               router_packed=packed)
        torch.cuda.synchronize()
        assert torch.all(y == 0) and torch.all(ws == 0)
        res.append((ids, w, out))
    (i0, w0, o0), (i1, w1, o1) = res
    assert torch.equal(i0, i1) and torch.equal(w0.view(torch.int32), w1.view(torch.int32))
    R = int(o0["offsets"][-1])
    for key in ("counts", "offsets", "token_row"):
        assert torch.equal(o0[key], o1[key]), key
    assert torch.equal(o0["row_token"][:R], o1["row_token"][:R])
    ids_o, _, _ = O.route(inp["x"], inp["w_router"], inp["bias"], cfg.k)
    assert np.array_equal(i1.cpu().numpy(), ids_o)


def test_route_dispatch_empty_batch_zeroes_counts():
    ws = moe.moe_route_dispatch_workspace()
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda")
    out = dict(counts=torch.full((8,), -7, dtype=torch.int32, device="cuda"),
               offsets=torch.full((9,), -7, dtype=torch.int32, device="cuda"),
               row_token=torch.empty(1, dtype=torch.int32, device="cuda"),
               row_w=torch.empty(1, dtype=torch.float32, device="cuda"),
               token_row=torch.empty((0, 4), dtype=torch.int32, device="cuda"))
    moe.moe_route_dispatch(x, wr, None, 4, 16, 4, 12, ws, torch.empty((0, 4), dtype=torch.int32, device="cuda"),
                           torch.empty((0, 4), dtype=torch.float32, device="cuda"), out)
    torch.cuda.synchronize()
    assert torch.all(out["counts"] == 0) and torch.all(out["offsets"] == 0)


# ----------------------------------------------------------------------------
# shared expert: standalone against the oracle, and added to the routed layer
# ----------------------------------------------------------------------------
SHARED_CASES = [
    # T <= 128: weight-streaming kernel; larger T: the direct-to-LDS tile kernel (bf16 and fp8 weights); fp32 model
    LayerConfig("sh_decode", T=64, H=256, E=4, k=2, I=64, seed=401, w_std=0.05, I_s=384),
    LayerConfig("sh_tail", T=129, H=384, E=4, k=2, I=64, seed=402, w_std=0.05, I_s=320),
    LayerConfig("sh_prefill", T=700, H=384, E=4, k=2, I=64, seed=403, w_std=0.05, I_s=448),
    LayerConfig("sh_fp8", T=300, H=256, E=4, k=2, I=64, wdt="fp8", seed=404, w_std=0.05, I_s=256),
    LayerConfig("sh_fp8_small", T=40, H=256, E=4, k=2, I=64, wdt="fp8", seed=405, w_std=0.05, I_s=192),
    LayerConfig("sh_f32", T=50, H=128, E=4, k=2, I=64, act="f32", wdt="f32", init="fan_in", seed=406, I_s=128),
    LayerConfig("sh_t1", T=1, H=4096, E=4, k=2, I=64, seed=407, w_std=0.02, I_s=1536),  # one token, split K
]


@pytest.mark.parametrize("cfg", SHARED_CASES, ids=lambda c: c.name)
def test_shared_expert_matches_oracle(cfg):
    inp = host_inputs(cfg)
    dev = L.to_device(inp)
    say(f"shared expert {cfg.name}: T={cfg.T} H={cfg.H} I_s={cfg.I_s} {cfg.wdt}")
    y = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], y, dev["ss_gate_up"], dev["ss_down"],
                          zero_y=True)
    torch.cuda.synchronize()
    y_o = O.shared_tokens(np.arange(cfg.T), inp["x"], inp["ws_gate_up"], inp["ws_down"], inp["ss_gate_up"],
                          inp["ss_down"], round_h=cfg.act != "f32")
    check_y(y.cpu().numpy(), y_o, cfg.name)
    # accumulating onto an existing y adds the same contribution: bit for bit when every element
    # gets one add (T > 128), within fp32 rounding of the split-K partial sums otherwise
    base = torch.randn((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    y2 = base.clone()
    moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], y2, dev["ss_gate_up"], dev["ss_down"])
    torch.cuda.synchronize()
    if cfg.T > 128 or cfg.act == "f32":
        assert torch.equal(y2, base + y)
    else:
        check_y((y2 - base).cpu().numpy(), y_o, cfg.name + " (accumulated)")


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "combine"])
@pytest.mark.parametrize("cfg", [SHARED_CASES[0], SHARED_CASES[2], SHARED_CASES[3]], ids=lambda c: c.name)
def test_layer_with_shared_expert_matches_oracle(cfg, fused):
    inp = host_inputs(cfg)
    dev = L.to_device(inp)
    bufs = L.LayerBuffers(cfg, fused=fused)
    say(f"layer + shared expert {cfg.name} fused={fused}")
    y = L.run_layer(dev, bufs).cpu().numpy()
    r = O.layer(inp)
    assert np.array_equal(bufs.topk_ids.cpu().numpy(), r["topk_ids"])
    y_o = r["y"].astype(np.float64) + O.shared_tokens(np.arange(cfg.T), inp["x"], inp["ws_gate_up"],
                                                      inp["ws_down"], inp["ss_gate_up"], inp["ss_down"])
    check_y(y, y_o, cfg.name + " + shared")


# ----------------------------------------------------------------------------
# W8A8 MXFP8: quantisation (bit-exact) and the MX grouped FFN against the MX oracle
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["bf16", "f32", "bf16_large"])
def test_quantize_mx_matches_oracle(dt):
    rng = np.random.default_rng(301)
    rows, K = 333, 384
    if dt == "bf16_large":  # more 8-value vectors than lanes in the grid: the grid-stride loop runs twice
        rows, K, dt = 2100, 4096, "bf16"
    x32 = (rng.standard_normal((rows, K)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    x32[0, :32] = 0.0                                  # all-zero block
    x32[1, :32] = -0.0                                 # negative zeros keep their sign bit
    x32[2, 0] = 500.0                                  # saturating element
    x32[3, 5] = 1e-30                                  # flushes to a zero code inside a normal block
    x32[4, 32:64] = np.linspace(-3, 3, 32)
    x = f32_to_bf16_bits(x32) if dt == "bf16" else x32
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() if dt == "bf16" else torch.from_numpy(x).cuda()
    codes, scales = moe.moe_quantize_mx(xd)
    torch.cuda.synchronize()
    oc, os_ = O.mx_quantize(x)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


def mx_layer(dev, cfg, ids_d, w_d, fused, packed=False, y_rows=None):
    """The W8A8 layer on the GPU; returns (y, perm dict, MX intermediate (codes, scales) from the workspace).
    ``packed``: the weight codes go in as packed copies (moe_pack_weights).  ``y_rows``: a list that
    receives the per-row outputs of the unfused path."""
    p = moe.moe_permute(ids_d, w_d, cfg.E, cfg.lo, cfg.hi)
    R_cap = p["R_cap"]
    xq, xs = moe.moe_quantize_mx(dev["x"])
    y = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_ffn_mx_workspace_size(R_cap, cfg.I), dtype=torch.uint8, device="cuda")
    wgu, wd = dev["w_gate_up"], dev["w_down"]
    if packed:
        wgu, wd = moe.moe_pack_weights(wgu), moe.moe_pack_weights(wd)
    args = (xq, xs, p["offsets"], p["row_token"], p["row_w"], cfg.T, R_cap, wgu, dev["s_gate_up"], wd, dev["s_down"])
    if fused:
        y.fill_(float("nan"))
        moe.moe_grouped_ffn_mx(*args, y=y, zero_y=True, workspace=ws, packed=packed)
    else:
        yp = torch.empty((max(R_cap, 1), cfg.H), dtype=torch.float32, device="cuda")
        moe.moe_grouped_ffn_mx(*args, y_perm=yp, workspace=ws, packed=packed)
        moe.moe_combine(yp, p["token_row"], w_d, y=y)
        if y_rows is not None:
            y_rows.append(yp)
    torch.cuda.synchronize()
    wsn = ws.cpu().numpy()
    hbytes = -(-R_cap * cfg.I // 256) * 256
    h_codes = wsn[:R_cap * cfg.I].reshape(R_cap, cfg.I)
    h_scales = wsn[hbytes:hbytes + R_cap * cfg.I // 32].reshape(R_cap, cfg.I // 32)
    return y.cpu().numpy(), p, (h_codes, h_scales)


E4M3 = np.array([O.e4m3_value(c) for c in range(256)])
U32 = 2.0 ** -24


def h_exact_and_slack(inp, t, e, cols, I, H):
    """Unrounded h = silu(G) * U (fp64) of token t, local expert e, intermediate columns ``cols``,
    and a bound on how far an fp32 evaluation may stray from it: the fp32 sum of the H exact
    products of G (or U) is within H * 2^-24 * sum|products| of the exact sum (twice that
    allowed here), and SiLU, its product with U and the rounding of h add a few units of
    2^-24 relative."""
    xq, xs = O.mx_quantize(np.asarray(inp["x"])[t:t + 1])
    xv = O.mx_dequantize(xq, xs)[0]
    wg = O.mx_dequantize(inp["w_gate_up"][e][cols], inp["s_gate_up"][e][cols])
    wu = O.mx_dequantize(inp["w_gate_up"][e][I + cols], inp["s_gate_up"][e][I + cols])
    G, U = wg @ xv, wu @ xv
    dG, dU = 2 * H * U32 * (np.abs(wg) @ np.abs(xv)), 2 * H * U32 * (np.abs(wu) @ np.abs(xv))
    sg = G / (1.0 + np.exp(-G))
    h = sg * U
    slack = 1.1 * dG * np.abs(U) + np.abs(sg) * dU + dG * dU + 8 * U32 * np.abs(h)
    return h, slack


@functools.lru_cache(maxsize=None)
def oracle_full_mx(name):
    """Oracle MX intermediate of every assignment row and y of every token of a full MXFP8
    workload, computed once and shared by its row-major and packed-weight runs."""
    cfg = CONFIGS[name]
    inp = host_inputs(cfg)
    ids, w = oracle_routing(cfg)
    perm = O.permute(ids, w, cfg.lo, cfg.hi)
    row_exp = np.repeat(np.arange(cfg.E_loc, dtype=np.int32), perm["counts"])
    say(f"  {name}: oracle MX intermediate of all {perm['R']} rows and y of all {cfg.T} tokens "
        f"({O.num_threads()} threads)")
    hq, hs = O.h_mx(perm["row_token"], row_exp, inp["x"], inp["w_gate_up"], inp["s_gate_up"])
    y = O.layer_tokens_mx(np.arange(cfg.T), inp["x"], ids, w, cfg.lo, cfg.hi, inp["w_gate_up"], inp["s_gate_up"],
                          inp["w_down"], inp["s_down"])
    return hq, hs, y


def check_mx_layer(cfg, inp, ids, w, y, h_gpu, tokens=None):
    """MX parity.  h is the quantisation of an fp32 value whose last bits depend on the order
    of the fp32 accumulation, so a GPU code may differ from the oracle's where the exact h lies
    within that rounding noise of the boundary between two E4M3 codes (or a block scale one
    step off where the block maximum lies that close to a power of two).  Checked: every
    differing code is a correct rounding of some value within the fp32 error bound of the exact
    h; every differing scale has its block maximum within that bound of the power of two
    between; every token whose intermediate rows agree matches the oracle within 1e-2 * RMS,
    every other token within that plus the exact effect of its differing h values through the
    down projection.  The permutation is the oracle's (the GPU's is bit-exact)."""
    perm = O.permute(ids, w, cfg.lo, cfg.hi)
    R, I, H = perm["R"], cfg.I, cfg.H
    counts = perm["counts"]
    row_tok = perm["row_token"]
    row_exp = np.repeat(np.arange(cfg.E_loc, dtype=np.int32), counts)
    sel = np.arange(R) if tokens is None else np.nonzero(np.isin(row_tok, tokens))[0]
    if tokens is None and CONFIGS.get(cfg.name) == cfg:
        hq_o, hs_o, y_full = oracle_full_mx(cfg.name)
    else:
        hq_o, hs_o = O.h_mx(row_tok[sel], row_exp[sel], inp["x"], inp["w_gate_up"], inp["s_gate_up"])
        y_full = None
    hq_g, hs_g = h_gpu[0][sel], h_gpu[1][sel]
    sc_o = np.repeat(hs_o.astype(np.int64), 32, axis=1) - 127
    sc_g = np.repeat(hs_g.astype(np.int64), 32, axis=1) - 127
    v_o = E4M3[hq_o] * np.exp2(sc_o)
    v_g = E4M3[hq_g] * np.exp2(sc_g)
    sdiff = hs_g != hs_o
    diff = v_g != v_o
    say(f"  {cfg.name}: {int(diff.sum())} of {diff.size} h values and {int(sdiff.sum())} of {sdiff.size} "
        f"block scales differ from the oracle's ({diff.mean() if diff.size else 0:.2e})")
    assert np.all(np.abs(hs_g.astype(np.int64) - hs_o) <= 1), "block scale more than one step off"
    worst = 0.0
    for q, blk in zip(*np.nonzero(sdiff)):
        cols = np.arange(32 * blk, 32 * blk + 32)
        h, slack = h_exact_and_slack(inp, int(row_tok[sel[q]]), int(row_exp[sel[q]]), cols, I, H)
        m = int(np.argmax(np.abs(h)))
        edge = 2.0 ** (max(int(hs_o[q, blk]), int(hs_g[q, blk])) - 127 + 8)
        worst = max(worst, abs(abs(h[m]) - edge) / slack[m])
    # every differing value is a correct E4M3 rounding, at the GPU's block scale, of some value
    # within the fp32 error bound of the exact h (small h, where G or U cancel, may move by
    # several codes: the bound is absolute, the E4M3 step near zero is 2^-9 of a block unit)
    for q in np.nonzero(diff.any(axis=1))[0]:
        cols = np.nonzero(diff[q])[0]
        h, slack = h_exact_and_slack(inp, int(row_tok[sel[q]]), int(row_exp[sel[q]]), cols, I, H)
        unit = np.exp2(sc_g[q, cols].astype(np.float64))
        code = hq_g[q, cols]
        a = np.abs(E4M3[code])
        step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
        dist = np.abs(h / unit - E4M3[code]) - step / 2
        sat = ((code & 0x7F) == 0x7E) & (np.sign(h) == np.sign(E4M3[code])) & (np.abs(h) / unit >= 448)
        dist = np.where(sat, 0.0, dist)
        worst = max(worst, float(np.max(np.maximum(dist, 0.0) / (slack / unit))))
    say(f"  {cfg.name}: largest distance of a differing value from its rounding boundary = "
        f"{worst:.3f} x the fp32 error bound")
    assert worst <= 1.0, "an h value differs where fp32 rounding cannot explain it"
    # y: oracle rows, tolerance widened only by the differing h values of each token
    toks = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    y_o = y_full if y_full is not None else O.layer_tokens_mx(toks, inp["x"], ids, w, cfg.lo, cfg.hi,
                                                              inp["w_gate_up"], inp["s_gate_up"], inp["w_down"],
                                                              inp["s_down"])
    rms = np.sqrt(np.mean(y_o.astype(np.float64) ** 2))
    bound = np.full(len(toks), Y_TOL * rms)
    pos = {int(t): n for n, t in enumerate(toks)}
    wd = {}
    for q in np.nonzero(diff.any(axis=1))[0]:
        r = sel[q]
        e = int(row_exp[r])
        if e not in wd:
            wd[e] = O.mx_dequantize(inp["w_down"][e], inp["s_down"][e])
        cols = np.nonzero(diff[q])[0]
        dh = np.abs(v_g[q, cols] - v_o[q, cols])
        bound[pos[int(row_tok[r])]] += abs(perm["row_w"][r]) * np.max(np.abs(wd[e][:, cols]) @ dh)
    err = np.max(np.abs(y[toks].astype(np.float64) - y_o), axis=1)
    say(f"  {cfg.name}: max|err| = {err.max():.3e}, RMS = {rms:.3e}, tokens with differing h: "
        f"{int((bound > Y_TOL * rms).sum())}")
    assert np.all(err <= bound)


def mx_dev(inp):
    dev = L.to_device(inp)
    for kname in ("s_gate_up", "s_down"):
        dev[kname] = torch.from_numpy(np.ascontiguousarray(inp[kname])).cuda()
    return dev


MX_CASES = [
    # several M and N tiles with ragged expert counts; N tail of the down projection (H % 256 == 128)
    LayerConfig("mx_small", T=700, H=384, E=6, k=3, I=256, wdt="mxfp8", seed=302, w_std=0.05),
    LayerConfig("mx_local", T=500, H=256, E=8, k=2, I=384, wdt="mxfp8", e_begin=2, e_end=6, seed=303, w_std=0.05),
    # few rows per expert: the weight-streaming kernel with 32-row tiles (down N tail: H % 256 == 128),
    # with 64-row tiles (more than 16 rows per local expert on average), one hot expert over many tiles
    LayerConfig("mx_stream", T=64, H=384, E=16, k=4, I=256, wdt="mxfp8", seed=306, w_std=0.05),
    LayerConfig("mx_stream_local", T=48, H=512, E=16, k=4, I=384, wdt="mxfp8", e_begin=4, e_end=12, seed=307,
                w_std=0.05),
    # K a multiple of 512 in both halves: scales read four K steps at a time
    LayerConfig("mx_stream_s4", T=64, H=512, E=16, k=4, I=512, wdt="mxfp8", seed=309, w_std=0.05),
    LayerConfig("mx_stream_hot", T=120, H=256, E=16, k=2, I=256, wdt="mxfp8", bias="zipf", seed=308, w_std=0.05),
    # tile kernel with K a multiple of 512 in both halves: scales moved four K steps at a time (two
    # groups per gate/up tile, one per down tile, whose second load is the clamped refetch)
    LayerConfig("mx_tiles_s4", T=800, H=1024, E=6, k=3, I=512, wdt="mxfp8", seed=310, w_std=0.05),
]


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "combine"])
@pytest.mark.parametrize("cfg", MX_CASES, ids=lambda c: c.name)
def test_layer_mx_matches_oracle(cfg, fused):
    inp = host_inputs(cfg)
    dev = mx_dev(inp)
    ids, w = oracle_routing(cfg)
    say(f"layer {cfg.name} fused={fused}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} MXFP8")
    ids_d, w_d = to_dev_routing(ids, w)
    y, p, h = mx_layer(dev, cfg, ids_d, w_d, fused)
    check_mx_layer(cfg, inp, ids, w, y, h)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "combine"])
def test_layer_mx_tile_boundaries(fused):
    counts = TILE_COUNTS
    cfg = LayerConfig("mx_tiles", T=1000, H=256, E=len(counts), k=5, I=256, wdt="mxfp8", seed=304, w_std=0.05)
    inp = host_inputs(cfg)
    dev = mx_dev(inp)
    ids, w = constructed_routing(counts, cfg.T, cfg.k, seed=305)
    ids_d, w_d = to_dev_routing(ids, w)
    y, p, h = mx_layer(dev, cfg, ids_d, w_d, fused)
    assert p["counts"].cpu().tolist() == counts
    check_mx_layer(cfg, inp, ids, w, y, h)


@pytest.mark.parametrize("cfg", [MX_CASES[0], MX_CASES[2], MX_CASES[3], MX_CASES[4]], ids=lambda c: c.name)
def test_mx_packed_weights_bit_identical(cfg):
    """Packed MX weight codes (tile kernel: mx_small; streaming kernel: the others) give the same
    MX intermediate and per-row outputs, bit for bit, as row-major codes; the fused layer with
    packed codes passes the oracle check."""
    inp = host_inputs(cfg)
    dev = mx_dev(inp)
    ids, w = oracle_routing(cfg)
    ids_d, w_d = to_dev_routing(ids, w)
    say(f"MX packed weights {cfg.name}: T={cfg.T} H={cfg.H} E_loc={cfg.E_loc} I={cfg.I}")
    rows_rm, rows_pk = [], []
    _, p, h_rm = mx_layer(dev, cfg, ids_d, w_d, fused=False, y_rows=rows_rm)
    _, _, h_pk = mx_layer(dev, cfg, ids_d, w_d, fused=False, packed=True, y_rows=rows_pk)
    R = int(p["offsets"][-1])
    assert np.array_equal(h_rm[0][:R], h_pk[0][:R]) and np.array_equal(h_rm[1][:R], h_pk[1][:R])
    assert torch.equal(rows_rm[0][:R].view(torch.int32), rows_pk[0][:R].view(torch.int32))
    y, _, h = mx_layer(dev, cfg, ids_d, w_d, fused=True, packed=True)
    check_mx_layer(cfg, inp, ids, w, y, h)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,fused,packed", [("prefill_mx", False, False), ("prefill_mx", False, True),
                                               ("decode_mx", True, False), ("decode_mx", False, False),
                                               ("decode_mx", True, True)])
def test_full_workload_layer_mx(name, fused, packed):
    """Full MXFP8 workloads in the benchmark's launch configuration: every assignment row's MX
    intermediate and every token's output row against the oracle."""
    cfg = CONFIGS[name]
    ids, w = oracle_routing(cfg)
    inp = host_inputs(cfg)
    dev = mx_dev(inp)  # mx_layer packs the weight codes itself when ``packed``
    say(f"full MX layer {cfg.name}: T={cfg.T}, fused={fused}, packed={packed}, all rows")
    ids_d, w_d = to_dev_routing(ids, w)
    y, p, h = mx_layer(dev, cfg, ids_d, w_d, fused=fused, packed=packed)
    del dev
    torch.cuda.empty_cache()
    check_mx_layer(cfg, inp, ids, w, y, h)


@pytest.mark.timeout(900)
def test_layer_mx_at_the_size_limit():
    """The W8A8 layer at the largest T its grouped FFN takes (R_cap * H = 2^30 - 32768, per-row
    outputs + combine, packed codes): the MX intermediate rows and y of every token that owns one of
    the highest 256 output rows, the first and last 16 tokens and 64 others."""
    cfg = MAX_CFG.replace(name="max_rows_mx", wdt="mxfp8", seed=11)
    say(f"MX size limit: generating T={cfg.T} (R_cap={cfg.R_cap})")
    inp = synth.make_inputs(cfg)
    dev = mx_dev(inp)
    ids, w, _ = O.route(inp["x"], inp["w_router"], inp["bias"], cfg.k)
    ids_d, w_d = to_dev_routing(ids, w)
    say(f"MX size limit: layer, per-row outputs {cfg.R_cap * cfg.H * 4} bytes")
    y, p, h = mx_layer(dev, cfg, ids_d, w_d, fused=False, packed=True)
    del dev
    torch.cuda.empty_cache()
    p_or = O.permute(ids, w, cfg.lo, cfg.hi)
    check_permutation(p, p_or, cfg.T, cfg.k)
    R = p_or["R"]
    rng = np.random.default_rng(11)
    toks = set(p_or["row_token"][R - 256:].tolist()) | set(range(16)) | set(range(cfg.T - 16, cfg.T))
    toks |= set(rng.choice(cfg.T, 64, replace=False).tolist())
    toks = np.array(sorted(toks), dtype=np.int32)
    say(f"MX size limit: oracle on {toks.size} tokens")
    check_mx_layer(cfg, inp, ids, w, y, h, tokens=toks)


# ----------------------------------------------------------------------------
# packed weight layout: the reorder itself, and bit-identical FFN outputs
# ----------------------------------------------------------------------------
def np_packed(w):
    """The packed block layout written with numpy: 32-row groups, 64-wide K chunks; fp8 blocks
    row-major, bf16 blocks ordered (piece q of 4 within a 32-value half g, half g, row n, 8 values)."""
    E, N, K = w.shape
    b = w.reshape(E * N // 32, 32, K // 64, 64).transpose(0, 2, 1, 3)  # [group, chunk, row, value]
    if w.dtype == np.uint16:
        b = b.reshape(b.shape[0], b.shape[1], 32, 2, 4, 8).transpose(0, 1, 4, 3, 2, 5)
    return np.ascontiguousarray(b).reshape(E, N, K)


@pytest.mark.parametrize("dt,shape", [("bf16", (3, 96, 192)), ("fp8", (2, 64, 320)), ("bf16", (64, 128)),
                                      ("fp8", (5, 32, 64))])
def test_pack_weights_layout(dt, shape):
    rng = np.random.default_rng(501)
    if dt == "bf16":
        w = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        w = rng.integers(0, 256, size=shape, dtype=np.uint8)
        wd = torch.from_numpy(w).cuda()
    out = moe.moe_pack_weights(wd)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else out.cpu().numpy()
    ref = np_packed(w.reshape((1,) + shape if len(shape) == 2 else shape)).reshape(shape)
    assert np.array_equal(got, ref)
    src = wd.cpu().view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else wd.cpu().numpy()
    assert np.array_equal(src, w)  # the source is left as it was


def ffn_rows(dev, cfg, ids_d, w_d, packed):
    """Per-row outputs y_perm (one plain store per element: deterministic) of the grouped FFN."""
    p = moe.moe_permute(ids_d, w_d, cfg.E, cfg.lo, cfg.hi)
    yp = torch.full((max(p["R_cap"], 1), cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, p["R_cap"], dev["w_gate_up"],
                        dev["w_down"], dev["s_gate_up"], dev["s_down"], y_perm=yp, packed=packed)
    torch.cuda.synchronize()
    return yp, p


PACKED_CASES = ["stream_bf16", "stream_fp8_local", "stream_hot", "ffn_bf16", "ffn_fp8_local", "ffn_skew_empty",
                "tiles_fp8"]


@pytest.mark.parametrize("name", PACKED_CASES)
def test_ffn_packed_weights_bit_identical(name):
    """Weight streaming (bf16, fp8) and direct-to-LDS tiles (bf16, fp8)
    read packed weights to the same bits as row-major ones; the fused combine matches the oracle."""
    if name == "tiles_fp8":
        cfg = LayerConfig("tiles_fp8", T=1000, H=320, E=len(TILE_COUNTS), k=5, I=192, wdt="fp8", seed=210,
                          w_std=0.05)
        ids, w = constructed_routing(TILE_COUNTS, cfg.T, cfg.k, seed=211)
    else:
        cfg = next(c for c in FFN_CASES if c.name == name)
        ids, w = oracle_routing(cfg)
    inp = host_inputs(cfg)
    dev = L.to_device(inp)
    ids_d, w_d = to_dev_routing(ids, w)
    say(f"packed weights {name}: T={cfg.T} H={cfg.H} E_loc={cfg.E_loc} I={cfg.I} {cfg.wdt}")
    y_row, p = ffn_rows(dev, cfg, ids_d, w_d, packed=False)
    L.pack_weights(dev)
    y_pk, _ = ffn_rows(dev, cfg, ids_d, w_d, packed=True)
    R = int(p["offsets"][-1])  # rows of local assignments (rows past them up to R_cap stay unwritten)
    assert R > 0 and torch.equal(y_pk[:R], y_row[:R])
    y, _ = gpu_layer_packed(dev, cfg, ids_d, w_d)
    y_o = O.layer_tokens(np.arange(cfg.T), inp["x"], ids, w, cfg.lo, cfg.hi, inp["w_gate_up"], inp["w_down"],
                         inp["s_gate_up"], inp["s_down"], round_h=True)
    check_y(y, y_o, name + " packed fused")


def gpu_layer_packed(dev, cfg, ids_d, w_d):
    p = moe.moe_permute(ids_d, w_d, cfg.E, cfg.lo, cfg.hi)
    y = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(dev["x"], p["offsets"], p["row_token"], p["row_w"], cfg.T, p["R_cap"], dev["w_gate_up"],
                        dev["w_down"], dev["s_gate_up"], dev["s_down"], y=y, zero_y=True, packed=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), p


@pytest.mark.parametrize("cfg", [SHARED_CASES[0], SHARED_CASES[2], SHARED_CASES[3], SHARED_CASES[4], SHARED_CASES[6]],
                         ids=lambda c: c.name)
def test_shared_expert_packed_weights(cfg):
    """Packed shared-expert weights: the same bits where every element of y gets one add (T > 128),
    the oracle's result within tolerance on the split-K path."""
    inp = host_inputs(cfg)
    dev = L.to_device(inp)
    say(f"shared expert packed {cfg.name}: T={cfg.T} H={cfg.H} I_s={cfg.I_s} {cfg.wdt}")
    y_row = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], y_row, dev["ss_gate_up"], dev["ss_down"],
                          zero_y=True)
    L.pack_weights(dev)
    y_pk = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_shared_expert(dev["x"], dev["ws_gate_up"], dev["ws_down"], y_pk, dev["ss_gate_up"], dev["ss_down"],
                          zero_y=True, packed=True)
    torch.cuda.synchronize()
    if cfg.T > 128:
        assert torch.equal(y_pk, y_row)
    y_o = O.shared_tokens(np.arange(cfg.T), inp["x"], inp["ws_gate_up"], inp["ws_down"], inp["ss_gate_up"],
                          inp["ss_down"], round_h=True)
    check_y(y_pk.cpu().numpy(), y_o, cfg.name + " packed")
