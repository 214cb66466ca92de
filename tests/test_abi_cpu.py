"""CPU checks of the C ABI: the library loads without a GPU, exports every symbol
the header declares, and rejects bad arguments on the host before any HIP call
(nothing here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest
import torch

from expert_routed_grouped_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    L = moe.lib()
    names = header_functions()
    assert set(names) == set(moe.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert moe.moe_version() == 100


def test_status_strings():
    L = moe.lib()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.moe_status_str(code)
    assert L.moe_status_str(-99) == b"unknown status"


P = ctypes.c_void_p
FAKE = P(0x1000)  # never dereferenced: every call below fails validation first
FAKE_ODD = P(0x1004)


def route(**kw):
    a = dict(x=FAKE, xd=1, w=FAKE, wd=1, b=None, T=4, H=64, E=8, k=2, ids=FAKE, gw=FAKE)
    a.update(kw)
    return moe.lib().moe_route(a["x"], a["xd"], a["w"], a["wd"], a["b"], a["T"], a["H"], a["E"], a["k"], a["ids"],
                               a["gw"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), -2), (dict(k=9), -2), (dict(E=1025, k=2), -2), (dict(E=64, k=33), -2), (dict(T=-1), -2),
    (dict(H=0), -2), (dict(xd=2), -3), (dict(wd=7), -3), (dict(x=None), -1), (dict(ids=None), -1),
    (dict(gw=None), -1), (dict(T=0), 0),
])
def test_route_validation(kw, code):
    assert route(**kw) == code


def permute(**kw):
    a = dict(ids=FAKE, w=FAKE, T=4, k=2, E=8, lo=0, hi=8, c=FAKE, o=FAKE, rt=FAKE, rw=FAKE, tr=FAKE, x=None, xd=1,
             H=0, xp=None, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return moe.lib().moe_permute(a["ids"], a["w"], a["T"], a["k"], a["E"], a["lo"], a["hi"], a["c"], a["o"], a["rt"],
                                 a["rw"], a["tr"], a["x"], a["xd"], a["H"], a["xp"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(lo=3, hi=3), -2), (dict(lo=-1), -2), (dict(hi=9), -2), (dict(k=9), -2), (dict(E=1100, hi=1100), -2),
    (dict(c=None), -1), (dict(rt=None), -1), (dict(x=FAKE), -1), (dict(xp=FAKE), -1),
    (dict(x=FAKE, xp=FAKE, H=12), -2), (dict(x=FAKE, xp=FAKE, H=64, xd=2), -3),
    (dict(x=FAKE_ODD, xp=FAKE, H=64), -6), (dict(ws=None), -4), (dict(wsb=0), -4), (dict(ws=P(0x1010)), -6),
])
def test_permute_validation(kw, code):
    assert permute(**kw) == code


def ffn(**kw):
    a = dict(a=FAKE, ad=1, off=FAKE, rt=FAKE, rw=FAKE, El=8, T=16, R=32, H=128, I=64, wgu=FAKE, wd=FAKE, wdt=1,
             sgu=None, sd=None, y=FAKE, yp=None, ws=FAKE, wsb=1 << 30, flags=3)
    a.update(kw)
    return moe.lib().moe_grouped_ffn(a["a"], a["ad"], a["off"], a["rt"], a["rw"], a["El"], a["T"], a["R"], a["H"],
                                     a["I"], a["wgu"], a["wd"], a["wdt"], a["sgu"], a["sd"], a["y"], a["yp"], a["ws"],
                                     a["wsb"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=100), -2), (dict(I=96), -2), (dict(El=0), -2), (dict(R=16 * 8 + 1), -2), (dict(T=-1), -2),
    (dict(ad=0), -3), (dict(wdt=0), -3), (dict(ad=2, wdt=2), -3),
    (dict(y=None), -1), (dict(yp=FAKE), -1), (dict(wdt=2), -1), (dict(rt=None), -1), (dict(rw=None), -1),
    (dict(ws=None), -4), (dict(wsb=10), -4), (dict(a=FAKE_ODD), -6), (dict(ws=P(0x1010)), -6),
    (dict(T=1 << 20, R=1 << 20, H=1024), -2), (dict(flags=3 | 32), -2), (dict(ad=0, wdt=0, flags=3 | 16), -3),
    (dict(T=32768, R=262144, H=4096, I=1536), -2),  # R_cap * H = 2^30: one row past the limit
])
def test_ffn_validation(kw, code):
    assert ffn(**kw) == code


def ffn_mx(**kw):
    a = dict(a=FAKE, as_=FAKE, off=FAKE, rt=FAKE, rw=FAKE, El=8, T=16, R=32, H=256, I=128, wgu=FAKE, wgus=FAKE,
             wd=FAKE, wds=FAKE, y=FAKE, yp=None, ws=FAKE, wsb=1 << 30, flags=3)
    a.update(kw)
    return moe.lib().moe_grouped_ffn_mx(a["a"], a["as_"], a["off"], a["rt"], a["rw"], a["El"], a["T"], a["R"], a["H"],
                                        a["I"], a["wgu"], a["wgus"], a["wd"], a["wds"], a["y"], a["yp"], a["ws"],
                                        a["wsb"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=192), -2), (dict(I=64), -2), (dict(El=0), -2), (dict(R=16 * 8 + 1), -2), (dict(T=1 << 20, R=1 << 20, H=1024), -2),
    (dict(y=None), -1), (dict(yp=FAKE), -1), (dict(as_=None), -1), (dict(wds=None), -1), (dict(rt=None), -1),
    (dict(ws=None), -4), (dict(wsb=10), -4), (dict(a=FAKE_ODD), -6), (dict(as_=P(0x1002)), -6),
    (dict(ws=P(0x1010)), -6), (dict(flags=3 | 4 | 8), -2), (dict(T=32768, R=262144, H=4096, I=1536), -2),
])
def test_ffn_mx_validation(kw, code):
    assert ffn_mx(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(K=48), -2), (dict(K=0), -2), (dict(rows=-1), -2), (dict(xd=2), -3), (dict(x=None), -1),
    (dict(q=None), -1), (dict(rows=0), 0), (dict(x=FAKE_ODD), -6), (dict(q=FAKE_ODD), -6),
])
def test_quantize_mx_validation(kw, code):
    a = dict(x=FAKE, xd=1, rows=4, K=64, q=FAKE, s=FAKE)
    a.update(kw)
    assert moe.lib().moe_quantize_mx(a["x"], a["xd"], a["rows"], a["K"], a["q"], a["s"], None) == code


def shared(x=FAKE, xd=1, T=8, H=64, I_s=64, wgu=FAKE, wd=FAKE, wdt=1, sgu=None, sd=None, y=FAKE, ws=FAKE,
           wsb=1 << 20, flags=0):
    return moe.lib().moe_shared_expert(x, xd, T, H, I_s, wgu, wd, wdt, sgu, sd, y, ws, wsb, flags, None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=96), -2), (dict(I_s=32), -2), (dict(T=-1), -2), (dict(T=1 << 20, H=2048), -2), (dict(flags=1), -2),
    (dict(xd=0), -3), (dict(wdt=3), -3), (dict(x=None), -1), (dict(y=None), -1), (dict(wd=None), -1),
    (dict(wdt=2), -1), (dict(ws=None), -4), (dict(wsb=64), -4), (dict(y=FAKE_ODD), -6), (dict(T=0), 0),
    (dict(flags=16 | 1), -2), (dict(flags=32), -2), (dict(xd=0, wdt=0, flags=16), -3), (dict(T=0, flags=16 | 2), 0),
])
def test_shared_expert_validation(kw, code):
    # every case is rejected (or is empty) on the host before anything is launched
    assert shared(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dt=0), -3), (dict(dt=3), -3), (dict(E=0), -2), (dict(N=48), -2), (dict(N=0), -2), (dict(K=96), -2),
    (dict(K=32), -2), (dict(w=None), -1), (dict(out=None), -1), (dict(w=FAKE_ODD), -6), (dict(out=P(0x9008)), -6),
    (dict(out=P(0x1000 + 4096 - 16)), -2), (dict(out=FAKE), -2), (dict(w=P(0x1000 + 2048), out=FAKE, dt=2, K=128), -2),
])
def test_pack_weights_validation(kw, code):
    # every case is rejected on the host before anything is launched (the last three overlap)
    a = dict(w=FAKE, dt=1, E=1, N=32, K=64, out=P(0x9000))
    a.update(kw)
    assert moe.lib().moe_pack_weights(a["w"], a["dt"], a["E"], a["N"], a["K"], a["out"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), -3), (dict(dt=4), -3), (dict(E=0), -2), (dict(E=1025), -2), (dict(H=6), -2), (dict(H=0), -2),
    (dict(w=None), -1), (dict(out=None), -1), (dict(w=P(0x1001)), -6), (dict(out=P(0x9008)), -6),
    (dict(dt=0, w=P(0x1002)), -6),
])
def test_pack_router_validation(kw, code):
    # every case is rejected on the host before anything is launched
    a = dict(w=FAKE, dt=1, E=128, H=4096, out=P(0x9000))
    a.update(kw)
    assert moe.lib().moe_pack_router(a["w"], a["dt"], a["E"], a["H"], a["out"], None) == code


def route_dispatch(x=FAKE, xd=1, w=FAKE, wd=1, T=64, H=256, E=16, k=4, lo=0, hi=16, ids=FAKE, g=FAKE, c=FAKE,
                   o=FAKE, rt=FAKE, rw=FAKE, tr=FAKE, y=None, ws=FAKE, wsb=256):
    return moe.lib().moe_route_dispatch(x, xd, w, wd, None, T, H, E, k, lo, hi, ids, g, c, o, rt, rw, tr, y, ws, wsb,
                                        None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=513), -2), (dict(T=300, k=32, E=64, hi=64), -2), (dict(E=257, hi=257), -2), (dict(H=100), -2),
    (dict(k=17, E=16), -2), (dict(lo=4, hi=4), -2), (dict(hi=17), -2), (dict(x=FAKE_ODD), -2), (dict(xd=2), -3),
    (dict(x=None), -1), (dict(c=None), -1), (dict(rt=None), -1), (dict(ws=None), -4), (dict(wsb=16), -4),
    (dict(wd=5), -3), (dict(wd=2), -3), (dict(wd=4, ws=None), -4),
    (dict(y=FAKE_ODD), -6),
])
def test_route_dispatch_validation(kw, code):
    # every case is rejected (or is empty) on the host before anything is launched
    assert route_dispatch(**kw) == code


def test_workspace_size():
    L = moe.lib()
    # per-chunk (1024 assignments) expert counts
    assert L.moe_permute_workspace_size(6000, 8, 128) >= 47 * 128 * 4
    assert L.moe_permute_workspace_size(0, 8, 128) > 0
    # h [R_cap, I] bf16 plus an aligned schedule prefix
    ws = L.moe_ffn_workspace_size(48000, 128, 4096, 1536, 1)
    assert ws >= 48000 * 1536 * 2 and ws % 256 == 0
    assert L.moe_ffn_workspace_size(100, 4, 64, 64, 0) >= 100 * 64 * 4
    # h as MXFP8: codes [R_cap, I] and scales [R_cap, I/32], each 256-byte aligned
    ws = L.moe_ffn_mx_workspace_size(48000, 1536)
    assert ws >= 48000 * 1536 + 48000 * 48 and ws % 256 == 0
    assert L.moe_route_dispatch_workspace_size() == 256
    # shared expert: h [T, I_s] plus its row maps (offsets, row_token, row_w)
    ws = L.moe_shared_workspace_size(6000, 1536, 1)
    assert ws >= 6000 * 1536 * 2 + 8 + 2 * 6000 * 4 and ws % 256 == 0


@pytest.mark.parametrize("kw,code", [
    (dict(H=6), -2), (dict(k=0), -2), (dict(y=None), -1), (dict(yp=FAKE_ODD), -6), (dict(T=0), 0),
])
def test_combine_validation(kw, code):
    a = dict(yp=FAKE, tr=FAKE, w=FAKE, T=4, k=2, H=64, y=FAKE)
    a.update(kw)
    assert moe.lib().moe_combine(a["yp"], a["tr"], a["w"], a["T"], a["k"], a["H"], a["y"], None) == code


def test_python_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        moe.lib()


def test_binding_rejects_host_and_strided_tensors():
    # a host pointer handed to a kernel would fault the GPU: the binding refuses it first
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    wr = torch.zeros((8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on the GPU"):
        moe.moe_route(x, wr, None, 2, torch.zeros((4, 2), dtype=torch.int32), torch.zeros((4, 2)))
    with pytest.raises(ValueError, match="contiguous"):
        moe.moe_quantize_mx(torch.zeros((64, 64)).t())


def test_binding_checks_packed_router_layout():
    # the C ABI cannot see buffer sizes: a raw [E, H] bf16 weight passed as packed fp32 would be read
    # past its end, so the binding checks the moe_pack_router layout before calling the library
    T, H, E, k = 4, 64, 8, 2
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    out = {}
    ids, gw = torch.zeros((T, k), dtype=torch.int32), torch.zeros((T, k))
    for bad in (torch.zeros((E, H), dtype=torch.bfloat16), torch.zeros((H // 4, E, 4), dtype=torch.bfloat16),
                torch.zeros((H // 4, E + 1, 4))):
        with pytest.raises(ValueError, match="moe_pack_router"):
            moe.moe_route_dispatch(x, bad, None, k, E, 0, E, None, ids, gw, out, router_packed=True)
    with pytest.raises(ValueError, match=r"\[E, H\]"):
        moe.moe_route_dispatch(x, torch.zeros((H // 4, E, 4)), None, k, E, 0, E, None, ids, gw, out)


def test_layer_repacks_router_after_the_weight_changes(monkeypatch):
    # layer.pack_router records which tensor (and which in-place version of it) the packed copy came
    # from; a replaced or edited router weight is packed again instead of routing with stale values
    from expert_routed_grouped_amd import layer as L
    calls = []
    monkeypatch.setattr(moe, "moe_pack_router", lambda w: calls.append(w) or ("packed", w.clone()))
    dev = {"w_router": torch.zeros((8, 64))}
    L.pack_router(dev)
    L.pack_router(dev)
    assert len(calls) == 1 and L._router_pack_current(dev)
    dev["w_router"].add_(1.0)  # edited in place
    assert not L._router_pack_current(dev)
    L.pack_router(dev)
    assert len(calls) == 2 and L._router_pack_current(dev)
    dev["w_router"] = torch.ones((8, 64))  # replaced
    assert not L._router_pack_current(dev)


@pytest.mark.parametrize("kw,code", [
    # h [R_cap, I] bf16 past the 32 MiB static scratch: 10923 rows x 1536 x 2 bytes
    (dict(T=10923, R=10923, H=4096, I=1536, El=128), -4),
    (dict(T=64, R=1 << 20, H=64, I=64, El=1 << 15), -2),
    (dict(ad=2), -3), (dict(y=None), -1), (dict(y=FAKE, yp=FAKE), -1), (dict(a=FAKE_ODD), -6),
    (dict(flags=1 << 7), -2), (dict(flags=4 | 8), -2),
])
def test_ffn_noalloc_validation(kw, code):
    # every argument error is found on the host before the static scratch is looked up (no GPU needed)
    a = dict(a=FAKE, ad=1, off=FAKE, rt=FAKE, rw=FAKE, El=8, T=16, R=32, H=128, I=64, wgu=FAKE, wd=FAKE, wdt=1,
             sgu=None, sd=None, y=FAKE, yp=None, flags=3)
    a.update(kw)
    assert moe.lib().moe_grouped_ffn_noalloc(a["a"], a["ad"], a["off"], a["rt"], a["rw"], a["El"], a["T"], a["R"],
                                             a["H"], a["I"], a["wgu"], a["wd"], a["wdt"], a["sgu"], a["sd"], a["y"],
                                             a["yp"], a["flags"], None) == code


def test_noalloc_limit_matches_header():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)" in src
    assert moe.MOE_NOALLOC_SCRATCH_BYTES == 32 << 20
    # the largest decode-sized h that fits: 10922 rows of I = 1536 bf16 values
    assert moe.moe_ffn_workspace_size(10922, 128, 4096, 1536, moe.MOE_BF16) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    assert moe.moe_ffn_workspace_size(10923, 128, 4096, 1536, moe.MOE_BF16) > moe.MOE_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,code", [
    (dict(T=65), -2), (dict(H=96), -2), (dict(I=100), -2), (dict(E=257, hi=257), -2), (dict(k=0), -2),
    (dict(lo=4, hi=4), -2), (dict(xd=0), -3), (dict(wrd=2), -3), (dict(wd=0), -3), (dict(flags=1), -2),
    (dict(y=None), -1), (dict(wgu=None), -1), (dict(wd=2, sgu=None), -1), (dict(ws=None), -4), (dict(wsb=64), -4),
    (dict(ws=P(0x1010)), -6), (dict(x=FAKE_ODD), -6),
])
def test_decode_layer_validation(kw, code):
    # every case is refused on the host before anything is launched (no GPU needed)
    a = dict(x=FAKE, xd=1, wr=FAKE, wrd=1, b=None, T=64, H=256, E=16, k=4, lo=0, hi=16, I=128, wgu=FAKE, wd=1,
             wdown=FAKE, sgu=FAKE, sd=FAKE, ids=FAKE, gw=FAKE, c=FAKE, o=FAKE, rt=FAKE, rw=FAKE, tr=FAKE, y=FAKE,
             ws=FAKE, wsb=1 << 30, flags=0)
    a.update(kw)
    wdt = a["wd"]
    assert moe.lib().moe_decode_layer(a["x"], a["xd"], a["wr"], a["wrd"], a["b"], a["T"], a["H"], a["E"], a["k"],
                                      a["lo"], a["hi"], a["I"], a["wgu"], a["wdown"], 2 if wdt == 2 else wdt,
                                      a["sgu"], a["sd"], a["ids"], a["gw"], a["c"], a["o"], a["rt"], a["rw"], a["tr"],
                                      a["y"], a["ws"], a["wsb"], a["flags"], None) == code


def test_decode_layer_workspace_size():
    L = moe.lib()
    # control words (64 + E_loc, 256-byte aligned), then the dense h [E_loc, T, I] bf16
    assert L.moe_decode_layer_workspace_size(64, 8, 128, 1536) == 768 + 128 * 64 * 1536 * 2
    assert L.moe_decode_layer_workspace_size(1, 4, 16, 128) == 512 + 16 * 128 * 2


@pytest.mark.parametrize("T,k,El,H,I", [(6000, 8, 128, 4096, 1536), (64, 8, 128, 4096, 1536), (1, 1, 1, 64, 64),
                                        (8192, 8, 32, 4096, 1536), (0, 4, 16, 256, 128), (70, 32, 1024, 256, 64)])
def test_workspace_size_by_operation(T, k, El, H, I):
    # moe_workspace_size(op, ...) gives the per-call functions' numbers
    L = moe.lib()
    R = T * min(k, El)
    assert moe.moe_workspace_size(moe.MOE_OP_PERMUTE, T, k, El, H, I) == L.moe_permute_workspace_size(T, k, El)
    assert moe.moe_workspace_size(moe.MOE_OP_GROUPED_FFN, T, k, El, H, I) == moe.moe_ffn_workspace_size(R, El, H, I, 1)
    assert (moe.moe_workspace_size(moe.MOE_OP_GROUPED_FFN_F32, T, k, El, H, I)
            == moe.moe_ffn_workspace_size(R, El, H, I, 0))
    assert moe.moe_workspace_size(moe.MOE_OP_GROUPED_FFN_MX, T, k, El, H, I) == moe.moe_ffn_mx_workspace_size(R, I)
    assert moe.moe_workspace_size(moe.MOE_OP_ROUTE_DISPATCH, T, k, El, H, I) == 256
    assert (moe.moe_workspace_size(moe.MOE_OP_DECODE_LAYER, T, k, El, H, I)
            == L.moe_decode_layer_workspace_size(T, k, El, I))
    assert moe.moe_workspace_size(moe.MOE_OP_SHARED_EXPERT, T, k, El, H, I) == moe.moe_shared_workspace_size(T, I, 1)
    assert (moe.moe_workspace_size(moe.MOE_OP_SHARED_EXPERT_F32, T, k, El, H, I)
            == moe.moe_shared_workspace_size(T, I, 0))
    assert moe.moe_workspace_size(99, T, k, El, H, I) == 0
    assert moe.moe_workspace_size(moe.MOE_OP_PERMUTE, -1, k, El, H, I) == 0
