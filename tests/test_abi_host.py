"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libfp8kv.so loads and exports every function include/fp8kv.h declares;
* each refusal the header documents comes back as its status code, with a
  message, before anything is enqueued (FreeToken #354: unsupported fp8
  combinations are refused, not ignored; its review thread: bounds are
  checked on the host where the host can check them);
* the workspace size follows the documented layout.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8kv.h")

OK, E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_UNSUPPORTED, E_WORKSPACE, E_LAUNCH = \
    0, -1, -2, -3, -4, -5, -6, -7
E_NOT_DEVICE, E_RANGE = -8, -9
BF16, FP16, FP32 = 1, 2, 3


@pytest.fixture(scope="module")
def L():
    import fp8_e4m3_paged_kv_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        from fp8_e4m3_paged_kv_amd import build
        build.build()
    return pkg.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8kv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_strings(L):
    text = open(HEADER).read()
    ver = int(re.search(r"#define FP8KV_ABI_VERSION (\d+)", text).group(1))
    assert L.fp8kv_abi_version() == ver
    for st in (OK, E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_UNSUPPORTED,
               E_WORKSPACE, E_LAUNCH, E_NOT_DEVICE, E_RANGE):
        assert L.fp8kv_status_string(st).decode() != "unknown status"
    for name, st in (("E_NOT_DEVICE", E_NOT_DEVICE), ("E_RANGE", E_RANGE)):
        assert re.search(rf"FP8KV_{name} = {st}\b", text), name


def test_checked_mode_switch(L):
    prev = L.fp8kv_set_checked(1)
    try:
        assert L.fp8kv_set_checked(1) == 1
        assert L.fp8kv_set_checked(0) == 1
        assert L.fp8kv_set_checked(0) == 0
        assert L.fp8kv_set_checked(7) == 0       # any nonzero value switches it on
        assert L.fp8kv_set_checked(0) == 1
    finally:
        L.fp8kv_set_checked(prev)


def test_checked_mode_keeps_the_host_checks_first(L):
    """In checked mode the O(1) refusals still come first, and a call whose
    pointers the runtime does not know as device memory is refused (here:
    fake addresses) -- nothing is launched either way."""
    prev = L.fp8kv_set_checked(1)
    try:
        assert qs(L, k=0) == E_NULL
        assert qs(L, D=96) == E_UNSUPPORTED
        st = qs(L)
        assert st in (E_NOT_DEVICE, E_LAUNCH), st    # E_LAUNCH: no HIP device here
        assert L.fp8kv_last_error().decode()
    finally:
        L.fp8kv_set_checked(prev)


# A fake, well-aligned "device" address: validation never dereferences it.
A = 1 << 40


def qs(L, **kw):
    a = dict(k=A, kst=6144, ksh=128, v=A + 8192, vst=6144, vsh=128,
             dtype=BF16, T=16, H=8, D=128, slots=A, kc=A, vc=A, css=1024,
             csh=128, ks=A, vs=A, sss=8, ssh=1, S=1 << 20)
    a.update(kw)
    return L.fp8kv_kv_quant_scatter(
        a["k"], a["kst"], a["ksh"], a["v"], a["vst"], a["vsh"], a["dtype"],
        a["T"], a["H"], a["D"], a["slots"], a["kc"], a["vc"], a["css"],
        a["csh"], a["ks"], a["vs"], a["sss"], a["ssh"], a["S"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=FP16), E_UNSUPPORTED),
    (dict(dtype=FP32), E_UNSUPPORTED),
    (dict(D=96), E_UNSUPPORTED),
    (dict(D=256), E_UNSUPPORTED),
    (dict(T=-1), E_SHAPE),
    (dict(H=0), E_SHAPE),
    (dict(k=0), E_NULL),
    (dict(slots=0), E_NULL),
    (dict(vs=0), E_NULL),
    (dict(vst=-384), E_STRIDE),
    (dict(k=A + 2), E_ALIGN),
    (dict(vst=6140), E_ALIGN),
    (dict(kc=A + 8), E_ALIGN),
    (dict(css=1000), E_ALIGN),
    (dict(slots=A + 4), E_ALIGN),
    (dict(T=0), OK),                     # nothing to do: nothing launched
])
def test_quant_scatter_refusals(L, kw, status):
    assert qs(L, **kw) == status
    if status != OK:
        assert L.fp8kv_last_error().decode()


def dec(L, fn="fp8kv_paged_decode_attn_fp8", **kw):
    a = dict(q=A, qsb=4096, qsr=4096, qsh=128, qdt=BF16, kc=A, vc=A,
             css=1024, csh=128, ks=A, vs=A, sss=1, ssh=1 << 20, S=1 << 20,
             bt=A, bts=2048, cl=A, B=64, R=1, Hq=32, H=8, D=128, bs=16,
             scale=0.088, P=384, maxc=32768, ws=A, wsb=1 << 34, out=A,
             osb=4096, osr=4096, osh=128, odt=BF16)
    a.update(kw)
    common = [a["q"], a["qsb"], a["qsr"], a["qsh"], a["qdt"], a["kc"],
              a["vc"], a["css"], a["csh"], a["ks"], a["vs"], a["sss"],
              a["ssh"], a["S"], a["bt"], a["bts"], a["cl"], a["B"], a["R"],
              a["Hq"], a["H"], a["D"], a["bs"], ctypes.c_float(a["scale"]),
              a["P"], a["maxc"], a["ws"], a["wsb"]]
    if fn == "fp8kv_paged_decode_partials":
        return getattr(L, fn)(*common, None)
    return getattr(L, fn)(*common, a["out"], a["osb"], a["osr"], a["osh"],
                          a["odt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qdt=FP16), E_UNSUPPORTED),
    (dict(odt=FP16), E_UNSUPPORTED),
    (dict(D=96), E_UNSUPPORTED),
    (dict(Hq=30), E_SHAPE),              # not a multiple of Hkv
    (dict(R=5), E_UNSUPPORTED),          # 5 * 4 > 16 stacked rows
    (dict(Hq=64, H=2), E_UNSUPPORTED),   # group 32 > 16
    (dict(bs=8), E_UNSUPPORTED),
    (dict(bs=24), E_UNSUPPORTED),
    (dict(P=-1), E_SHAPE),               # num_ranges
    (dict(P=1 << 21), E_SHAPE),
    (dict(maxc=-1), E_SHAPE),
    (dict(B=-1), E_SHAPE),
    (dict(q=0), E_NULL),
    (dict(bt=0), E_NULL),
    (dict(out=0), E_NULL),
    (dict(ws=0), E_WORKSPACE),
    (dict(wsb=1024), E_WORKSPACE),
    (dict(css=-1024), E_STRIDE),
    (dict(q=A + 8), E_ALIGN),
    (dict(qsh=100), E_ALIGN),
    (dict(css=1000), E_ALIGN),
    (dict(ws=A + 64), E_ALIGN),
    (dict(S=8), E_SHAPE),                # no whole block in the pool
])
def test_decode_refusals(L, kw, status):
    assert dec(L, **kw) == status
    assert L.fp8kv_last_error().decode()


def test_partials_refusals(L):
    assert dec(L, fn="fp8kv_paged_decode_partials", qdt=FP32) == E_UNSUPPORTED
    assert dec(L, fn="fp8kv_paged_decode_partials", wsb=16) == E_WORKSPACE


def test_workspace_layout(L):
    B, R, Hq, H, D, NR = 64, 1, 32, 8, 128, 384
    n = L.fp8kv_paged_decode_workspace_bytes(B, R, Hq, H, D, NR)
    M = R * Hq // H
    units = (B + NR - 1) * H * M          # piece ids b + r < B + NR - 1
    rnd = lambda x: (x + 255) // 256 * 256
    assert n == rnd(units * D * 4) + rnd(units * 4) + rnd((B + 1) * 4)
    assert L.fp8kv_paged_decode_workspace_bytes(B, R, Hq, H, 96, NR) == E_UNSUPPORTED
    assert L.fp8kv_paged_decode_workspace_bytes(B, R, Hq, H, D, -3) == E_SHAPE


def test_num_ranges(L):
    f = L.fp8kv_paged_decode_num_ranges
    assert f(8, 384) == 384
    assert f(4, 1) == 1
    assert f(8, -1) == E_SHAPE
    assert f(0, 16) == E_SHAPE


def test_binding_refuses_host_tensors():
    import torch
    import fp8_e4m3_paged_kv_amd as fk
    k = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fk.kv_quant_scatter(k, k, torch.zeros(4, dtype=torch.int64),
                            torch.zeros((16, 2, 64), dtype=torch.uint8),
                            torch.zeros((16, 2, 64), dtype=torch.uint8),
                            torch.zeros((16, 2)), torch.zeros((16, 2)))


MXFP4, E4M3 = 0, 1


def ikq(L, **kw):
    a = dict(keys=A, ks=128, n=1024, D=128, fmt=MXFP4, codes=A, cs=64,
             scales=A, ss=4)
    a.update(kw)
    return L.fp8kv_index_keys_quantize(a["keys"], a["ks"], a["n"], a["D"],
                                       a["fmt"], a["codes"], a["cs"],
                                       a["scales"], a["ss"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), E_UNSUPPORTED),
    (dict(fmt=2), E_UNSUPPORTED),
    (dict(n=-1), E_SHAPE),
    (dict(keys=0), E_NULL),
    (dict(scales=0), E_NULL),
    (dict(ks=-128), E_STRIDE),
    (dict(keys=A + 8), E_ALIGN),
    (dict(ks=132), E_ALIGN),
    (dict(codes=A + 2), E_ALIGN),
    (dict(fmt=E4M3, cs=132), E_ALIGN),   # E4M3 code rows are 8-byte aligned
    (dict(fmt=E4M3, cs=128, scales=A + 2), E_ALIGN),
    (dict(n=0), OK),
])
def test_index_keys_refusals(L, kw, status):
    assert ikq(L, **kw) == status
    if status != OK:
        assert L.fp8kv_last_error().decode()


def isc(L, **kw):
    a = dict(q=A, qsb=1 << 19, qsr=2048, qsh=128, qdt=BF16, w=A, wsb=4096,
             wsr=16, wsh=1, fmt=MXFP4, codes=A, csb=1 << 22, csk=64, scales=A,
             ssb=1 << 18, ssk=4, B=8, R=256, H=16, D=128, N=65536, chunk=4096,
             out=A, osb=1 << 24, osr=65536)
    a.update(kw)
    return L.fp8kv_index_score_mxfp4(
        a["q"], a["qsb"], a["qsr"], a["qsh"], a["qdt"], a["w"], a["wsb"],
        a["wsr"], a["wsh"], a["fmt"], a["codes"], a["csb"], a["csk"],
        a["scales"], a["ssb"], a["ssk"], a["B"], a["R"], a["H"], a["D"],
        a["N"], a["chunk"], a["out"], a["osb"], a["osr"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), E_UNSUPPORTED),
    (dict(qdt=FP16), E_UNSUPPORTED),
    (dict(fmt=3), E_UNSUPPORTED),
    (dict(H=17), E_UNSUPPORTED),
    (dict(H=0), E_UNSUPPORTED),
    (dict(R=0), E_SHAPE),
    (dict(B=-1), E_SHAPE),
    (dict(N=-5), E_SHAPE),
    (dict(chunk=24), E_SHAPE),
    (dict(chunk=-16), E_SHAPE),
    (dict(q=0), E_NULL),
    (dict(w=0), E_NULL),
    (dict(out=0), E_NULL),
    (dict(wsh=-1), E_STRIDE),
    (dict(osr=-1), E_STRIDE),
    (dict(q=A + 4), E_ALIGN),
    (dict(qsh=100), E_ALIGN),
    (dict(csk=72), E_ALIGN),
    (dict(codes=A + 8), E_ALIGN),
    (dict(fmt=E4M3, csk=128, scales=A + 1), E_ALIGN),
    (dict(out=A + 2), E_ALIGN),
    (dict(osr=1 << 22), E_SHAPE),        # one request's scores span >= 2^30 bytes
    (dict(osr=65535), E_STRIDE),         # score rows overlap
    (dict(R=2, osr=1 << 27), E_SHAPE),   # a wave's rows past the end would pass 2^31 bytes
    (dict(B=0), OK),
    (dict(N=0), OK),
])
def test_index_score_refusals(L, kw, status):
    assert isc(L, **kw) == status
    if status != OK:
        assert L.fp8kv_last_error().decode()


def sdec(L, fn="fp8kv_sparse_decode_attn_fp8", bv=A, bvs=2048, **kw):
    """The sparse calls take (block_valid, stride) after the block table."""
    a = dict(q=A, qsb=4096, qsr=4096, qsh=128, qdt=BF16, kc=A, vc=A,
             css=1024, csh=128, ks=A, vs=A, sss=1, ssh=1 << 20, S=1 << 20,
             bt=A, bts=2048, cl=A, B=64, R=1, Hq=32, H=8, D=128, bs=16,
             scale=0.088, P=384, maxc=32768, ws=A, wsb=1 << 34, out=A,
             osb=4096, osr=4096, osh=128, odt=BF16)
    a.update(kw)
    common = [a["q"], a["qsb"], a["qsr"], a["qsh"], a["qdt"], a["kc"],
              a["vc"], a["css"], a["csh"], a["ks"], a["vs"], a["sss"],
              a["ssh"], a["S"], a["bt"], a["bts"], bv, bvs, a["cl"], a["B"],
              a["R"], a["Hq"], a["H"], a["D"], a["bs"],
              ctypes.c_float(a["scale"]), a["P"], a["maxc"], a["ws"], a["wsb"]]
    if fn == "fp8kv_sparse_decode_partials":
        return getattr(L, fn)(*common, None)
    return getattr(L, fn)(*common, a["out"], a["osb"], a["osr"], a["osh"],
                          a["odt"], None)


@pytest.mark.parametrize("fn", ["fp8kv_sparse_decode_attn_fp8",
                                "fp8kv_sparse_decode_partials"])
@pytest.mark.parametrize("kw,status", [
    (dict(bv=0), E_NULL),
    (dict(bv=A + 2), E_ALIGN),
    (dict(bvs=-1), E_STRIDE),
    (dict(qdt=FP16), E_UNSUPPORTED),
    (dict(D=96), E_UNSUPPORTED),
    (dict(bs=24), E_UNSUPPORTED),
    (dict(wsb=1024), E_WORKSPACE),
    (dict(bt=0), E_NULL),
])
def test_sparse_decode_refusals(L, fn, kw, status):
    assert sdec(L, fn=fn, **kw) == status
    assert L.fp8kv_last_error().decode()


def ikb(L, **kw):
    a = dict(raw=A, rsb=1 << 25, rst=128, B=8, g0=0, g1=65536, D=128, fmt=MXFP4,
             codes=A, csb=1 << 22, csk=64, scales=A, ssb=1 << 18, ssk=4)
    a.update(kw)
    return L.fp8kv_index_keys_build(a["raw"], a["rsb"], a["rst"], a["B"], a["g0"],
                                    a["g1"], a["D"], a["fmt"], a["codes"], a["csb"],
                                    a["csk"], a["scales"], a["ssb"], a["ssk"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), E_UNSUPPORTED),
    (dict(fmt=3), E_UNSUPPORTED),
    (dict(g1=-1), E_SHAPE),
    (dict(g0=5, g1=4), E_SHAPE),
    (dict(B=-1), E_SHAPE),
    (dict(raw=0), E_NULL),
    (dict(scales=0), E_NULL),
    (dict(fmt=2, scales=0, csk=256, g0=3, g1=3), OK),   # BF16 keys need no scales
    (dict(rst=-128), E_STRIDE),
    (dict(raw=A + 8), E_ALIGN),
    (dict(rst=132), E_ALIGN),
    (dict(fmt=2, csk=264), E_ALIGN),        # BF16 rows are 16-byte aligned
    (dict(fmt=1, csk=132), E_ALIGN),
    (dict(g0=7, g1=7), OK),
])
def test_index_keys_build_refusals(L, kw, status):
    assert ikb(L, **kw) == status
    if status != OK:
        assert L.fp8kv_last_error().decode()


def pf(L, **kw):
    a = dict(q=A, qsb=1 << 20, qst=4096, qsh=128, qdt=BF16, kc=A, vc=A, css=1024,
             csh=128, ks=A, vs=A, sss=1, ssh=1 << 20, S=1 << 20, bt=A, bts=2048,
             cl=A, ql=A, B=1, Q=4096, Hq=32, H=8, D=128, bs=16, scale=0.088,
             maxc=32768, out=A, osb=1 << 20, ost=4096, osh=128, odt=BF16)
    a.update(kw)
    return L.fp8kv_prefill_attn_fp8(
        a["q"], a["qsb"], a["qst"], a["qsh"], a["qdt"], a["kc"], a["vc"], a["css"],
        a["csh"], a["ks"], a["vs"], a["sss"], a["ssh"], a["S"], a["bt"], a["bts"],
        a["cl"], a["ql"], a["B"], a["Q"], a["Hq"], a["H"], a["D"], a["bs"],
        ctypes.c_float(a["scale"]), a["maxc"], a["out"], a["osb"], a["ost"], a["osh"],
        a["odt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), E_UNSUPPORTED),
    (dict(qdt=FP32), E_UNSUPPORTED),
    (dict(odt=FP16), E_UNSUPPORTED),
    (dict(Hq=24, H=8), E_UNSUPPORTED),   # group 3 does not divide 16
    (dict(Hq=64, H=2), E_UNSUPPORTED),   # group 32
    (dict(Hq=30), E_SHAPE),
    (dict(bs=8), E_UNSUPPORTED),
    (dict(B=-1), E_SHAPE),
    (dict(ql=0), E_NULL),
    (dict(out=0), E_NULL),
    (dict(qst=-8), E_STRIDE),
    (dict(q=A + 8), E_ALIGN),
    (dict(out=A + 4), E_ALIGN),
    (dict(osh=101), E_ALIGN),            # bf16 rows must start on 8 bytes
    (dict(Q=0), OK),
])
def test_prefill_refusals(L, kw, status):
    assert pf(L, **kw) == status
    if status != OK:
        assert L.fp8kv_last_error().decode()


def qsu(L, **kw):
    a = dict(k=A, kst=6144, ksh=128, v=A + 8192, vst=6144, vsh=128,
             dtype=BF16, T=16, H=8, D=128, slots=A, kc=A, vc=A, css=1024,
             csh=128, S=1 << 20, fmt=0)
    a.update(kw)
    return L.fp8kv_kv_quant_scatter_unscaled(
        a["k"], a["kst"], a["ksh"], a["v"], a["vst"], a["vsh"], a["dtype"],
        a["T"], a["H"], a["D"], a["slots"], a["kc"], a["vc"], a["css"],
        a["csh"], a["S"], a["fmt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=2), E_UNSUPPORTED),
    (dict(fmt=-1), E_UNSUPPORTED),
    (dict(D=96), E_UNSUPPORTED),
    (dict(kc=0), E_NULL),
    (dict(slots=0), E_NULL),
    (dict(kst=-1), E_STRIDE),
    (dict(kc=A + 8), E_ALIGN),
    (dict(T=0), OK),                      # nothing to do, nothing launched
])
def test_unscaled_quant_scatter_refusals(L, kw, status):
    assert qsu(L, **kw) == status
    if status != OK:
        assert L.fp8kv_last_error().decode()


def test_unscaled_decode_refusals(L):
    def call(**kw):
        a = dict(q=A, kc=A, vc=A, css=1024, csh=128, S=1 << 20, bt=A, bts=64, cl=A,
                 B=4, R=1, Hq=32, Hkv=8, D=128, bs=16, scale=0.088, nr=16, maxc=1024,
                 ws=A, wsb=1 << 30, fmt=1)
        a.update(kw)
        return L.fp8kv_paged_decode_partials_unscaled(
            a["q"], 8 * 32 * 128, 32 * 128, 128, BF16, a["kc"], a["vc"], a["css"], a["csh"],
            a["S"], a["bt"], a["bts"], a["cl"], a["B"], a["R"], a["Hq"], a["Hkv"], a["D"],
            a["bs"], a["scale"], a["nr"], a["maxc"], a["ws"], a["wsb"], a["fmt"], None)
    assert call(fmt=2) == E_UNSUPPORTED
    assert call(kc=0) == E_NULL
    assert call(D=96) == E_UNSUPPORTED
    assert call(wsb=16) == E_WORKSPACE
    assert call(B=0) == OK


def test_zero_size_calls_accept_null_pointers(L):
    """Nothing to do: status OK with every pointer NULL, no device touched
    (explicit num_ranges, so no device query either); a bad shape or dtype
    is still refused."""
    assert qs(L, T=0, k=0, v=0, slots=0, kc=0, vc=0, ks=0, vs=0) == OK
    assert qs(L, T=0, D=96, k=0, v=0, slots=0, kc=0, vc=0, ks=0, vs=0) == E_UNSUPPORTED
    for fn in ("fp8kv_paged_decode_attn_fp8", "fp8kv_paged_decode_partials"):
        assert dec(L, fn=fn, B=0, q=0, kc=0, vc=0, ks=0, vs=0, bt=0, cl=0, ws=0,
                   out=0) == OK
        assert dec(L, fn=fn, B=0, D=96, q=0, kc=0, vc=0, ks=0, vs=0, bt=0, cl=0, ws=0,
                   out=0) == E_UNSUPPORTED
    assert sdec(L, B=0, q=0, kc=0, vc=0, ks=0, vs=0, bt=0, bv=0, cl=0, ws=0,
                out=0) == OK
    assert L.fp8kv_paged_decode_merge(0, 1, 32, 8, 128, 384, None, 0, None, 0, 0, 0,
                                      BF16, None) == OK


def noalloc(L, **kw):
    """fp8kv_paged_decode_attn_fp8_noalloc with the arguments of dec() minus
    the workspace."""
    a = dict(q=A, qsb=4096, qsr=4096, qsh=128, qdt=BF16, kc=A, vc=A,
             css=1024, csh=128, ks=A, vs=A, sss=1, ssh=1 << 20, S=1 << 20,
             bt=A, bts=2048, cl=A, B=64, R=1, Hq=32, H=8, D=128, bs=16,
             scale=0.088, P=384, maxc=32768, out=A, osb=4096, osr=4096, osh=128,
             odt=BF16)
    a.update(kw)
    return L.fp8kv_paged_decode_attn_fp8_noalloc(
        a["q"], a["qsb"], a["qsr"], a["qsh"], a["qdt"], a["kc"], a["vc"], a["css"],
        a["csh"], a["ks"], a["vs"], a["sss"], a["ssh"], a["S"], a["bt"], a["bts"],
        a["cl"], a["B"], a["R"], a["Hq"], a["H"], a["D"], a["bs"],
        ctypes.c_float(a["scale"]), a["P"], a["maxc"], a["out"], a["osb"], a["osr"],
        a["osh"], a["odt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), E_UNSUPPORTED),
    (dict(R=5), E_UNSUPPORTED),
    (dict(P=-1), E_SHAPE),
    (dict(P=1 << 14), E_WORKSPACE),      # 64 + 16383 pieces x 8 heads x 4 rows x 512 B > 16 MiB
    (dict(B=40000, P=64), E_WORKSPACE),
    (dict(B=0, q=0, kc=0, vc=0, ks=0, vs=0, bt=0, cl=0, out=0), OK),
])
def test_noalloc_decode_refusals(L, kw, status):
    """The entry point that allocates nothing refuses sizes whose partials
    exceed the library's scratch (and everything the workspace call
    refuses) before it touches any device; nothing to do is OK."""
    assert noalloc(L, **kw) == status
    if status == E_WORKSPACE:
        assert "scratch" in L.fp8kv_last_error().decode()


def test_noalloc_scratch_limit_covers_the_bench_workloads(L):
    """16 MiB holds the partials of the decode workload (64 requests, Hq 32
    / Hkv 8, 128 ranges per KV head) and of the long-context verify
    workload (4 requests, 4 rows, Hq 16 / Hkv 4, 256 ranges per KV head)."""
    text = open(HEADER).read()
    limit = int(eval(re.search(r"#define FP8KV_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                               text).expand(r"\1 << \2")))
    assert limit == 16 << 20
    assert L.fp8kv_paged_decode_workspace_bytes(64, 1, 32, 8, 128, 128) <= limit
    assert L.fp8kv_paged_decode_workspace_bytes(4, 4, 16, 4, 128, 256) <= limit


def append(L, fn="fp8kv_paged_decode_append_attn_fp8", **kw):
    """The append calls with the arguments of dec() plus the new rows."""
    a = dict(q=A, qsb=4096, qsr=4096, qsh=128, qdt=BF16, kn=A, knb=1024, knr=1024,
             knh=128, vn=A, vnb=1024, vnr=1024, vnh=128, ndt=BF16, kc=A, vc=A,
             css=1024, csh=128, ks=A, vs=A, sss=1, ssh=1 << 20, S=1 << 20,
             bt=A, bts=2048, cl=A, B=64, R=1, Hq=32, H=8, D=128, bs=16,
             scale=0.088, P=384, maxc=32768, ws=A, wsb=1 << 34, out=A,
             osb=4096, osr=4096, osh=128, odt=BF16)
    a.update(kw)
    args = [a["q"], a["qsb"], a["qsr"], a["qsh"], a["qdt"], a["kn"], a["knb"], a["knr"],
            a["knh"], a["vn"], a["vnb"], a["vnr"], a["vnh"], a["ndt"], a["kc"], a["vc"],
            a["css"], a["csh"], a["ks"], a["vs"], a["sss"], a["ssh"], a["S"], a["bt"],
            a["bts"], a["cl"], a["B"], a["R"], a["Hq"], a["H"], a["D"], a["bs"],
            ctypes.c_float(a["scale"]), a["P"], a["maxc"], a["ws"], a["wsb"]]
    if fn == "fp8kv_paged_decode_append_partials":
        return getattr(L, fn)(*args, None)
    return getattr(L, fn)(*args, a["out"], a["osb"], a["osr"], a["osh"], a["odt"], None)


@pytest.mark.parametrize("fn", ["fp8kv_paged_decode_append_attn_fp8",
                                "fp8kv_paged_decode_append_partials"])
@pytest.mark.parametrize("kw,status", [
    (dict(ndt=FP16), E_UNSUPPORTED),
    (dict(ndt=FP32), E_UNSUPPORTED),
    (dict(kn=0), E_NULL),
    (dict(vn=0), E_NULL),
    (dict(knr=-1024), E_STRIDE),
    (dict(vnh=-128), E_STRIDE),
    (dict(kn=A + 8), E_ALIGN),           # rows on 16-byte boundaries at head_dim 128
    (dict(vnb=1028), E_ALIGN),
    (dict(D=64, knh=66), E_ALIGN),       # 8-byte boundaries at head_dim 64 (stride in bf16)
    (dict(D=96), E_UNSUPPORTED),
    (dict(R=5), E_UNSUPPORTED),
    (dict(ws=0), E_WORKSPACE),
    (dict(B=0, q=0, kn=0, vn=0, kc=0, vc=0, ks=0, vs=0, bt=0, cl=0, ws=0, out=0), OK),
])
def test_append_refusals(L, fn, kw, status):
    """The append calls refuse bad new rows (dtype, NULL, strides,
    alignment) and everything the decode refuses, before enqueueing."""
    assert append(L, fn, **kw) == status
    if status != OK:
        assert L.fp8kv_last_error().decode()
