"""GPU parity of fp8kv_kv_quant_scatter against the oracle: codes, scales
and slot placement bit-exact, every other byte of the pool untouched."""
import os

import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import (DevCache, SENTINEL, SCALE_SENTINEL, bf16_bits,
                       host_empty_like, log)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_both(k, v, slots, S, layout="head_major"):
    """GPU scatter into a sentinel pool and the oracle into a host copy of
    the same pool; returns (gpu arrays, oracle arrays)."""
    H, D = k.shape[1], k.shape[2]
    dc = DevCache(S, H, D, DEV, layout)
    fk.kv_quant_scatter(k.to(DEV) if not k.is_cuda else k,
                        v.to(DEV) if not v.is_cuda else v,
                        slots.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale,
                        dc.v_scale)
    torch.cuda.synchronize()
    ref = host_empty_like(dc)
    oracle.kv_quant_scatter_bf16(bf16_bits(k), bf16_bits(v),
                                 slots.cpu().numpy(), *ref)
    return dc.host(), ref


def assert_same(got, ref, what):
    names = ("k_cache", "v_cache", "k_scale", "v_scale")
    for n, g, r in zip(names, got, ref):
        if n.endswith("scale"):
            bad = np.flatnonzero(g.view(np.uint32) != r.view(np.uint32))
        else:
            bad = np.flatnonzero(g != r)
        assert bad.size == 0, f"{what}: {n} differs at {bad.size} places, e.g. {bad[:4]}"


@pytest.mark.parametrize("layout", ["head_major", "interleaved", "slot_major"])
def test_tiny_case_bit_exact(layout):
    case = synth.tiny_case(0)
    log(f"tiny quant-scatter layout={layout}")
    got, ref = run_both(case.k, case.v, case.layout.token_slots,
                        case.layout.num_slots, layout)
    assert_same(got, ref, "tiny")
    zt, zh = case.notes["zero_row"]
    slot = int(case.layout.token_slots[zt])
    assert got[2][slot, zh] == 0.0 and got[3][slot, zh] == 0.0


def test_prefill_chunk_full_size_bit_exact():
    """4096-token fused qkv, K/V strided slices, 4096 random slots out of a
    1,048,576-slot pool: every written row against the oracle, every other
    pool byte still the sentinel."""
    ch = synth.prefill_chunk(seed=1, device=DEV)
    k, v = ch.k_view(), ch.v_view()
    assert k.stride(0) == 6144 and not k.is_contiguous()
    log("prefill chunk 4096 x 8 x 128, pool 1M slots")
    dc = DevCache(ch.num_slots, 8, 128, DEV, "head_major")
    fk.kv_quant_scatter(k, v, ch.slot_ids, dc.k_cache, dc.v_cache,
                        dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    T = k.shape[0]
    # oracle on a compact pool whose slot t is the chunk's token t
    kc = np.full((T, 8, 128), SENTINEL, np.uint8)
    vc = kc.copy()
    ks = np.full((T, 8), SCALE_SENTINEL, np.float32)
    vs = ks.copy()
    oracle.kv_quant_scatter_bf16(bf16_bits(k), bf16_bits(v),
                                 np.arange(T, dtype=np.int64), kc, vc, ks, vs)
    sl = ch.slot_ids
    assert np.array_equal(dc.k_cache[sl].cpu().numpy(), kc)
    assert np.array_equal(dc.v_cache[sl].cpu().numpy(), vc)
    assert np.array_equal(dc.k_plane[:, sl].t().cpu().numpy().view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(dc.v_plane[:, sl].t().cpu().numpy().view(np.uint32), vs.view(np.uint32))
    # nothing else in the pool changed
    touched = torch.zeros(ch.num_slots, dtype=torch.bool, device=DEV)
    touched[sl] = True
    assert int((dc.k_cache[~touched] != SENTINEL).sum()) == 0
    assert int((dc.v_cache[~touched] != SENTINEL).sum()) == 0
    assert int((dc.k_plane[:, ~touched] != SCALE_SENTINEL).sum()) == 0
    assert int((dc.v_plane[:, ~touched] != SCALE_SENTINEL).sum()) == 0
    # the V distribution really has the x100 and zero rows
    assert int((ks == 0).sum()) == 0 and int((vs == 0).sum()) > 0


def test_strided_pitch_scenario_bit_exact():
    """K a view of the fused qkv slice (pitch 1152), V materialized by a
    clamp (pitch 384): 0 of 3072 codes may differ, in K and in V."""
    k, v = synth.strided_pitch_scenario()
    kd, vd = k.to(DEV), None
    # rebuild the same two views on the device
    qkv = torch.empty((k.shape[0], 3 * 384), dtype=torch.bfloat16, device=DEV)
    qkv[:, 384:768] = k.reshape(k.shape[0], 384).to(DEV)
    kd = qkv[:, 384:768].view(k.shape)
    vd = v.to(DEV).contiguous()
    assert kd.stride(0) == 1152 and vd.stride(0) == 384
    slots = torch.arange(k.shape[0], dtype=torch.int64)
    got, ref = run_both(kd, vd, slots, k.shape[0])
    assert_same(got, ref, "v-pitch scenario")
    # and the swap: K dense, V the strided view
    got, ref = run_both(vd, kd, slots, k.shape[0])
    assert_same(got, ref, "swapped pitches")


def edge_rows(D=128):
    g = synth.gen(5)
    rows = [torch.zeros(D), -torch.zeros(D)]
    x = torch.randn(D, generator=g)
    rows += [x, x * 1e-30, x * 1e-38, x / x.abs().max() * 3e38, -x]
    one = torch.zeros(D)
    one[17] = 2.0 ** -133                       # smallest bf16 subnormal
    rows.append(one)
    spike = torch.randn(D, generator=g) * 0.01
    spike[3] = 50.0
    rows.append(spike)
    # midpoint-rich row: values on e4m3 rounding boundaries of amax 448
    mid = torch.tensor(oracle.decode(np.arange(0, 0x7E, dtype=np.uint8)),
                       dtype=torch.float32)
    mid = torch.cat([mid[:D // 2], -mid[:D // 2]])
    mid[0] = 448.0
    rows.append(mid)
    out = torch.stack(rows).to(torch.bfloat16)
    assert torch.isfinite(out.float()).all()      # non-finite input is out of contract
    return out


def test_edge_rows_bit_exact():
    x = edge_rows()
    n = x.shape[0]
    k = x.view(n, 1, 128)
    v = x.flip(0).contiguous().view(n, 1, 128)
    got, ref = run_both(k, v, torch.arange(n, dtype=torch.int64), n)
    assert_same(got, ref, "edge rows")


def test_quotient_sweep_bit_exact():
    """For 96 row maxima spread over the bf16 exponent range, rows holding
    every bf16 value of magnitude <= the maximum (both signs): the
    fp32 quotient and its E4M3 rounding must match the oracle everywhere."""
    D = 128
    allb = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    g = synth.gen(11)
    amax_bits = torch.randint(0x0080, 0x7F80, (96,), generator=g)
    rows = []
    for ab in amax_bits.tolist():
        a = torch.tensor([ab], dtype=torch.int16).view(torch.bfloat16).float()
        vals = allb[allb <= a]
        vals = vals[torch.randperm(vals.numel(), generator=g)[:4096]]
        vals = torch.cat([vals, -vals])
        pad = (-vals.numel()) % (D - 1)
        vals = torch.cat([vals, torch.zeros(pad)])
        chunk = vals.view(-1, D - 1)
        chunk = torch.cat([a.expand(chunk.shape[0], 1), chunk], dim=1)
        rows.append(chunk)
    x = torch.cat(rows).to(torch.bfloat16)
    n = x.shape[0]
    log(f"quotient sweep: {n} rows")
    k = x.view(n, 1, D)
    got, ref = run_both(k, k, torch.arange(n, dtype=torch.int64), n)
    assert_same(got, ref, "quotient sweep")


def test_slot_ids_out_of_range_are_skipped():
    g = synth.gen(4)
    T, H, D, S = 64, 2, 64, 128
    k = synth.normal_bf16((T, H, D), g)
    v = synth.normal_bf16((T, H, D), g)
    slots = torch.randperm(S, generator=g)[:T].to(torch.int64)
    slots[::5] = -1
    slots[3] = S
    slots[4] = 1 << 40
    got, ref = run_both(k, v, slots, S, "slot_major")
    assert_same(got, ref, "skips")


def test_graph_capture_replays_with_new_slots():
    """One launch captured in a graph; slot ids and inputs change in place
    between replays, with eager work between them; every replay must equal
    the oracle."""
    g = synth.gen(8)
    T, H, D, S = 256, 8, 128, 4096
    k = synth.normal_bf16((T, H, D), g).to(DEV)
    v = synth.normal_bf16((T, H, D), g).to(DEV)
    slots = torch.randperm(S, generator=g)[:T].to(torch.int64).to(DEV)
    dc = DevCache(S, H, D, DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fk.kv_quant_scatter(k, v, slots, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fk.kv_quant_scatter(k, v, slots, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale)
    for rep in range(3):
        dc.k_cache.fill_(SENTINEL)
        dc.v_cache.fill_(SENTINEL)
        dc.k_plane.fill_(SCALE_SENTINEL)
        dc.v_plane.fill_(SCALE_SENTINEL)
        slots.copy_(torch.randperm(S, generator=g)[:T].to(torch.int64))
        k.copy_(synth.normal_bf16((T, H, D), g))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = host_empty_like(dc)
        oracle.kv_quant_scatter_bf16(bf16_bits(k), bf16_bits(v),
                                     slots.cpu().numpy(), *ref)
        assert_same(dc.host(), ref, f"replay {rep}")


def every_pair_rows(D=128):
    """Rows covering every (positive bf16 row maximum a, bf16 x in [0, a])
    pair: element 0 of each row is a, the other D-1 elements walk x through
    0 .. a (zero-padded at the end of each a). Built on the device."""
    amax = torch.arange(1, 0x7F80, device=DEV, dtype=torch.int64)   # bit patterns
    per = D - 1
    nrows = (amax + 1 + per - 1) // per
    a_of_row = torch.repeat_interleave(amax, nrows)
    first = torch.cumsum(nrows, 0) - nrows                           # first row of each a
    row_in_a = torch.arange(a_of_row.numel(), device=DEV) - torch.repeat_interleave(first, nrows)
    xb = row_in_a[:, None] * per + torch.arange(per, device=DEV)[None, :]
    xb = torch.where(xb <= a_of_row[:, None], xb, torch.zeros_like(xb))
    bits = torch.cat([a_of_row[:, None], xb], dim=1).to(torch.int32).to(torch.int16)
    return bits.view(torch.bfloat16)


def test_every_bf16_pair_bit_exact():
    """All 532,701,119 (row maximum, element) bf16 pairs through the kernel:
    K rows as built, V rows negated; K codes and scales against the oracle,
    V against K by the encoding's sign symmetry."""
    x = every_pair_rows()
    n = x.shape[0]
    log(f"every-pair rows: {n}")
    k = x.view(n, 1, 128)
    v = (-x.float()).to(torch.bfloat16).view(n, 1, 128)
    dc = DevCache(n, 1, 128, DEV, "slot_major", sentinel=False)
    fk.kv_quant_scatter(k, v, torch.arange(n, device=DEV, dtype=torch.int64),
                        dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(dc.v_cache, dc.k_cache | 0x80)
    assert torch.equal(dc.v_plane, dc.k_plane)
    threads = min(16, os.cpu_count() or 1)
    codes, scales = oracle.quantize_rows_bf16(bf16_bits(x), threads=threads)
    got = dc.k_cache.view(n, 128).cpu().numpy()
    bad = np.flatnonzero((got != codes).any(axis=1))
    assert bad.size == 0, f"{bad.size} rows differ, e.g. row {bad[:3]}"
    assert np.array_equal(dc.k_plane.view(n).cpu().numpy().view(np.uint32),
                          scales.view(np.uint32))
