"""GPU parity of the unscaled E4M3 / E5M2 cache ("feat(dsa): implement fp8
KV cache (e4m3) with a bf16 indexer cache", sglang-jax #1776: K/V cast to
the cache dtype with no scale).

Bar: the stored codes equal the oracle's, byte for byte (every finite bf16
value, strided K/V slices, placement); attention over the cache is within
max-abs 2e-3 / rel-L2 1e-3 of the oracle's unit-scale attention on the same
codes, and the bf16 output is the RNE of the same kernel's fp32 output."""
import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import SENTINEL, assert_attn_close, bf16_bits, bf16_rne, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMTS = [(fk.CODES_E4M3, oracle.E4M3), (fk.CODES_E5M2, oracle.E5M2)]


def dev_cache(S, H, D):
    kc = torch.full((S, H, D), SENTINEL, dtype=torch.uint8, device=DEV)
    return kc, torch.full_like(kc, SENTINEL)


def host_scatter(ofmt, k, v, slots, S):
    T, H, D = k.shape
    kc = np.full((S, H, D), SENTINEL, np.uint8)
    vc = np.full_like(kc, SENTINEL)
    oracle.kv_scatter_unscaled_bf16(ofmt, bf16_bits(k), bf16_bits(v),
                                    slots.cpu().numpy().astype(np.int64), kc, vc)
    return kc, vc


@pytest.mark.parametrize("cf,ofmt", FMTS)
@pytest.mark.parametrize("D", [64, 128])
def test_every_finite_bf16_value(cf, ofmt, D):
    """All 65,536 bf16 bit patterns except NaN and inf, as K and (reversed)
    as V: in-range values round to nearest even, the rest saturate."""
    bits = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    x = bits[torch.isfinite(bits.float())]
    n = x.numel() // D * D
    k = x[:n].reshape(-1, 1, D).contiguous()
    v = k.flip(0).contiguous()
    T = k.shape[0]
    slots = torch.randperm(2 * T, generator=synth.gen(60))[:T]
    log(f"unscaled fmt={cf} D={D}: {T} rows")
    kc, vc = dev_cache(2 * T, 1, D)
    fk.kv_quant_scatter_unscaled(k.to(DEV), v.to(DEV), slots.to(DEV), kc, vc, cf)
    torch.cuda.synchronize()
    rk, rv = host_scatter(ofmt, k, v, slots, 2 * T)
    assert np.array_equal(kc.cpu().numpy(), rk)
    assert np.array_equal(vc.cpu().numpy(), rv)


@pytest.mark.parametrize("cf,ofmt", FMTS)
def test_strided_slices_and_skipped_slots(cf, ofmt):
    """K and V as strided column slices of a fused qkv (the prefill-chunk
    recipe, 512 tokens), padding and out-of-range slot ids skipped."""
    c = synth.prefill_chunk(seed=61, tokens=512, num_slots=4096)
    slots = c.slot_ids.clone()
    slots[5] = -1
    slots[9] = 4096 + 7
    kc, vc = dev_cache(4096, 8, 128)
    qkv = c.qkv.to(DEV)
    T = qkv.shape[0]
    kv = qkv[:, 32 * 128:40 * 128].view(T, 8, 128)
    vv = qkv[:, 40 * 128:48 * 128].view(T, 8, 128)
    fk.kv_quant_scatter_unscaled(kv, vv, slots.to(DEV), kc, vc, cf)
    torch.cuda.synchronize()
    rk, rv = host_scatter(ofmt, c.k_view(), c.v_view(), slots, 4096)
    assert np.array_equal(kc.cpu().numpy(), rk)
    assert np.array_equal(vc.cpu().numpy(), rv)


def run_unscaled(case, kc, vc, cf, *, ranges=0, out_dtype=torch.float32):
    L = case.layout
    return fk.paged_decode_attn_unscaled(
        case.q.to(DEV), kc, vc, L.block_tables.to(DEV), L.context_lens.to(DEV),
        num_kv_heads=case.num_kv_heads, block_size=L.block_size,
        softmax_scale=case.softmax_scale, max_context=int(L.context_lens.max()),
        code_format=cf, num_ranges=ranges, out_dtype=out_dtype)


@pytest.mark.parametrize("cf,ofmt", FMTS)
@pytest.mark.parametrize("lens,Hq,Hkv,D,bs,rows,ranges", [
    ([1, 31, 700, 3000, 77], 8, 2, 128, 16, 1, 0),
    ([5, 900, 4000], 16, 4, 128, 64, 4, 7),      # 4 verify rows x 4 heads
    ([700, 129, 2], 16, 4, 64, 16, 2, 5),        # head_dim 64
    ([600, 333], 8, 8, 128, 48, 1, 3),           # MHA, block size 48
])
def test_decode_matches_oracle(cf, ofmt, lens, Hq, Hkv, D, bs, rows, ranges):
    case = synth.decode_case(lens, Hq, Hkv, D, bs, rows=rows, seed=62 + bs,
                             k_outlier_frac=0.005)
    L = case.layout
    S = L.num_slots
    log(f"unscaled decode fmt={cf} lens={lens} R={rows} D={D} bs={bs}")
    kc, vc = dev_cache(S, Hkv, D)
    fk.kv_quant_scatter_unscaled(case.k.to(DEV), case.v.to(DEV), L.token_slots.to(DEV),
                                 kc, vc, cf)
    out = run_unscaled(case, kc, vc, cf, ranges=ranges)
    torch.cuda.synchronize()
    hk, hv = kc.cpu().numpy(), vc.cpu().numpy()
    rk, rv = host_scatter(ofmt, case.k, case.v, L.token_slots, S)
    assert np.array_equal(hk, rk) and np.array_equal(hv, rv)
    ones = np.ones((S, Hkv), np.float32)
    ref = oracle.paged_decode_attn(bf16_bits(case.q), hk, hv, ones, ones,
                                   L.block_tables.numpy(), L.context_lens.numpy(), Hkv,
                                   bs, case.softmax_scale, fmt=ofmt)
    assert_attn_close(out.cpu().numpy(), ref, f"unscaled fmt {cf}")
    ob = run_unscaled(case, kc, vc, cf, ranges=ranges, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(ob, bf16_rne(out)), "bf16 output is not RNE of fp32"


def test_partials_then_merge_equal_fused():
    case = synth.decode_case([300, 1000], 16, 4, 128, 16, rows=1, seed=66)
    L = case.layout
    kc, vc = dev_cache(L.num_slots, 4, 128)
    fk.kv_quant_scatter_unscaled(case.k.to(DEV), case.v.to(DEV), L.token_slots.to(DEV),
                                 kc, vc, fk.CODES_E5M2)
    fused = run_unscaled(case, kc, vc, fk.CODES_E5M2, ranges=9)
    q = case.q.to(DEV)
    ws = fk.paged_decode_partials_unscaled(
        q, kc, vc, L.block_tables.to(DEV), L.context_lens.to(DEV), num_kv_heads=4,
        block_size=16, softmax_scale=case.softmax_scale,
        max_context=int(L.context_lens.max()), code_format=fk.CODES_E5M2, num_ranges=9)
    out = torch.empty(q.shape, device=DEV)
    fk.paged_decode_merge(ws, out, rows=1, num_q_heads=16, num_kv_heads=4, num_ranges=9)
    torch.cuda.synchronize()
    assert torch.equal(out, fused)
