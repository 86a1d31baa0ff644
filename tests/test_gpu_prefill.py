"""GPU parity of fp8kv_prefill_attn_fp8 (chunked-prefill attention over the
FP8 cache) against the oracle's attention on the same dequantized cache:
a chunk of C query tokens at the end of a request is the oracle's decode
attention with R = C causal rows.

Bar: as the decode -- fp32 output within max-abs 2e-3 and rel-L2 1e-3,
bf16 output equal to the RNE of the same kernel's fp32 output."""
import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import (assert_attn_close, assert_attn_close_scaled, bf16_bits,
                       bf16_rne, cache_case, compact_host_cache, log)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_prefill(case, dc, q_lens=None, out_dtype=torch.float32, out=None):
    L = case.layout
    B = case.q.shape[0]
    ql = torch.full((B,), case.q.shape[1], dtype=torch.int32) if q_lens is None else q_lens
    return fk.prefill_attn_fp8(
        case.q.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
        L.block_tables.to(DEV), L.context_lens.to(DEV), ql.to(DEV),
        num_kv_heads=case.num_kv_heads, block_size=L.block_size,
        softmax_scale=case.softmax_scale, max_context=int(L.context_lens.max()),
        out_dtype=out_dtype, out=out)


def oracle_prefill(case, host, rows=None):
    kc, vc, ks, vs = host
    L = case.layout
    return oracle.paged_decode_attn(bf16_bits(case.q), kc, vc, ks, vs,
                                    L.block_tables.numpy(), L.context_lens.numpy(),
                                    case.num_kv_heads, L.block_size,
                                    case.softmax_scale, rows=rows)


@pytest.mark.parametrize("lens,C,Hq,Hkv,D,bs", [
    ([100, 2000], 16, 32, 8, 128, 16),     # one query block per (request, head)
    ([37, 1500, 700], 37, 32, 8, 128, 16), # ragged chunk; a request that is all chunk
    ([900, 1300], 130, 8, 8, 128, 64),     # MHA (16 tokens per wave), bs 64
    ([600, 800], 45, 16, 2, 128, 32),      # GQA 8
    ([500, 777], 64, 16, 4, 64, 16),       # head_dim 64
    ([700, 1000], 40, 16, 4, 128, 48),     # block size 48 (division page walk)
    ([300, 420], 33, 32, 2, 128, 16),      # GQA 16 (one token per 16-row tile)
    ([300, 420], 21, 16, 8, 64, 16),       # GQA 2, head_dim 64
])
def test_chunk_matches_oracle(lens, C, Hq, Hkv, D, bs):
    case = synth.decode_case(lens, Hq, Hkv, D, bs, rows=C, seed=C + bs)
    log(f"prefill lens={lens} C={C} Hq={Hq} Hkv={Hkv} D={D} bs={bs}")
    dc = cache_case(case, DEV)
    out = run_prefill(case, dc)
    torch.cuda.synchronize()
    ref = oracle_prefill(case, dc.host())
    assert_attn_close(out.cpu().numpy(), ref, f"C={C}")
    ob = run_prefill(case, dc, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(ob, bf16_rne(out)), "bf16 output is not RNE of fp32"


def test_many_query_blocks_one_key_group():
    """Enough query blocks (20 requests x 8 KV heads x 5 blocks of 32
    tokens = 800 workgroups, more than one per CU on a 256-CU GPU) that each
    block's keys stay in one group of 4 waves; the small chunks above run
    two key groups per block, merged by log-sum-exp. Both meet the bar."""
    lens = [300 + 37 * i for i in range(20)]
    case = synth.decode_case(lens, 32, 8, 128, 16, rows=160, seed=160)
    log(f"prefill one key group: {len(lens)} requests, C=160")
    dc = cache_case(case, DEV)
    out = run_prefill(case, dc)
    torch.cuda.synchronize()
    ref = oracle_prefill(case, dc.host())
    assert_attn_close(out.cpu().numpy(), ref, "one key group")


def test_unread_scales_do_not_move_the_range():
    """One key group (800 workgroups): every scale the kernel must not read
    -- past each request's context in its last block, and in blocks no
    request uses -- set to 2^100. The kernel fixes its P' range exponent
    from the scales of the keys it reads; had it taken one of these, P'
    would underflow and the output would collapse towards zero."""
    lens = [300 + 37 * i for i in range(20)]
    case = synth.decode_case(lens, 32, 8, 128, 16, rows=160, seed=161)
    L = case.layout
    dc = cache_case(case, DEV)
    readable = torch.zeros(L.num_slots, dtype=torch.bool)
    for b, n in enumerate(L.context_lens.tolist()):
        for i in range((n + 15) // 16):
            blk = int(L.block_tables[b, i])
            readable[blk * 16: blk * 16 + min(16, n - i * 16)] = True
    far = readable.logical_not().to(DEV)
    log(f"prefill unread scales: {int(far.sum())} of {far.numel()} slots set to 2^100")
    dc.v_scale[far] = 2.0 ** 100
    dc.k_scale[far] = 2.0 ** 100
    out = run_prefill(case, dc)
    torch.cuda.synchronize()
    ref = oracle_prefill(case, dc.host())
    assert_attn_close(out.cpu().numpy(), ref, "unread scales")


def test_value_ranges_and_growing_scores():
    """Mixed V magnitudes (rows x1e-3, x100, zero, ~1e-33) with 1% K outlier
    channels, and K rows whose size grows along the sequence, so a row's
    running maximum moves many times, also by more than the kernel's lazy
    maximum slack."""
    case = synth.decode_case([900, 1500], 16, 4, 128, 16, rows=70, seed=98,
                             k_outlier_frac=0.01)
    T, H = case.k.shape[0], case.num_kv_heads
    g = torch.Generator().manual_seed(99)
    grow = torch.linspace(0.2, 6.0, T)[:, None, None]
    case.k = (case.k.float() * grow).to(torch.bfloat16)
    mult = torch.tensor([1.0, 1e-3, 100.0, 0.0])[torch.randint(0, 4, (T, H), generator=g)]
    vf = case.v.float() * mult[..., None]
    vf[torch.rand(T, H, generator=g) < 0.01] *= 1e-33
    case.v = vf.to(torch.bfloat16)
    log("prefill value ranges / growing scores")
    dc = cache_case(case, DEV)
    out = run_prefill(case, dc)
    torch.cuda.synchronize()
    ref = oracle_prefill(case, dc.host())
    # V rows x100 put outputs in the hundreds: the bar in the output's units
    assert_attn_close_scaled(out.cpu().numpy(), ref, "value ranges")


def test_per_request_chunk_lengths_and_untouched_rows():
    case = synth.decode_case([400, 350, 90], 32, 8, 128, 16, rows=48, seed=70)
    dc = cache_case(case, DEV)
    ql = torch.tensor([48, 13, 0], dtype=torch.int32)
    out = torch.full(case.q.shape, 7.0, device=DEV)
    run_prefill(case, dc, q_lens=ql, out=out)
    torch.cuda.synchronize()
    host = dc.host()
    L = case.layout
    for b, n in enumerate(ql.tolist()):
        if n:
            # request b's chunk is its last n tokens: the oracle's n causal rows
            q = case.q[b:b + 1, :n].clone()
            ref = oracle.paged_decode_attn(bf16_bits(q), *host, L.block_tables[b:b + 1].numpy(),
                                           L.context_lens[b:b + 1].numpy(), 8, 16,
                                           case.softmax_scale)
            assert_attn_close(out[b, :n].cpu().numpy(), ref[0], f"request {b}, {n} tokens")
        assert torch.all(out[b, n:] == 7.0)


def test_prefill_workload_full_size_sampled():
    """A 4096-token chunk at the end of a 32,768-token request (Hq 32 / Hkv 8,
    D 128, bs 16); the oracle recomputes 64 sampled rows."""
    case = synth.prefill_attn_workload(seed=71, device=DEV)
    dc = cache_case(case, DEV)
    out = run_prefill(case, dc)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    host, bt, cl = compact_host_cache(case, dc, [0])
    g = torch.Generator().manual_seed(72)
    C, Hq = case.q.shape[1], case.q.shape[2]
    toks = torch.cat([torch.tensor([0, 1, C - 1]), torch.randint(0, C, (13,), generator=g)])
    heads = torch.randint(0, Hq, (16,), generator=g)
    rows = [(int(t) * Hq + int(hh)) for t in toks for hh in heads[:4]]
    ref = oracle.paged_decode_attn(bf16_bits(case.q), *host, bt, cl, case.num_kv_heads,
                                   case.layout.block_size, case.softmax_scale, rows=rows)
    got = out[0].reshape(-1, 128)[rows].cpu().numpy()
    assert_attn_close(got, ref, "prefill sampled")


def test_1k_chunk_two_key_groups_full_size_sampled():
    """The last 1024 tokens of the prefill workload's 32,768-token request
    as the chunk (the benchmark's 1024-row views of q and out): 256 query
    blocks, so each block's keys run in two key groups of about 500 tiles,
    a barrier every second tile, merged by log-sum-exp; the oracle
    recomputes 64 sampled rows."""
    case = synth.prefill_attn_workload(seed=71, device=DEV)
    dc = cache_case(case, DEV)
    L = case.layout
    C1 = 1024
    q1 = case.q[:, :C1]
    out = torch.full(q1.shape, 7.0, device=DEV)
    ql = torch.full((1,), C1, dtype=torch.int32)
    fk.prefill_attn_fp8(q1.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                        L.block_tables.to(DEV), L.context_lens.to(DEV), ql.to(DEV),
                        num_kv_heads=case.num_kv_heads, block_size=L.block_size,
                        softmax_scale=case.softmax_scale,
                        max_context=L.block_size * L.block_tables.shape[1], out=out)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    host, bt, cl = compact_host_cache(case, dc, [0])
    g = torch.Generator().manual_seed(73)
    Hq = q1.shape[2]
    toks = torch.cat([torch.tensor([0, 1, 31, 32, C1 - 1]), torch.randint(0, C1, (11,), generator=g)])
    heads = torch.randint(0, Hq, (4,), generator=g)
    rows = [(int(t) * Hq + int(hh)) for t in toks for hh in heads]
    log(f"prefill 1024-token chunk, {len(rows)} sampled rows")
    ref = oracle.paged_decode_attn(bf16_bits(q1.contiguous()), *host, bt, cl, case.num_kv_heads,
                                   L.block_size, case.softmax_scale, rows=rows)
    got = out[0].reshape(-1, 128)[rows].cpu().numpy()
    assert_attn_close(got, ref, "1024-token chunk sampled")
