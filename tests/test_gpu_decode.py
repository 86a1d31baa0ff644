"""GPU parity of fp8kv_paged_decode_attn_fp8 against the oracle run on the
same dequantized cache (the cache itself written by the GPU quantizer).

Bar: fp32 output within max-abs 2e-3 and rel-L2 1e-3 of the oracle; bf16
output equal, bit for bit, to the round-to-nearest-even of the same
kernel's fp32 output (same split).

The split into ranges is exercised from one range per KV head (one wave
walks every request) to many more ranges than tiles (most ranges empty, so
the merge must skip them)."""
import math

import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import (DevCache, assert_attn_close, assert_attn_close_scaled,
                       attn_errors, bf16_rne, cache_case, compact_host_cache,
                       log, oracle_decode, oracle_decode_requests, run_decode)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def check_case(case, ranges=0, layout="head_major", also_bf16=True,
               max_context=None):
    log(f"decode {case.name}: lens={case.layout.context_lens.tolist()[:6]} "
        f"R={case.rows} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} bs={case.layout.block_size} ranges={ranges} {layout}")
    dc = cache_case(case, DEV, layout)
    out = run_decode(case, dc, ranges=ranges, max_context=max_context)
    torch.cuda.synchronize()
    ref = oracle_decode(case, dc.host())
    assert_attn_close(out.cpu().numpy(), ref, case.name)
    if also_bf16:
        ob = run_decode(case, dc, ranges=ranges, out_dtype=torch.bfloat16,
                        max_context=max_context)
        torch.cuda.synchronize()
        assert torch.equal(ob, bf16_rne(out)), "bf16 output is not RNE of fp32"
    return dc, out, ref


def test_tiny_case():
    case = synth.tiny_case(0)
    check_case(case)


@pytest.mark.parametrize("ranges", [0, 1, 3, 7, 64, 5000])
def test_ragged_lengths_across_ranges(ranges):
    """198 tiles per KV head: one range, ranges spanning several requests,
    ranges inside one request, and 5000 ranges (most of them empty)."""
    case = synth.decode_case([1, 31, 33, 1000, 5000, 77], 8, 2, 128, 16,
                             rows=1, seed=3)
    check_case(case, ranges=ranges)


@pytest.mark.parametrize("layout", ["head_major", "interleaved", "slot_major"])
@pytest.mark.parametrize("bs", [16, 32, 48, 64, 128])
def test_block_sizes_and_scale_layouts(bs, layout):
    """Power-of-two block sizes take the shift/mask page walk, 48 the
    division path."""
    case = synth.decode_case([300, 1290, 64], 8, 4, 128, bs, rows=1, seed=bs)
    check_case(case, ranges=11, layout=layout)


@pytest.mark.parametrize("Hq,Hkv,rows", [
    (8, 8, 1),        # MHA
    (32, 2, 1),       # G = 16: the whole 16-row tile
    (24, 8, 1),       # G = 3
    (30, 6, 2),       # G = 5, 2 verify rows (10 rows), Hkv not a multiple of 4
    (36, 12, 1),      # Hkv 12: 3 workgroups per range on one XCD
    (7, 1, 2),        # one KV head, G = 7, 2 verify rows (14 rows)
])
def test_group_and_row_stacking(Hq, Hkv, rows):
    case = synth.decode_case([1, 50, 1300, 777], Hq, Hkv, 128, 16, rows=rows,
                             seed=100 + Hq + Hkv)
    check_case(case, ranges=0)


def test_head_dim_64():
    case = synth.decode_case([700, 129, 2], 16, 4, 64, 16, rows=2, seed=6)
    check_case(case, ranges=5)


@pytest.mark.parametrize("ranges", [0, 2, 33])
def test_verify_rows_causal(ranges):
    """4 verify rows x 4 query heads stacked into the 16-row tile; request
    lengths include one shorter than the row count (row 0 sees nothing)."""
    case = synth.decode_case([3, 4, 2000, 9000], 16, 4, 128, 64, rows=4,
                             seed=12, k_outlier_frac=0.005)
    _, out, _ = check_case(case, ranges=ranges)
    assert torch.all(out[0, 0] == 0)


def test_outliers_and_zero_rows():
    case = synth.decode_case([500, 2048], 8, 2, 128, 16, rows=1, seed=21)
    k = case.k.float()
    v = case.v.float()
    k[5] = 0.0
    v[6] = 0.0
    k[100, 1, 7] = 3000.0
    v[101, 0, 9] = -5000.0
    v[200:260] *= 1e-3
    case.k, case.v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    check_case(case, ranges=9)


def test_tiny_value_scales():
    """V rows of ~1e-33 (value scales below 2^-112): the fp16 range factor
    of P' sits at its floor and must be undone exactly."""
    case = synth.decode_case([300, 77], 8, 2, 128, 16, rows=1, seed=23)
    v = case.v.float() * 1e-33
    v[10:20] *= 1e30                      # a few ordinary rows as well
    case.v = v.to(torch.bfloat16)
    dc, out, ref = check_case(case, ranges=0)
    tiny = synth.decode_case([300, 77], 8, 2, 128, 16, rows=1, seed=23)
    tiny.v = (tiny.v.float() * 1e-33).to(torch.bfloat16)
    dc2 = cache_case(tiny, DEV)
    out2 = run_decode(tiny, dc2)
    torch.cuda.synchronize()
    ref2 = oracle_decode(tiny, dc2.host())
    assert_attn_close_scaled(out2.cpu().numpy(), ref2, "all-tiny V")


def test_empty_contexts_and_zero_max_context():
    case = synth.decode_case([0, 40, 0], 8, 2, 128, 16, rows=1, seed=2)
    dc, out, _ = check_case(case, ranges=3)
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
    out0 = run_decode(case, dc, max_context=0)
    torch.cuda.synchronize()
    assert torch.all(out0 == 0)


def test_context_lens_above_max_context_are_clamped():
    case = synth.decode_case([900, 600], 8, 2, 128, 16, rows=1, seed=4)
    dc = cache_case(case, DEV)
    out = run_decode(case, dc, max_context=512, ranges=6)
    torch.cuda.synchronize()
    clamped = torch.tensor([512, 512], dtype=torch.int32)
    ref = oracle_decode(case, dc.host(), context_lens=clamped.numpy())
    assert_attn_close(out.cpu().numpy(), ref, "clamped")


def test_partials_then_merge_equal_fused():
    case = synth.decode_case([3000, 100, 7777], 16, 4, 128, 16, rows=2, seed=9)
    dc = cache_case(case, DEV)
    L = case.layout
    kw = dict(num_kv_heads=4, block_size=16, softmax_scale=case.softmax_scale,
              max_context=7777, num_ranges=37)
    fused = fk.paged_decode_attn_fp8(case.q.to(DEV), dc.k_cache, dc.v_cache,
                                     dc.k_scale, dc.v_scale,
                                     L.block_tables.to(DEV),
                                     L.context_lens.to(DEV),
                                     out_dtype=torch.float32, **kw)
    ws = fk.paged_decode_partials(case.q.to(DEV), dc.k_cache, dc.v_cache,
                                  dc.k_scale, dc.v_scale,
                                  L.block_tables.to(DEV),
                                  L.context_lens.to(DEV), **kw)
    out = torch.empty_like(fused)
    fk.paged_decode_merge(ws, out, rows=2, num_q_heads=16, num_kv_heads=4,
                          num_ranges=37)
    torch.cuda.synchronize()
    assert torch.equal(out, fused)


def test_graph_capture_replays_with_new_lengths():
    case = synth.decode_case([4000, 2500, 333], 8, 2, 128, 16, rows=1, seed=30)
    dc = cache_case(case, DEV)
    L = case.layout
    q = case.q.to(DEV).clone()
    cl = L.context_lens.to(DEV).clone()
    bt = L.block_tables.to(DEV)
    maxc = 4000                       # the page tables' coverage
    ws = torch.empty(fk.decode_workspace_bytes(3, 1, 8, 2, 128, 13),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    kw = dict(num_kv_heads=2, block_size=16, softmax_scale=case.softmax_scale,
              max_context=maxc, num_ranges=13, out=out, workspace=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fk.paged_decode_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale,
                                 dc.v_scale, bt, cl, **kw)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fk.paged_decode_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale,
                                 dc.v_scale, bt, cl, **kw)
    host = dc.host()
    g = synth.gen(31)
    for rep, lens in enumerate([[4000, 2500, 333], [17, 2400, 333], [3999, 1, 0]]):
        cl.copy_(torch.tensor(lens, dtype=torch.int32))
        q.copy_(synth.normal_bf16(q.shape, g))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle_decode(case, host, context_lens=np.array(lens, np.int32),
                            q=q.cpu())
        assert_attn_close(out.cpu().numpy(), ref, f"replay {rep}")


def check_full_size(case, dc, name, row_groups):
    """Every row of every request against the oracle (fp32 output, gated);
    the bf16 output's error against the oracle is reported, not gated."""
    out = run_decode(case, dc)
    ob = run_decode(case, dc, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    assert torch.equal(ob, bf16_rne(out)), "bf16 output is not RNE of fp32"
    B = case.q.shape[0]
    log(f"  oracle on all {B * case.q.shape[1] * case.q.shape[2]} rows of {name}")
    ref = oracle_decode_requests(case, dc, range(B), row_groups=row_groups)
    ref = np.stack([ref[b] for b in range(B)])
    assert_attn_close(out.cpu().numpy(), ref, f"{name}, fp32 output")
    e_abs, e_rel = attn_errors(ob.float().cpu().numpy(), ref)
    log(f"  {name}, bf16 output against the oracle (reported): "
        f"max_abs={e_abs:.3e} rel_l2={e_rel:.3e}")


def test_decode_workload_full_size():
    """64 requests, lengths U[1024, 32768], Hq 32 / Hkv 8, D 128, bs 16 --
    the benchmark's decode launch (library-chosen split); the oracle
    recomputes all 64 x 32 rows."""
    case = synth.decode_workload(seed=2, device=DEV)
    dc = cache_case(case, DEV)
    check_full_size(case, dc, "decode workload", row_groups=1)


def test_longctx_full_size():
    """4 requests of 256K..1M tokens, 4 causal verify rows, Hq 16 / Hkv 4,
    bs 64, library-chosen split: the oracle recomputes all 4 x 4 x 16
    rows, 4 rows per host task."""
    case = synth.longctx_workload(seed=3, device=DEV)
    dc = cache_case(case, DEV)
    check_full_size(case, dc, "long context", row_groups=16)
