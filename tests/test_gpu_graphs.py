"""The new entry points take every length on the device, so they can be
captured once into a HIP graph and replayed with new inputs: each replay
must equal an eager call on the same inputs. (The graphs hold only this
library's kernels: no memset nodes, no allocations.)"""
import numpy as np
import pytest
import torch

import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import cache_case, log

pytestmark = pytest.mark.gpu
DEV = "cuda"


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_sparse_decode_replays():
    case = synth.decode_case([3000, 700, 1500], 32, 8, 128, 16, rows=1, seed=80)
    dc = cache_case(case, DEV)
    sel = synth.sparse_selection(case.layout, 0.3, seed=81, partial_frac=0.3)
    q = case.q.to(DEV).clone()
    width = case.layout.block_tables.shape[1]          # room for any selection
    bt = torch.zeros((3, width), dtype=torch.int32, device=DEV)
    bv = torch.zeros_like(bt)
    m = sel.block_tables.shape[1]
    bt[:, :m].copy_(sel.block_tables)
    bv[:, :m].copy_(sel.block_valid)
    cl = sel.context_lens.to(DEV).clone()
    ws = torch.empty(fk.decode_workspace_bytes(3, 1, 32, 8, 128, 29), dtype=torch.uint8, device=DEV)
    out = torch.empty(q.shape, device=DEV)
    kw = dict(num_kv_heads=8, block_size=16, softmax_scale=case.softmax_scale,
              max_context=16 * width, num_ranges=29, workspace=ws)
    run = lambda o: fk.sparse_decode_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale,
                                              dc.v_scale, bt, bv, cl, out=o, **kw)
    g = capture(lambda: run(out))
    gen = synth.gen(82)
    for rep in range(3):
        sel2 = synth.sparse_selection(case.layout, 0.2 + 0.2 * rep, seed=83 + rep, partial_frac=0.5)
        m = sel2.block_tables.shape[1]
        bt.zero_(); bv.zero_()
        bt[:, :m].copy_(sel2.block_tables); bv[:, :m].copy_(sel2.block_valid)
        cl.copy_(sel2.context_lens)
        q.copy_(synth.normal_bf16(q.shape, gen))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = torch.empty_like(out)
        run(eager)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep


def test_prefill_replays():
    case = synth.decode_case([600, 900], 32, 8, 128, 16, rows=64, seed=84)
    dc = cache_case(case, DEV)
    L = case.layout
    q = case.q.to(DEV).clone()
    bt, cl = L.block_tables.to(DEV), L.context_lens.to(DEV).clone()
    ql = torch.full((2,), 64, dtype=torch.int32, device=DEV)
    out = torch.zeros(q.shape, device=DEV)
    run = lambda o: fk.prefill_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                                        bt, cl, ql, num_kv_heads=8, block_size=16,
                                        softmax_scale=case.softmax_scale, max_context=900,
                                        out=o)
    g = capture(lambda: run(out))
    gen = synth.gen(85)
    for rep, (lens, qls) in enumerate([([600, 900], [64, 64]), ([300, 899], [10, 64]),
                                       ([64, 1], [64, 1])]):
        cl.copy_(torch.tensor(lens, dtype=torch.int32))
        ql.copy_(torch.tensor(qls, dtype=torch.int32))
        q.copy_(synth.normal_bf16(q.shape, gen))
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = torch.zeros_like(out)
        run(eager)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep


@pytest.mark.parametrize("fmt", [fk.KEYS_MXFP4, fk.KEYS_E4M3])
def test_index_build_and_score_replay(fmt):
    B, R, H, N = 2, 40, 16, 500
    raw = synth.normal_bf16((B, 4 * N, 128), synth.gen(86)).to(DEV)
    nb = 64 if fmt == fk.KEYS_MXFP4 else 128
    codes = torch.empty((B, N, nb), dtype=torch.uint8, device=DEV)
    scales = (torch.empty((B, N, 4), dtype=torch.uint8, device=DEV) if fmt == fk.KEYS_MXFP4
              else torch.empty((B, N), device=DEV))
    case = synth.index_case(B, R, H, N, seed=87)
    q, w = case.q.to(DEV).clone(), case.w.to(DEV).clone()
    out = torch.empty((B, R, N), device=DEV)

    def step(o, c, s):
        fk.index_keys_build(raw, 0, N, fmt, c, s)
        fk.index_score_mxfp4(q, w, fmt, c, s, out=o)
    g = capture(lambda: step(out, codes, scales))
    gen = synth.gen(88)
    for rep in range(3):
        raw.copy_(synth.normal_bf16(raw.shape, gen))
        q.copy_(synth.normal_bf16(q.shape, gen))
        w.copy_(torch.rand(w.shape, generator=gen))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        c2, s2, o2 = torch.empty_like(codes), torch.empty_like(scales), torch.empty_like(out)
        step(o2, c2, s2)
        torch.cuda.synchronize()
        assert torch.equal(codes, c2) and torch.equal(scales, s2) and torch.equal(out, o2), rep


def test_unscaled_store_and_decode_replay():
    """One graph holding the unscaled E5M2 store of new tokens and the decode
    over the cache; replayed with new K/V, slots, queries and lengths."""
    case = synth.decode_case([800, 1200], 16, 4, 128, 16, rows=1, seed=86)
    L = case.layout
    S = L.num_slots
    kc = torch.zeros((S, 4, 128), dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    fk.kv_quant_scatter_unscaled(case.k.to(DEV), case.v.to(DEV), L.token_slots.to(DEV),
                                 kc, vc, fk.CODES_E5M2)
    gen = synth.gen(87)
    k_new = synth.normal_bf16((2, 4, 128), gen).to(DEV)
    v_new = synth.normal_bf16((2, 4, 128), gen).to(DEV)
    slots = torch.zeros(2, dtype=torch.int64, device=DEV)
    q = case.q.to(DEV).clone()
    bt, cl = L.block_tables.to(DEV), L.context_lens.to(DEV).clone()
    ws = torch.empty(fk.decode_workspace_bytes(2, 1, 16, 4, 128, 13), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty(q.shape, device=DEV)
    kw = dict(num_kv_heads=4, block_size=16, softmax_scale=case.softmax_scale,
              max_context=1200, code_format=fk.CODES_E5M2, num_ranges=13, workspace=ws)

    def step(o):
        fk.kv_quant_scatter_unscaled(k_new, v_new, slots, kc, vc, fk.CODES_E5M2)
        fk.paged_decode_attn_unscaled(q, kc, vc, bt, cl, out=o, **kw)
    slots.copy_(L.token_slots[torch.tensor([799, 1999])])
    g = capture(lambda: step(out))
    lens = L.context_lens.tolist()
    for rep in range(3):
        n = [lens[0] - 50 * rep, lens[1] - 70 * rep]
        cl.copy_(torch.tensor(n, dtype=torch.int32))
        slots.copy_(L.token_slots[torch.tensor([n[0] - 1, lens[0] + n[1] - 1])])
        k_new.copy_(synth.normal_bf16(k_new.shape, gen))
        v_new.copy_(synth.normal_bf16(v_new.shape, gen))
        q.copy_(synth.normal_bf16(q.shape, gen))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_k, got_v = kc.clone(), vc.clone()
        eager = torch.empty_like(out)
        step(eager)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        assert torch.equal(got_k, kc) and torch.equal(got_v, vc), rep
