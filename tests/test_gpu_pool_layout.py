"""The code pool stored head-major ([Hkv, slots, D], passed as a permuted
[slots, Hkv, D] view: a KV head's rows of a block are contiguous) against
the slot-major pool ([slots, Hkv, D]). Only the addresses differ: the
store writes the same codes and scales, and decode, the decode step with
its new tokens' store, selected-block decode and prefill give the same
outputs bit for bit; the head-major decode also meets the attention bar
against the oracle."""
import numpy as np
import pytest
import torch

import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import DevCache, assert_attn_close, cache_case, log, oracle_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"


def same_pool(a, b):
    return (torch.equal(a.k_cache.contiguous(), b.k_cache.contiguous())
            and torch.equal(a.v_cache.contiguous(), b.v_cache.contiguous())
            and torch.equal(a.k_plane, b.k_plane) and torch.equal(a.v_plane, b.v_plane))


def kw(case):
    L = case.layout
    return dict(num_kv_heads=case.num_kv_heads, block_size=L.block_size,
                softmax_scale=case.softmax_scale, max_context=L.block_size * L.block_tables.shape[1])


@pytest.mark.parametrize("bs,D", [(16, 128), (48, 128), (16, 64)])
def test_store_and_decode_same_on_both_pools(bs, D):
    case = synth.decode_case([1, 300, 2049, 777, 5000], 32, 8, D, bs, rows=2, seed=600 + bs + D)
    log(f"pool layouts: bs={bs} D={D}")
    slot = cache_case(case, DEV, pool="slot")
    head = cache_case(case, DEV, pool="head")
    torch.cuda.synchronize()
    assert same_pool(slot, head), "the store wrote different codes or scales"
    L = case.layout
    q, bt, cl = case.q.to(DEV), L.block_tables.to(DEV), L.context_lens.to(DEV)
    outs = []
    for dc in (slot, head):
        outs.append(fk.paged_decode_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                                             bt, cl, out_dtype=torch.float32, **kw(case)))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert_attn_close(outs[1].cpu().numpy(), oracle_decode(case, head.host()), "head-major pool")


def test_decode_step_with_append_same_on_both_pools():
    """The decode step: each request's newest token stored inside the split
    launch, then the merge."""
    case = synth.decode_case([40, 1000, 3000, 64], 16, 4, 128, 16, rows=1, seed=610)
    L = case.layout
    lens = L.context_lens.tolist()
    last = torch.tensor(np.cumsum(lens) - 1)
    keep = torch.ones(case.k.shape[0], dtype=torch.bool)
    keep[last] = False
    q, bt, cl = case.q.to(DEV), L.block_tables.to(DEV), L.context_lens.to(DEV)
    k_new = case.k[last].unsqueeze(1).contiguous().to(DEV)
    v_new = case.v[last].unsqueeze(1).contiguous().to(DEV)
    res = []
    for pool in ("slot", "head"):
        dc = DevCache(L.num_slots, 4, 128, DEV, "head_major", pool=pool)
        dc.scatter(case.k[keep].to(DEV), case.v[keep].to(DEV), L.token_slots[keep].to(DEV))
        out = fk.paged_decode_append_attn_fp8(q, k_new, v_new, dc.k_cache, dc.v_cache, dc.k_scale,
                                              dc.v_scale, bt, cl, out_dtype=torch.float32,
                                              **kw(case))
        torch.cuda.synchronize()
        res.append((dc, out))
    assert same_pool(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1])


def test_prefill_and_selected_blocks_same_on_both_pools():
    case = synth.decode_case([700, 1500], 32, 8, 128, 16, rows=64, seed=620)
    L = case.layout
    ql = torch.tensor([64, 40], dtype=torch.int32)
    sel = synth.prefill_selection(L, ql, 0.3, seed=621, partial_frac=0.3)
    outs = []
    for pool in ("slot", "head"):
        dc = cache_case(case, DEV, pool=pool)
        dense = fk.prefill_attn_fp8(case.q.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                                    L.block_tables.to(DEV), L.context_lens.to(DEV), ql.to(DEV),
                                    out_dtype=torch.float32, **kw(case))
        sparse = fk.sparse_prefill_attn_fp8(
            case.q.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
            sel.block_tables.to(DEV), sel.block_valid.to(DEV), sel.context_lens.to(DEV),
            ql.to(DEV), num_kv_heads=8, block_size=16, softmax_scale=case.softmax_scale,
            max_context=16 * sel.block_tables.shape[1], out_dtype=torch.float32)
        torch.cuda.synchronize()
        outs.append((dense, sparse))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_decode_workload_step_full_size_head_major_pool():
    """The benchmark's decode step (64 requests, lengths U[1024, 32768],
    Hq 32 / Hkv 8, bs 16, newest token appended) on a head-major pool:
    pool and output equal to the slot-major pool's bit for bit."""
    case = synth.decode_workload(seed=2, device=DEV)
    L = case.layout
    lens = L.context_lens.tolist()
    last = torch.tensor(np.cumsum(lens) - 1, device=DEV)
    keep = torch.ones(case.k.shape[0], dtype=torch.bool, device=DEV)
    keep[last] = False
    slots = L.token_slots.to(DEV)
    q, bt, cl = case.q.to(DEV), L.block_tables.to(DEV), L.context_lens.to(DEV)
    k_new = case.k[last].unsqueeze(1).contiguous()
    v_new = case.v[last].unsqueeze(1).contiguous()
    res = []
    for pool in ("slot", "head"):
        log(f"  decode workload step, {pool}-major pool")
        dc = DevCache(L.num_slots, 8, 128, DEV, "head_major", pool=pool)
        dc.scatter(case.k[keep], case.v[keep], slots[keep])
        out = fk.paged_decode_append_attn_fp8(q, k_new, v_new, dc.k_cache, dc.v_cache,
                                              dc.k_scale, dc.v_scale, bt, cl,
                                              out_dtype=torch.float32, **kw(case))
        torch.cuda.synchronize()
        res.append((dc, out))
    assert same_pool(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1])
