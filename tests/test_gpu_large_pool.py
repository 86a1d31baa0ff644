"""The GPU path on a pool whose used blocks lie past 4 GiB: a 32-bit slot or
byte offset anywhere in the store, the decode page walk, the selected-block
walk or the prefill loader would wrap and read or write the wrong place.

The same cases run on a compact pool and on a 5.12 GB pool (Hkv 8, D 128,
5,000,000 slots) with every block id shifted to its top end. Bar: the
stored codes and scales are the same bytes; nothing below the shifted
blocks changes; the attention outputs are the same bits (same kernels,
same data, only the addresses differ) and within the attention bar of the
oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import (SCALE_SENTINEL, SENTINEL, DevCache, assert_attn_close,
                       cache_case, log, oracle_decode, run_decode)

pytestmark = pytest.mark.gpu
DEV = "cuda"
H, D, BS = 8, 128, 16
BIG_SLOTS = 5_000_000                       # 5.12 GB per code buffer


def shifted(case):
    """The case with every block id moved to the top of the big pool."""
    L = case.layout
    total = BIG_SLOTS // BS
    off = total - L.num_blocks
    lay = synth.PagedLayout(L.context_lens, L.block_tables + off,
                            L.token_slots + off * BS, BS, total)
    return dataclasses.replace(case, layout=lay), off


def untouched_below(t, end, value, chunk=1 << 28):
    flat = t.reshape(-1)
    for i in range(0, end, chunk):
        if bool((flat[i:min(i + chunk, end)] != value).any()):
            return False
    return True


def test_store_and_decode_past_4gib():
    case = synth.decode_case([300, 1000, 77, 2048], 32, H, D, BS, rows=2, seed=120)
    big_case, off = shifted(case)
    assert off * BS * H * D > 2 ** 32
    log(f"large pool: blocks shifted by {off} ({off * BS * H * D / 2**30:.2f} GiB)")
    small = cache_case(case, DEV)
    big = DevCache(BIG_SLOTS, H, D, DEV)                 # sentinel-filled
    big.scatter(case.k.to(DEV), case.v.to(DEV), big_case.layout.token_slots.to(DEV))
    ss = case.layout.token_slots.to(DEV)
    bsl = big_case.layout.token_slots.to(DEV)
    torch.cuda.synchronize()
    assert torch.equal(big.k_cache[bsl], small.k_cache[ss])
    assert torch.equal(big.v_cache[bsl], small.v_cache[ss])
    assert torch.equal(big.k_scale[bsl], small.k_scale[ss])
    assert torch.equal(big.v_scale[bsl], small.v_scale[ss])
    lo = off * BS
    assert untouched_below(big.k_cache, lo * H * D, SENTINEL)
    assert untouched_below(big.v_cache, lo * H * D, SENTINEL)
    for h in range(H):
        assert untouched_below(big.k_plane[h], lo, SCALE_SENTINEL)
        assert untouched_below(big.v_plane[h], lo, SCALE_SENTINEL)

    for ranges in (0, 7):
        got = run_decode(big_case, big, ranges=ranges)
        ref = run_decode(case, small, ranges=ranges)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"ranges={ranges}"
    want = oracle_decode(case, small.host())
    assert_attn_close(got.cpu().numpy(), want, "large pool decode")


def test_selected_blocks_and_prefill_past_4gib():
    case = synth.decode_case([900, 2000, 64], 32, H, D, BS, rows=40, seed=121)
    big_case, off = shifted(case)
    small = cache_case(case, DEV)
    big = DevCache(BIG_SLOTS, H, D, DEV, sentinel=False)
    big.scatter(case.k.to(DEV), case.v.to(DEV), big_case.layout.token_slots.to(DEV))
    L = case.layout
    kw = dict(num_kv_heads=H, block_size=BS, softmax_scale=case.softmax_scale,
              max_context=int(L.context_lens.max()))

    # prefill: the last 40 tokens of each request
    ql = torch.full((3,), 40, dtype=torch.int32, device=DEV)
    q = case.q.to(DEV)
    outs = []
    for lay, dc in ((big_case.layout, big), (L, small)):
        outs.append(fk.prefill_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                                        lay.block_tables.to(DEV), lay.context_lens.to(DEV), ql,
                                        out_dtype=torch.float32, **kw))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "prefill"

    # selected blocks, decode of the first 2 verify rows
    sel = synth.sparse_selection(L, 0.4, seed=122, partial_frac=0.3)
    q2 = case.q[:, :2].contiguous().to(DEV)
    outs = []
    for shift, dc in ((off, big), (0, small)):
        outs.append(fk.sparse_decode_attn_fp8(
            q2, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
            (sel.block_tables + shift).to(DEV), sel.block_valid.to(DEV),
            sel.context_lens.to(DEV), num_ranges=5, out_dtype=torch.float32,
            num_kv_heads=H, block_size=BS, softmax_scale=case.softmax_scale,
            max_context=int(sel.context_lens.max())))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "selected blocks"
    assert bool(torch.isfinite(outs[0]).all())
