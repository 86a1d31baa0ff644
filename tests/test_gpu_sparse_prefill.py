"""GPU parity of fp8kv_sparse_prefill_attn_fp8 (chunked-prefill attention
over the selected blocks only) against the oracle's attention over selected
blocks with R = the chunk's rows, on the same dequantized cache.

Bar: as the dense prefill -- fp32 output within max-abs 2e-3 and rel-L2
1e-3, bf16 output equal to the RNE of the same kernel's fp32 output. A
selection of every block with full counts walks the same keys as the dense
prefill; the dense kernel (head_dim 128) splits each query block's keys
into two groups merged by log-sum-exp, so the two agree within the same
bar rather than bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import (assert_attn_close, bf16_bits, bf16_rne, cache_case,
                       compact_host_cache, log)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(case, dc, sel, q_lens, out_dtype=torch.float32, out=None):
    return fk.sparse_prefill_attn_fp8(
        case.q.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
        sel.block_tables.to(DEV), sel.block_valid.to(DEV), sel.context_lens.to(DEV),
        q_lens.to(DEV), num_kv_heads=case.num_kv_heads, block_size=case.layout.block_size,
        softmax_scale=case.softmax_scale,
        max_context=case.layout.block_size * sel.block_tables.shape[1],
        out_dtype=out_dtype, out=out)


def oracle_rows(case, host, sel, b, n):
    """The oracle's selected-block attention of request b's n chunk rows."""
    kc, vc, ks, vs = host
    q = case.q[b:b + 1, :n].clone()
    return oracle.sparse_decode_attn(
        bf16_bits(q), kc, vc, ks, vs, sel.block_tables[b:b + 1].numpy(),
        sel.block_valid[b:b + 1].numpy(), sel.context_lens[b:b + 1].numpy(),
        case.num_kv_heads, case.layout.block_size, case.softmax_scale)[0]


def check(case, sel, q_lens, name, layout="head_major"):
    log(f"sparse prefill {name}: lens={case.layout.context_lens.tolist()} "
        f"virtual={sel.context_lens.tolist()} q_lens={q_lens.tolist()} "
        f"Hq={case.num_q_heads} Hkv={case.num_kv_heads} D={case.head_dim} "
        f"bs={case.layout.block_size}")
    dc = cache_case(case, DEV, layout)
    out = torch.full(case.q.shape, 7.0, device=DEV)
    run(case, dc, sel, q_lens, out=out)
    torch.cuda.synchronize()
    host = dc.host()
    for b, n in enumerate(q_lens.tolist()):
        if n:
            ref = oracle_rows(case, host, sel, b, n)
            assert_attn_close(out[b, :n].cpu().numpy(), ref, f"{name}, request {b}")
        assert torch.all(out[b, n:] == 7.0), "rows past the chunk were written"
    ob = torch.full(case.q.shape, 7.0, dtype=torch.bfloat16, device=DEV)
    run(case, dc, sel, q_lens, out=ob)
    torch.cuda.synchronize()
    for b, n in enumerate(q_lens.tolist()):
        assert torch.equal(ob[b, :n], bf16_rne(out[b, :n])), "bf16 is not RNE of fp32"
    return dc, out


@pytest.mark.parametrize("bs", [16, 48, 64])
@pytest.mark.parametrize("keep,partial", [(0.25, 0.0), (0.3, 0.5), (1.0, 0.3)])
def test_selected_blocks_match_oracle(bs, keep, partial):
    case = synth.decode_case([900, 2000, 130], 32, 8, 128, bs, rows=70, seed=200 + bs)
    ql = torch.tensor([70, 33, 70], dtype=torch.int32)
    sel = synth.prefill_selection(case.layout, ql, keep, seed=201, partial_frac=partial)
    check(case, sel, ql, f"bs{bs} keep{keep} partial{partial}")


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 2, 128), (8, 8, 128), (16, 4, 64), (32, 2, 128)])
def test_groups_and_head_dims(Hq, Hkv, D):
    case = synth.decode_case([1500, 700], Hq, Hkv, D, 16, rows=45, seed=210 + Hq + D)
    ql = torch.tensor([45, 20], dtype=torch.int32)
    sel = synth.prefill_selection(case.layout, ql, 0.2, seed=211, partial_frac=0.4)
    check(case, sel, ql, f"Hq{Hq} Hkv{Hkv} D{D}", layout="slot_major" if D == 64 else "head_major")


def test_unread_scales_do_not_move_the_range():
    """Every value and key scale the kernel must not read -- past a selected
    block's valid count, and in blocks no request selected -- set to 2^100.
    The kernel fixes its P' range exponent from the scales of the keys it
    reads; had it taken one of these, P' would underflow and the output
    would collapse towards zero."""
    case = synth.decode_case([900, 2000, 130], 32, 8, 128, 16, rows=70, seed=230)
    ql = torch.tensor([70, 33, 70], dtype=torch.int32)
    sel = synth.prefill_selection(case.layout, ql, 0.3, seed=231, partial_frac=0.6)
    bs = case.layout.block_size
    dc = cache_case(case, DEV)
    readable = torch.zeros(case.layout.num_slots, dtype=torch.bool)
    for b, vlen in enumerate(sel.context_lens.tolist()):
        for i in range((vlen + bs - 1) // bs):
            n = min(bs, vlen - i * bs, max(int(sel.block_valid[b, i]), 0))
            blk = int(sel.block_tables[b, i])
            readable[blk * bs: blk * bs + max(n, 0)] = True
    far = readable.logical_not().to(DEV)
    log(f"unread scales: {int(far.sum())} of {far.numel()} slots set to 2^100")
    dc.v_scale[far] = 2.0 ** 100
    dc.k_scale[far] = 2.0 ** 100
    out = run(case, dc, sel, ql)
    torch.cuda.synchronize()
    host = dc.host()
    for b, n in enumerate(ql.tolist()):
        ref = oracle_rows(case, host, sel, b, n)
        assert_attn_close(out[b, :n].cpu().numpy(), ref, f"unread scales, request {b}")


def test_every_block_full_matches_dense():
    case = synth.decode_case([3000, 777], 32, 8, 128, 16, rows=64, seed=220)
    L = case.layout
    ql = torch.tensor([64, 50], dtype=torch.int32)
    bv = torch.zeros_like(L.block_tables)
    for b, n in enumerate(L.context_lens.tolist()):
        nb = (n + 15) // 16
        bv[b, :nb] = 16
        bv[b, nb - 1] = n - (nb - 1) * 16
    sel = synth.SparseSelection(L.block_tables.clone(), bv, L.context_lens.clone())
    dc = cache_case(case, DEV)
    sparse = run(case, dc, sel, ql)
    dense = fk.prefill_attn_fp8(
        case.q.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
        L.block_tables.to(DEV), L.context_lens.to(DEV), ql.to(DEV), num_kv_heads=8,
        block_size=16, softmax_scale=case.softmax_scale,
        max_context=16 * L.block_tables.shape[1], out_dtype=torch.float32)
    torch.cuda.synchronize()
    host = dc.host()
    for b, n in enumerate(ql.tolist()):
        ref = oracle_rows(case, host, sel, b, n)
        assert_attn_close(sparse[b, :n].cpu().numpy(), ref, f"selected, request {b}")
        assert_attn_close(dense[b, :n].cpu().numpy(), ref, f"dense, request {b}")
    assert_attn_close(sparse.cpu().numpy(), dense.cpu().numpy().astype(np.float64),
                      "selected vs dense")


def test_tokens_that_see_no_key_output_zero():
    """Every block before the chunk selected with no valid key and the
    chunk's first block emptied too: the chunk's first tokens see nothing
    (output 0), later ones only the chunk's own keys."""
    case = synth.decode_case([640, 300], 16, 4, 128, 16, rows=40, seed=230)
    ql = torch.tensor([40, 40], dtype=torch.int32)
    sel = synth.prefill_selection(case.layout, ql, 0.5, seed=231)
    nb = [(n + 15) // 16 for n in case.layout.context_lens.tolist()]
    first = [(n - 40) // 16 for n in case.layout.context_lens.tolist()]
    empty_until = []
    for b in range(2):
        nsel = int((sel.block_valid[b] > 0).sum())
        before = nsel - (nb[b] - first[b])
        sel.block_valid[b, :before + 1] = 0            # ... and the chunk's first block
        empty_until.append(16 * (before + 1))          # virtual positions with no key
    dc, out = check(case, sel, ql, "keys only late in the chunk")
    for b in range(2):
        P = int(sel.context_lens[b]) - 40
        blind = max(0, empty_until[b] - P)             # chunk tokens that see no key
        assert blind > 0
        assert torch.all(out[b, :blind] == 0), "a token with no key is not 0"
        assert torch.any(out[b, blind:40] != 0)


def test_prefill_workload_selection_full_size_sampled():
    """The prefill workload (a 4096-token chunk at the end of a 32,768-token
    request, Hq 32 / Hkv 8, bs 16) with 1/8 of the blocks before the chunk
    selected plus the chunk's own; the oracle recomputes sampled rows."""
    case = synth.prefill_attn_workload(seed=71, device=DEV)
    C = case.q.shape[1]
    ql = torch.tensor([C], dtype=torch.int32)
    sel = synth.prefill_selection(case.layout, ql, 0.125, seed=72)
    dc = cache_case(case, DEV)
    out = run(case, dc, sel, ql)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    # compact host copy of the selected blocks, table remapped onto it
    nsel = int((sel.block_valid[0] > 0).sum())
    blocks = sel.block_tables[0, :nsel].long()
    NB = dc.S // 16
    idx = blocks.to(DEV)
    kc = dc.k_cache.view(NB, 16, dc.H, dc.D)[idx].reshape(-1, dc.H, dc.D).cpu().numpy()
    vc = dc.v_cache.view(NB, 16, dc.H, dc.D)[idx].reshape(-1, dc.H, dc.D).cpu().numpy()
    kp = dc.k_plane.view(dc.H, NB, 16)[:, idx].reshape(dc.H, -1).cpu().numpy()
    vp = dc.v_plane.view(dc.H, NB, 16)[:, idx].reshape(dc.H, -1).cpu().numpy()
    bt = torch.arange(nsel, dtype=torch.int32)[None]
    bv = sel.block_valid[:, :nsel].clone()
    g = torch.Generator().manual_seed(73)
    Hq = case.q.shape[2]
    toks = torch.cat([torch.tensor([0, 1, C - 1]), torch.randint(0, C, (13,), generator=g)])
    heads = torch.randint(0, Hq, (4,), generator=g)
    rows = [int(t) * Hq + int(h) for t in toks for h in heads]
    log(f"  {nsel} selected blocks ({int(sel.context_lens[0])} virtual positions), "
        f"{len(rows)} sampled rows")
    ref = oracle.sparse_decode_attn(bf16_bits(case.q), kc, vc, kp.T, vp.T, bt.numpy(),
                                    bv.numpy(), sel.context_lens.numpy(), 8, 16,
                                    case.softmax_scale, rows=rows)
    got = out[0].reshape(-1, 128)[rows].cpu().numpy()
    assert_attn_close(got, ref, "sparse prefill sampled")
