"""Pins of the oracle's decode attention over selected blocks ([ATOM]
"fix(qwen4-exp): register the QSA FP8 scale planes for KV offload",
description, K/V bullet: the sparse GQA kernel reads E4M3 tiles with the key
scale applied to each score and the value scale to each probability weight;
FreeToken #354 description: only the chosen rows of the cache are fetched,
as codes).

Fixed outside the oracle:
* torch float64 softmax(scale * q K^T) V over exactly the keys the
  selection names (gathered here from the page table and valid counts,
  dequantized with torch's float8_e4m3fn view and the fp32 row scales);
* a selection of every block with full valid counts equals the dense
  paged decode (itself pinned in test_oracle_attn.py);
* closed form: a selection holding a single key returns its value row;
* structure: a selected block with no valid key changes nothing; the
  order of the selected blocks before the last one does not matter.
"""
import numpy as np
import torch

import oracle
from fp8_e4m3_paged_kv_amd import synth

from test_oracle_attn import bf16_bits, build_cache, run_oracle


def run_sparse(case, cache, sel, q=None, rows=None):
    kc, vc, ks, vs = cache
    q = case.q if q is None else q
    return oracle.sparse_decode_attn(
        bf16_bits(q), kc, vc, ks, vs, sel.block_tables.numpy(),
        sel.block_valid.numpy(), sel.context_lens.numpy(), case.num_kv_heads,
        case.layout.block_size, case.softmax_scale, rows=rows)


def torch_sparse_reference(case, cache, sel):
    kc, vc, ks, vs = cache
    B, R, Hq, D = case.q.shape
    G = Hq // case.num_kv_heads
    bs = case.layout.block_size
    kd = torch.from_numpy(kc).view(torch.float8_e4m3fn).double() * torch.from_numpy(ks).double()[..., None]
    vd = torch.from_numpy(vc).view(torch.float8_e4m3fn).double() * torch.from_numpy(vs).double()[..., None]
    out = torch.zeros((B, R, Hq, D), dtype=torch.float64)
    for b in range(B):
        V = int(sel.context_lens[b])
        for r in range(R):
            last = V - R + r                      # last visible virtual position
            slots = []
            for j in range(last + 1):
                i, o = divmod(j, bs)
                if o < int(sel.block_valid[b, i]):
                    slots.append(int(sel.block_tables[b, i]) * bs + o)
            if not slots:
                continue
            sl = torch.tensor(slots)
            for hq in range(Hq):
                h = hq // G
                q = case.q[b, r, hq].double()
                s = (kd[sl, h] @ q) * case.softmax_scale
                out[b, r, hq] = torch.softmax(s, 0) @ vd[sl, h]
    return out.numpy()


def test_matches_torch_on_gathered_keys():
    case = synth.decode_case([300, 77, 1000], 8, 2, 64, 16, rows=3, seed=5)
    cache = build_cache(case)
    sel = synth.sparse_selection(case.layout, 0.4, seed=6, partial_frac=0.5)
    got = run_sparse(case, cache, sel)
    ref = torch_sparse_reference(case, cache, sel)
    assert np.abs(got - ref).max() < 1e-12


def test_every_block_full_equals_dense():
    case = synth.decode_case([300, 77, 1000], 8, 2, 64, 16, rows=2, seed=7)
    cache = build_cache(case)
    L = case.layout
    bt = L.block_tables.clone()
    bv = torch.zeros_like(bt)
    for b, n in enumerate(L.context_lens.tolist()):
        nb = (n + 15) // 16
        bv[b, :nb] = 16
        bv[b, nb - 1] = n - (nb - 1) * 16
    sel = synth.SparseSelection(bt, bv, L.context_lens.clone())
    assert np.abs(run_sparse(case, cache, sel) - run_oracle(case, cache)).max() < 1e-13


def test_single_key_returns_its_value_row():
    case = synth.decode_case([200], 4, 2, 64, 16, rows=1, seed=8)
    cache = build_cache(case)
    kc, vc, ks, vs = cache
    blk = int(case.layout.block_tables[0, 5])
    sel = synth.SparseSelection(torch.tensor([[blk]], dtype=torch.int32),
                                torch.tensor([[1]], dtype=torch.int32),
                                torch.tensor([1], dtype=torch.int32))
    got = run_sparse(case, cache, sel)
    slot = blk * 16
    for hq in range(4):
        h = hq // 2
        want = oracle.decode(vc[slot, h]) * float(vs[slot, h])
        assert np.array_equal(got[0, 0, hq], want)


def test_empty_blocks_and_order_do_not_matter():
    case = synth.decode_case([640], 8, 2, 64, 16, rows=1, seed=9)
    cache = build_cache(case)
    sel = synth.sparse_selection(case.layout, 0.5, seed=10, partial_frac=0.3)
    base = run_sparse(case, cache, sel)
    n = int((sel.block_valid[0] > 0).sum())
    k = sel.block_tables.shape[1]
    # an extra selected block with no valid key, placed first
    bt = torch.cat([case.layout.block_tables[:1, :1], sel.block_tables], 1)
    bv = torch.cat([torch.zeros((1, 1), dtype=torch.int32), sel.block_valid], 1)
    ext = synth.SparseSelection(bt, bv, sel.context_lens + 16)
    assert np.abs(run_sparse(case, cache, ext) - base).max() < 1e-13
    # the selected blocks before the last one, reversed
    perm = list(range(k - 2, -1, -1)) + [k - 1]
    rev = synth.SparseSelection(sel.block_tables[:, perm].contiguous(),
                                sel.block_valid[:, perm].contiguous(), sel.context_lens)
    assert np.abs(run_sparse(case, cache, rev) - base).max() < 1e-12
    assert n >= 2
