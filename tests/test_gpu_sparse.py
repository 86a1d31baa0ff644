"""GPU parity of fp8kv_sparse_decode_attn_fp8 (decode attention over the
selected blocks only) against the oracle on the same dequantized cache.

Bar: as the dense decode -- fp32 output within max-abs 2e-3 and rel-L2 1e-3
of the oracle, bf16 output equal to the RNE of the same kernel's fp32
output. A selection of every block with full counts must give the dense
kernel's output bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import (DevCache, assert_attn_close, bf16_bits, bf16_rne,
                       cache_case, log, run_decode)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_sparse(case, dc, sel, *, ranges=0, out_dtype=torch.float32,
               max_context=None, q=None):
    q = (case.q if q is None else q).to(DEV)
    if max_context is None:
        max_context = int(sel.context_lens.max()) if len(sel.context_lens) else 0
    return fk.sparse_decode_attn_fp8(
        q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
        sel.block_tables.to(DEV), sel.block_valid.to(DEV),
        sel.context_lens.to(DEV), num_kv_heads=case.num_kv_heads,
        block_size=case.layout.block_size, softmax_scale=case.softmax_scale,
        max_context=max_context, num_ranges=ranges, out_dtype=out_dtype)


def oracle_sparse(case, host, sel, rows=None, q=None):
    kc, vc, ks, vs = host
    return oracle.sparse_decode_attn(
        bf16_bits(case.q if q is None else q), kc, vc, ks, vs,
        sel.block_tables.numpy(), sel.block_valid.numpy(),
        sel.context_lens.numpy(), case.num_kv_heads, case.layout.block_size,
        case.softmax_scale, rows=rows)


def check(case, sel, ranges=0, layout="head_major", name=""):
    log(f"sparse {name}: lens={sel.context_lens.tolist()[:6]} R={case.rows} "
        f"bs={case.layout.block_size} selected={int((sel.block_valid > 0).sum())} "
        f"ranges={ranges} {layout}")
    dc = cache_case(case, DEV, layout)
    out = run_sparse(case, dc, sel, ranges=ranges)
    torch.cuda.synchronize()
    ref = oracle_sparse(case, dc.host(), sel)
    assert_attn_close(out.cpu().numpy(), ref, name)
    ob = run_sparse(case, dc, sel, ranges=ranges, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(ob, bf16_rne(out)), "bf16 output is not RNE of fp32"
    return dc, out


@pytest.mark.parametrize("bs", [16, 48, 64])
@pytest.mark.parametrize("keep,partial", [(0.3, 0.0), (0.3, 0.5), (0.05, 0.2), (1.0, 0.7)])
def test_selected_blocks_match_oracle(bs, keep, partial):
    case = synth.decode_case([1, 31, 700, 3000, 77], 8, 2, 128, bs, rows=1,
                             seed=40 + bs)
    sel = synth.sparse_selection(case.layout, keep, seed=41, partial_frac=partial)
    check(case, sel, name=f"bs{bs} keep{keep} partial{partial}")


@pytest.mark.parametrize("ranges", [0, 3, 500])
def test_verify_rows_on_virtual_positions(ranges):
    """4 verify rows x 4 query heads; causal on the virtual positions."""
    case = synth.decode_case([5, 900, 4000], 16, 4, 128, 16, rows=4, seed=44,
                             k_outlier_frac=0.005)
    sel = synth.sparse_selection(case.layout, 0.25, seed=45, partial_frac=0.3)
    check(case, sel, ranges=ranges, name=f"verify ranges={ranges}")


def test_head_dim_64_slot_major():
    case = synth.decode_case([640, 129], 16, 4, 64, 32, rows=2, seed=46)
    sel = synth.sparse_selection(case.layout, 0.4, seed=47, partial_frac=0.4)
    check(case, sel, layout="slot_major", name="D64 slot-major")


def test_every_block_full_equals_dense_bit_for_bit():
    case = synth.decode_case([3000, 100, 7777], 16, 4, 128, 16, rows=2, seed=48)
    L = case.layout
    bv = torch.zeros_like(L.block_tables)
    for b, n in enumerate(L.context_lens.tolist()):
        nb = (n + 15) // 16
        bv[b, :nb] = 16
        bv[b, nb - 1] = n - (nb - 1) * 16
    sel = synth.SparseSelection(L.block_tables.clone(), bv, L.context_lens.clone())
    dc = cache_case(case, DEV)
    dense = run_decode(case, dc, ranges=37)
    sparse = run_sparse(case, dc, sel, ranges=37)
    torch.cuda.synchronize()
    assert torch.equal(sparse, dense)


def test_requests_without_keys_output_zero():
    case = synth.decode_case([400, 300, 0], 8, 2, 128, 16, rows=1, seed=49)
    sel = synth.sparse_selection(case.layout, 0.5, seed=50)
    sel.block_valid[1] = 0                  # request 1 selects blocks with no key
    dc, out = check(case, sel, name="empty")
    assert torch.all(out[1] == 0) and torch.all(out[2] == 0)


def test_decode_workload_selection_full_size_sampled():
    """The decode workload (64 requests, U[1024, 32768], Hq 32 / Hkv 8, bs 16)
    with 1/8 of each request's blocks selected plus its last block, the
    library's split; the oracle recomputes 4 sampled requests."""
    case = synth.decode_workload(seed=2, device=DEV)
    dc = cache_case(case, DEV)
    sel = synth.sparse_selection(case.layout, 0.125, seed=51)
    out = run_sparse(case, dc, sel, max_context=16 * sel.block_tables.shape[1])
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    picks = [0, 17, 40, 63]
    bs = 16
    # compact host copy of the sampled requests' selected blocks
    blocks = torch.unique(torch.cat([sel.block_tables[b, :int((sel.block_valid[b] > 0).sum()) or 1]
                                     for b in picks]).long())
    remap = {int(x): i for i, x in enumerate(blocks.tolist())}
    NB = dc.S // bs
    idx = blocks.to(DEV)
    kc = dc.k_cache.view(NB, bs, dc.H, dc.D)[idx].reshape(-1, dc.H, dc.D).cpu().numpy()
    vc = dc.v_cache.view(NB, bs, dc.H, dc.D)[idx].reshape(-1, dc.H, dc.D).cpu().numpy()
    kp = dc.k_plane.view(dc.H, NB, bs)[:, idx].reshape(dc.H, -1).cpu().numpy()
    vp = dc.v_plane.view(dc.H, NB, bs)[:, idx].reshape(dc.H, -1).cpu().numpy()
    bt = sel.block_tables[picks].clone()
    bv = sel.block_valid[picks].clone()
    for i in range(len(picks)):
        for j in range(bt.shape[1]):
            bt[i, j] = remap.get(int(bt[i, j]), 0) if bv[i, j] > 0 else 0
    sub = synth.SparseSelection(bt, bv, sel.context_lens[picks].clone())
    sub_case = synth.DecodeCase("sparse-sub", case.layout, None, None, case.q[picks],
                                32, 8, 128, 1, case.softmax_scale)
    ref = oracle_sparse(sub_case, (kc, vc, kp.T, vp.T), sub, q=case.q[picks])
    assert_attn_close(out[picks].cpu().numpy(), ref, "sparse decode sampled")
