"""GPU parity of fp8kv_paged_decode_append_attn_fp8 (one decode step: the
store of each request's new tokens and the attention that reads them, in
the decode's two launches).

Bar: the call equals fp8kv_kv_quant_scatter of the new rows at the page
table's slots followed by fp8kv_paged_decode_attn_fp8 with the same split,
bit for bit -- every code and scale byte of the pool and the output, fp32
and bf16 -- and its fp32 output meets the attention bar against the oracle
on the same cache. Pools start sentinel-filled, so a new row that was not
stored, or stored to the wrong slot, shows."""
import numpy as np
import pytest
import torch

import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import DevCache, assert_attn_close, bf16_rne, log, oracle_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"


def split_tokens(case):
    """Indices of the old tokens (all but each request's last R), the new
    rows k_new / v_new [B, R, Hkv, D] (zeros for positions below 0), and
    the slots of the new positions (-1 for positions below 0)."""
    L = case.layout
    R, H, D = case.rows, case.num_kv_heads, case.head_dim
    lens = L.context_lens.tolist()
    B = len(lens)
    old, slots = [], torch.full((B, R), -1, dtype=torch.int64)
    k_new = torch.zeros((B, R, H, D), dtype=torch.bfloat16)
    v_new = torch.zeros_like(k_new)
    off = 0
    for b, n in enumerate(lens):
        first = n - R
        for j in range(n):
            if j < first:
                old.append(off + j)
            else:
                k_new[b, j - first] = case.k[off + j]
                v_new[b, j - first] = case.v[off + j]
                slots[b, j - first] = L.token_slots[off + j]
        off += n
    return torch.tensor(old, dtype=torch.int64), k_new, v_new, slots


def old_cache(case, old, layout):
    dc = DevCache(case.layout.num_slots, case.num_kv_heads, case.head_dim, DEV, layout)
    if old.numel():
        dc.scatter(case.k[old].to(DEV), case.v[old].to(DEV), case.layout.token_slots[old].to(DEV))
    return dc


def kw(case, ranges):
    L = case.layout
    return dict(num_kv_heads=case.num_kv_heads, block_size=L.block_size,
                softmax_scale=case.softmax_scale,
                max_context=L.block_size * L.block_tables.shape[1], num_ranges=ranges)


def run_both(case, ranges=0, layout="head_major", out_dtype=torch.float32):
    """(append path cache, append output, reference cache, reference output)."""
    old, k_new, v_new, slots = split_tokens(case)
    L = case.layout
    q, bt, cl = case.q.to(DEV), L.block_tables.to(DEV), L.context_lens.to(DEV)
    a = old_cache(case, old, layout)
    out_a = fk.paged_decode_append_attn_fp8(
        q, k_new.to(DEV), v_new.to(DEV), a.k_cache, a.v_cache, a.k_scale, a.v_scale,
        bt, cl, out_dtype=out_dtype, **kw(case, ranges))
    r = old_cache(case, old, layout)
    flat = slots.reshape(-1)
    keep = flat >= 0
    if keep.any():
        H, D = case.num_kv_heads, case.head_dim
        fk.kv_quant_scatter(k_new.reshape(-1, H, D)[keep].to(DEV),
                            v_new.reshape(-1, H, D)[keep].to(DEV), flat[keep].to(DEV),
                            r.k_cache, r.v_cache, r.k_scale, r.v_scale)
    out_r = fk.paged_decode_attn_fp8(q, r.k_cache, r.v_cache, r.k_scale, r.v_scale, bt, cl,
                                     out_dtype=out_dtype, **kw(case, ranges))
    torch.cuda.synchronize()
    return a, out_a, r, out_r


def same_cache(a, r):
    return (torch.equal(a.k_cache, r.k_cache) and torch.equal(a.v_cache, r.v_cache)
            and torch.equal(a.k_plane.view(torch.int32), r.k_plane.view(torch.int32))
            and torch.equal(a.v_plane.view(torch.int32), r.v_plane.view(torch.int32)))


def check(case, ranges=0, layout="head_major", name=""):
    log(f"append {name}: lens={case.layout.context_lens.tolist()} R={case.rows} "
        f"Hq={case.num_q_heads} Hkv={case.num_kv_heads} D={case.head_dim} "
        f"bs={case.layout.block_size} ranges={ranges} {layout}")
    a, out_a, r, out_r = run_both(case, ranges, layout)
    assert same_cache(a, r), "the appended rows differ from the quantizer's"
    assert torch.equal(out_a, out_r), "the output differs from store-then-decode"
    assert_attn_close(out_a.cpu().numpy(), oracle_decode(case, a.host()), name)
    _, ob, _, ob_r = run_both(case, ranges, layout, torch.bfloat16)
    assert torch.equal(ob, ob_r) and torch.equal(ob, bf16_rne(out_a))
    return out_a


@pytest.mark.parametrize("ranges", [0, 1, 7, 400])
def test_single_new_token(ranges):
    case = synth.decode_case([1, 31, 33, 1000, 5000, 77], 8, 2, 128, 16, rows=1, seed=300)
    check(case, ranges, name=f"R1 ranges={ranges}")


@pytest.mark.parametrize("ranges", [0, 3, 300])
def test_verify_rows_across_two_tiles(ranges):
    """4 verify tokens; requests of 33 and 66 tokens put them in two
    32-token tiles, which a range of one tile hands to two waves; 3 tokens
    and 1 token leave positions below 0 (skipped)."""
    case = synth.decode_case([33, 66, 3, 1, 2000, 9000], 16, 4, 128, 64, rows=4, seed=301,
                             k_outlier_frac=0.005)
    check(case, ranges, name=f"R4 ranges={ranges}")


@pytest.mark.parametrize("layout", ["head_major", "interleaved", "slot_major"])
@pytest.mark.parametrize("bs", [16, 48])
def test_block_sizes_and_scale_layouts(bs, layout):
    case = synth.decode_case([300, 1290, 64], 8, 4, 128, bs, rows=2, seed=302 + bs)
    check(case, 11, layout, name=f"bs{bs}")


def test_head_dim_64_and_gqa_5():
    check(synth.decode_case([700, 129, 2], 16, 4, 64, 16, rows=2, seed=303), 5, name="D64")
    check(synth.decode_case([1, 50, 1300, 777], 30, 6, 128, 16, rows=2, seed=304), 0,
          name="G5 Hkv6")


def test_graph_capture_replays_with_new_rows():
    """One captured append call, replayed with new K/V rows, queries and
    lengths written into its device buffers; every replay equals the
    store-then-decode reference on a pool copied before the replay."""
    case = synth.decode_case([4000, 2500, 333], 8, 2, 128, 16, rows=1, seed=305)
    L = case.layout
    old, k_new0, v_new0, _ = split_tokens(case)
    dc = old_cache(case, old, "head_major")
    q = case.q.to(DEV).clone()
    kn, vn = k_new0.to(DEV).clone(), v_new0.to(DEV).clone()
    bt, cl = L.block_tables.to(DEV), L.context_lens.to(DEV).clone()
    args = kw(case, 13)
    ws = torch.empty(fk.decode_workspace_bytes(3, 1, 8, 2, 128, 13), dtype=torch.uint8, device=DEV)
    out = torch.empty(q.shape, device=DEV)
    call = lambda: fk.paged_decode_append_attn_fp8(q, kn, vn, dc.k_cache, dc.v_cache, dc.k_scale,
                                                   dc.v_scale, bt, cl, out=out, workspace=ws,
                                                   **args)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    g = synth.gen(306)
    for rep, lens in enumerate([[4000, 2500, 333], [3999, 17, 300], [4000, 1, 0]]):
        cl.copy_(torch.tensor(lens, dtype=torch.int32))
        q.copy_(synth.normal_bf16(q.shape, g))
        kn.copy_(synth.normal_bf16(kn.shape, g))
        vn.copy_(synth.normal_bf16(vn.shape, g))
        ref = DevCache(dc.S, dc.H, dc.D, DEV, "head_major")
        ref.k_cache.copy_(dc.k_cache); ref.v_cache.copy_(dc.v_cache)
        ref.k_plane.copy_(dc.k_plane); ref.v_plane.copy_(dc.v_plane)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # reference: the new row of request b at position lens[b] - 1
        slots = []
        for b, n in enumerate(lens):
            if n:
                blk = int(L.block_tables[b, (n - 1) // 16])
                slots.append(blk * 16 + (n - 1) % 16)
            else:
                slots.append(-1)
        sl = torch.tensor(slots, dtype=torch.int64, device=DEV)
        fk.kv_quant_scatter(kn[:, 0], vn[:, 0], sl, ref.k_cache, ref.v_cache,
                            ref.k_scale, ref.v_scale)
        out_r = fk.paged_decode_attn_fp8(q, ref.k_cache, ref.v_cache, ref.k_scale, ref.v_scale,
                                         bt, cl, out_dtype=torch.float32, **args)
        torch.cuda.synchronize()
        assert same_cache(dc, ref), f"replay {rep}: pool differs"
        assert torch.equal(out, out_r), f"replay {rep}: output differs"
        log(f"  replay {rep}: pool and output equal to store-then-decode")


def test_decode_workload_step_full_size():
    """The benchmark's decode step: 64 requests, lengths U[1024, 32768],
    Hq 32 / Hkv 8, bs 16, the newest token of each request appended; equal
    to store-then-decode bit for bit, pool and output."""
    case = synth.decode_workload(seed=2, device=DEV)
    L = case.layout
    lens = L.context_lens.tolist()
    last = torch.tensor(np.cumsum(lens) - 1, device=DEV)
    keep = torch.ones(case.k.shape[0], dtype=torch.bool, device=DEV)
    keep[last] = False
    slots = L.token_slots.to(DEV)
    caches = []
    for _ in range(2):
        dc = DevCache(L.num_slots, 8, 128, DEV, "head_major")
        dc.scatter(case.k[keep], case.v[keep], slots[keep])
        caches.append(dc)
    a, r = caches
    q, bt, cl = case.q.to(DEV), L.block_tables.to(DEV), L.context_lens.to(DEV)
    k_new = case.k[last].unsqueeze(1).contiguous()
    v_new = case.v[last].unsqueeze(1).contiguous()
    args = kw(case, 0)
    out_a = fk.paged_decode_append_attn_fp8(q, k_new, v_new, a.k_cache, a.v_cache, a.k_scale,
                                            a.v_scale, bt, cl, out_dtype=torch.float32, **args)
    fk.kv_quant_scatter(k_new[:, 0], v_new[:, 0], slots[last], r.k_cache, r.v_cache,
                        r.k_scale, r.v_scale)
    out_r = fk.paged_decode_attn_fp8(q, r.k_cache, r.v_cache, r.k_scale, r.v_scale, bt, cl,
                                     out_dtype=torch.float32, **args)
    torch.cuda.synchronize()
    assert same_cache(a, r)
    assert torch.equal(out_a, out_r)
