"""The library's checked mode on the GPU: host pointers and out-of-range
device ids are refused before anything is enqueued ("feat(kvcache): store
the KV cache as fp8 e4m3 codes", FreeToken #354, review thread: a CPU tensor
reached the kernel; out-of-range ids are undefined on the fast path), valid
calls give the same bits as in the default mode, and the mode refuses to
run under graph capture.

Every refusal here is decided on the host: no kernel ever sees a bad
pointer or id."""
import numpy as np
import pytest
import torch

import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import cache_case, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
E_UNSUPPORTED, E_NOT_DEVICE, E_RANGE = -5, -8, -9


@pytest.fixture
def checked():
    prev = fk.set_checked(True)
    try:
        yield
    finally:
        fk.set_checked(prev)


def decode_kw(case):
    return dict(num_kv_heads=case.num_kv_heads, block_size=case.layout.block_size,
                softmax_scale=case.softmax_scale,
                max_context=int(case.layout.context_lens.max()))


def run_dense(case, dc, bt=None, cl=None, **over):
    L = case.layout
    kw = decode_kw(case)
    kw.update(over)
    return fk.paged_decode_attn_fp8(
        case.q.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
        (L.block_tables if bt is None else bt).to(DEV),
        (L.context_lens if cl is None else cl).to(DEV), out_dtype=torch.float32, **kw)


def expect(status, fn):
    with pytest.raises(fk.Fp8KvError) as e:
        fn()
    assert e.value.status == status, str(e.value)
    log(f"refused: {e.value}")


def test_set_checked_returns_previous():
    prev = fk.set_checked(True)
    try:
        assert fk.set_checked(True) is True
        assert fk.set_checked(False) is True
        assert fk.set_checked(False) is False
    finally:
        fk.set_checked(prev)


def test_valid_calls_give_the_same_bits(checked):
    case = synth.decode_case([700, 33, 2000], 16, 4, 128, 16, rows=2, seed=90)
    dc = cache_case(case, DEV)
    got = run_dense(case, dc, num_ranges=9)
    torch.cuda.synchronize()
    fk.set_checked(False)
    ref = run_dense(case, dc, num_ranges=9)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)

    # the quantizer, with padding slot ids (< 0), in checked mode
    fk.set_checked(True)
    g = synth.gen(91, DEV)
    k = synth.normal_bf16((8, 4, 128), g, device=DEV)
    v = synth.normal_bf16((8, 4, 128), g, device=DEV)
    slots = torch.tensor([3, -1, 7, 0, -5, 11, 2, 9], dtype=torch.int64, device=DEV)
    dc2 = cache_case(case, DEV)
    fk.kv_quant_scatter(k, v, slots, dc2.k_cache, dc2.v_cache, dc2.k_scale, dc2.v_scale)
    fk.set_checked(False)
    dc3 = cache_case(case, DEV)
    fk.kv_quant_scatter(k, v, slots, dc3.k_cache, dc3.v_cache, dc3.k_scale, dc3.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(dc2.k_cache, dc3.k_cache) and torch.equal(dc2.v_plane, dc3.v_plane)


def test_host_pointers_are_refused(checked):
    case = synth.decode_case([300, 90], 8, 2, 128, 16, rows=1, seed=92)
    dc = cache_case(case, DEV)
    L = case.layout
    q = case.q.to(DEV)
    args, ws = fk._decode_args(q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                               L.block_tables.to(DEV), L.context_lens.to(DEV),
                               case.num_kv_heads, L.block_size, case.softmax_scale,
                               int(L.context_lens.max()), 0, None)
    stream = torch.cuda.current_stream().cuda_stream
    pinned = torch.empty(q.shape, dtype=q.dtype, pin_memory=True)
    pageable = np.zeros(q.numel() + 64, dtype=np.uint16)
    page_ptr = (pageable.ctypes.data + 15) // 16 * 16
    for host_ptr, what in ((pinned.data_ptr(), "pinned host q"), (page_ptr, "pageable host q")):
        bad = list(args)
        bad[0] = host_ptr
        st = fk.lib().fp8kv_paged_decode_partials(*bad, stream)
        log(f"{what}: status {st}: {fk.lib().fp8kv_last_error().decode()}")
        assert st == E_NOT_DEVICE
    # a host block table
    bad = list(args)
    host_bt = torch.empty(L.block_tables.shape, dtype=torch.int32, pin_memory=True)
    bad[14] = host_bt.data_ptr()
    assert fk.lib().fp8kv_paged_decode_partials(*bad, stream) == E_NOT_DEVICE
    torch.cuda.synchronize()


def test_out_of_range_ids_are_refused(checked):
    case = synth.decode_case([300, 90], 8, 2, 128, 16, rows=1, seed=93)
    dc = cache_case(case, DEV)
    L = case.layout
    num_blocks = dc.S // L.block_size
    # a context length above max_context
    cl = L.context_lens.clone()
    cl[1] = 301
    expect(E_RANGE, lambda: run_dense(case, dc, cl=cl, max_context=300))
    # a negative context length
    cl = L.context_lens.clone()
    cl[0] = -1
    expect(E_RANGE, lambda: run_dense(case, dc, cl=cl))
    # a block id of a request's tokens outside the pool
    for bad_id in (num_blocks, -3):
        bt = L.block_tables.clone()
        bt[0, 4] = bad_id
        expect(E_RANGE, lambda: run_dense(case, dc, bt=bt))
    # entries past a request's last block are not read, so not checked
    bt = L.block_tables.clone()
    nb1 = (int(L.context_lens[1]) + 15) // 16
    if bt.shape[1] > nb1:
        bt[1, nb1:] = num_blocks + 100
        run_dense(case, dc, bt=bt)

    # quantize+scatter: a slot id at num_slots
    g = synth.gen(94, DEV)
    k = synth.normal_bf16((4, 2, 128), g, device=DEV)
    slots = torch.tensor([0, 5, dc.S, 1], dtype=torch.int64, device=DEV)
    expect(E_RANGE, lambda: fk.kv_quant_scatter(k, k, slots, dc.k_cache, dc.v_cache,
                                                dc.k_scale, dc.v_scale))

    # selected blocks: a valid count above the block size
    sel = synth.sparse_selection(L, 0.5, seed=95)
    bv = sel.block_valid.clone()
    bv[0, 0] = L.block_size + 1
    expect(E_RANGE, lambda: fk.sparse_decode_attn_fp8(
        case.q.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
        sel.block_tables.to(DEV), bv.to(DEV), sel.context_lens.to(DEV),
        **dict(decode_kw(case), max_context=L.block_size * sel.block_tables.shape[1])))

    # prefill: a chunk longer than its request
    pc = synth.decode_case([100, 60], 8, 2, 128, 16, rows=64, seed=96)
    pdc = cache_case(pc, DEV)
    ql = torch.tensor([64, 61], dtype=torch.int32)
    expect(E_RANGE, lambda: fk.prefill_attn_fp8(
        pc.q.to(DEV), pdc.k_cache, pdc.v_cache, pdc.k_scale, pdc.v_scale,
        pc.layout.block_tables.to(DEV), pc.layout.context_lens.to(DEV), ql.to(DEV),
        **decode_kw(pc)))
    torch.cuda.synchronize()


# the refused call leaves nothing to capture: torch's empty-graph warning is expected
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_checked_mode_refuses_graph_capture(checked):
    case = synth.decode_case([200, 64], 8, 2, 128, 16, rows=1, seed=97)
    dc = cache_case(case, DEV)
    L = case.layout
    q = case.q.to(DEV)
    bt = L.block_tables.to(DEV)
    cl = L.context_lens.to(DEV)
    out = torch.empty(q.shape, device=DEV)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    status = []
    with torch.cuda.graph(graph, stream=s):
        try:
            fk.paged_decode_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                                     bt, cl, out=out, **decode_kw(case))
        except fk.Fp8KvError as e:
            status.append(e.status)
    torch.cuda.synchronize()
    assert status == [E_UNSUPPORTED]
