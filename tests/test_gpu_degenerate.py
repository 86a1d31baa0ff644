"""Calls with nothing to do, through the binding with empty tensors (which
have no storage): each returns normally and writes nothing. The cache and
scale buffers are sentinel-filled and checked after every call."""
import pytest
import torch

import fp8_e4m3_paged_kv_amd as fk

from gpu_cases import SCALE_SENTINEL, SENTINEL, DevCache, log

pytestmark = pytest.mark.gpu
DEV = "cuda"


def untouched(dc):
    return (bool((dc.k_cache == SENTINEL).all()) and bool((dc.v_cache == SENTINEL).all())
            and bool((dc.k_plane == SCALE_SENTINEL).all())
            and bool((dc.v_plane == SCALE_SENTINEL).all()))


def test_store_of_no_tokens():
    log("store of 0 tokens")
    dc = DevCache(64, 2, 128, DEV)
    k = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=DEV)
    slots = torch.empty(0, dtype=torch.int64, device=DEV)
    fk.kv_quant_scatter(k, k, slots, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale)
    fk.kv_quant_scatter_unscaled(k, k, slots, dc.k_cache, dc.v_cache)
    torch.cuda.synchronize()
    assert untouched(dc)


@pytest.mark.parametrize("fused_call", ["dense", "sparse", "partials"])
def test_decode_of_no_requests(fused_call):
    log(f"decode of 0 requests ({fused_call})")
    dc = DevCache(64, 2, 128, DEV)
    q = torch.empty((0, 1, 8, 128), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    cl = torch.zeros(0, dtype=torch.int32, device=DEV)
    kw = dict(num_kv_heads=2, block_size=16, softmax_scale=128 ** -0.5,
              max_context=64, num_ranges=4)
    if fused_call == "dense":
        out = fk.paged_decode_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale,
                                       dc.v_scale, bt, cl, **kw)
        assert out.shape == q.shape
    elif fused_call == "sparse":
        out = fk.sparse_decode_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale,
                                        dc.v_scale, bt, bt.clone(), cl, **kw)
        assert out.shape == q.shape
    else:
        ws = fk.paged_decode_partials(q, dc.k_cache, dc.v_cache, dc.k_scale,
                                      dc.v_scale, bt, cl, **kw)
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
        fk.paged_decode_merge(ws, out, rows=1, num_q_heads=8, num_kv_heads=2,
                              num_ranges=4)
    torch.cuda.synchronize()
    assert untouched(dc)


def test_prefill_of_no_requests():
    log("prefill of 0 requests")
    dc = DevCache(64, 2, 128, DEV)
    q = torch.empty((0, 0, 8, 128), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    cl = torch.zeros(0, dtype=torch.int32, device=DEV)
    out = fk.prefill_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                              bt, cl, cl.clone(), num_kv_heads=2, block_size=16,
                              softmax_scale=128 ** -0.5, max_context=64)
    torch.cuda.synchronize()
    assert out.shape == q.shape
    assert untouched(dc)


@pytest.mark.parametrize("fmt", [fk.KEYS_MXFP4, fk.KEYS_E4M3])
def test_index_calls_with_no_keys(fmt):
    log(f"index keys / scorer with 0 keys, format {fmt}")
    keys = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    codes, scales = fk.index_keys_quantize(keys, fmt)
    torch.cuda.synchronize()
    assert codes.shape[0] == 0 and scales.shape[0] == 0
    q = torch.zeros((1, 2, 4, 128), dtype=torch.bfloat16, device=DEV)
    w = torch.ones((1, 2, 4), dtype=torch.float32, device=DEV)
    out = fk.index_score_mxfp4(q, w, fmt, codes.unsqueeze(0), scales.unsqueeze(0))
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0)
