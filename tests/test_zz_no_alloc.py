"""fp8kv_paged_decode_attn_fp8_noalloc (the decode entry point that
allocates nothing) through the C ABI: its output equals, bit for bit, that
of fp8kv_paged_decode_attn_fp8 with a caller workspace and the same split,
and meets the attention bar against the oracle -- on two calls in a row,
the second with a smaller input, so the library's scratch array holds the
first call's partials when the second one runs."""
import pytest
import torch

import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import assert_attn_close, bf16_rne, cache_case, log, oracle_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"
E_WORKSPACE = -6


def both(case, dc, out_dtype, num_ranges=0):
    L = case.layout
    q = case.q.to(DEV)
    bt, cl = L.block_tables.to(DEV), L.context_lens.to(DEV)
    kw = dict(num_kv_heads=case.num_kv_heads, block_size=L.block_size,
              softmax_scale=case.softmax_scale,
              max_context=int(L.context_lens.max()), num_ranges=num_ranges)
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=DEV)
    fk.paged_decode_attn_fp8_noalloc(q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                                     bt, cl, out, **kw)
    ref = fk.paged_decode_attn_fp8(q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                                   bt, cl, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_two_calls_second_smaller(out_dtype):
    big = synth.decode_case([5000, 1, 3000, 12000, 777, 64, 2048, 9000], 32, 8, 128, 16,
                            rows=1, seed=130)
    small = synth.decode_case([300, 41], 16, 4, 128, 64, rows=4, seed=131,
                              k_outlier_frac=0.005)
    for name, case, nr in (("first call (8 requests)", big, 0),
                           ("second call (2 requests, 4 verify rows)", small, 0)):
        log(f"no-alloc decode, {name}, {out_dtype}")
        dc = cache_case(case, DEV)
        out, ref = both(case, dc, out_dtype, nr)
        assert torch.equal(out, ref), f"{name}: differs from the workspace call"
        if out_dtype == torch.float32:
            assert_attn_close(out.cpu().numpy(), oracle_decode(case, dc.host()), name)
        else:
            f32 = both(case, dc, torch.float32, nr)[0]
            assert torch.equal(out, bf16_rne(f32)), f"{name}: bf16 is not RNE of fp32"


def test_explicit_split_and_scratch_limit():
    """An explicit split gives the workspace call's bits; sizes whose
    partials exceed the scratch are refused before anything is launched."""
    case = synth.decode_case([900, 33, 4000], 8, 2, 128, 16, rows=1, seed=132)
    dc = cache_case(case, DEV)
    out, ref = both(case, dc, torch.float32, num_ranges=37)
    assert torch.equal(out, ref)
    need = fk.decode_workspace_bytes(3, 1, 8, 2, 128, 1 << 16)
    assert need > fk.NOALLOC_SCRATCH_BYTES
    L = case.layout
    sentinel = torch.full(case.q.shape, 5.0, device=DEV)
    with pytest.raises(fk.Fp8KvError) as e:
        fk.paged_decode_attn_fp8_noalloc(
            case.q.to(DEV), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
            L.block_tables.to(DEV), L.context_lens.to(DEV), sentinel, num_kv_heads=2,
            block_size=16, softmax_scale=case.softmax_scale,
            max_context=int(L.context_lens.max()), num_ranges=1 << 16)
    assert e.value.status == E_WORKSPACE, str(e.value)
    torch.cuda.synchronize()
    assert torch.all(sentinel == 5.0)
