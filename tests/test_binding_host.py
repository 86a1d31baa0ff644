"""Host-side geometry checks of the Python binding (no GPU needed, nothing
is launched): every mismatch between the tensors of a call -- one that
would make a kernel read or write outside an allocation -- raises
ValueError before the device check and before any launch. CPU tensors
with a consistent geometry reach the device check, which names it."""
import pytest
import torch

import fp8_e4m3_paged_kv_amd as fk

S, H, D, BS = 64, 2, 128, 16
B, R, HQ = 2, 1, 8


def caches(S=S, H=H, D=D):
    kc = torch.zeros((S, H, D), dtype=torch.uint8)
    return kc, torch.zeros_like(kc)


def planes(S=S, H=H):
    kp = torch.zeros((H, S))
    return kp.t(), torch.zeros((H, S)).t()


def store_args(**over):
    kc, vc = caches()
    ks, vs = planes()
    a = dict(k=torch.zeros((4, H, D), dtype=torch.bfloat16),
             v=torch.zeros((4, H, D), dtype=torch.bfloat16),
             slot_ids=torch.zeros(4, dtype=torch.int64), k_cache=kc, v_cache=vc,
             k_scale=ks, v_scale=vs)
    a.update(over)
    return a


def decode_args(**over):
    kc, vc = caches()
    ks, vs = planes()
    a = dict(q=torch.zeros((B, R, HQ, D), dtype=torch.bfloat16), k_cache=kc,
             v_cache=vc, k_scale=ks, v_scale=vs,
             block_tables=torch.zeros((B, 2), dtype=torch.int32),
             context_lens=torch.zeros(B, dtype=torch.int32))
    kw = dict(num_kv_heads=H, block_size=BS, softmax_scale=0.088, max_context=32)
    for k, v in over.items():
        (kw if k in kw else a)[k] = v
    return a, kw


def expect(fn, words):
    with pytest.raises(ValueError) as ei:
        fn()
    msg = str(ei.value)
    assert words in msg, msg
    assert "GPU" not in msg or words == "GPU", msg


def test_store_geometry_mismatches_raise():
    call = lambda **o: fk.kv_quant_scatter(**store_args(**o))
    expect(lambda: call(v_cache=torch.zeros((S - 16, H, D), dtype=torch.uint8)),
           "share shape")
    kp = torch.zeros((H, S - 1)).t()
    expect(lambda: call(k_scale=kp, v_scale=kp), "scale plane covers")
    kp3 = torch.zeros((H + 1, S)).t()
    expect(lambda: call(k_scale=kp3, v_scale=kp3), "scale plane covers")
    ks, _ = planes()
    expect(lambda: call(v_scale=torch.zeros((S, H))), "share strides")
    wide = torch.zeros((S, H, 2 * D), dtype=torch.uint8)[:, :, ::2]
    expect(lambda: call(k_cache=wide, v_cache=wide), "contiguous")
    expect(lambda: call(k_cache=torch.zeros((S, H, D), dtype=torch.int8)), "uint8")
    expect(lambda: call(k_scale=torch.zeros((S, H), dtype=torch.float64)), "float32")
    expect(lambda: call(slot_ids=torch.zeros(5, dtype=torch.int64)), "slot_ids")
    expect(lambda: call(), "GPU")


def test_unscaled_store_geometry_mismatches_raise():
    kc, vc = caches()
    k = torch.zeros((4, H, D), dtype=torch.bfloat16)
    sl = torch.zeros(4, dtype=torch.int64)
    expect(lambda: fk.kv_quant_scatter_unscaled(k, k, sl, kc, torch.zeros((S, H, 64), dtype=torch.uint8)),
           "share shape")
    expect(lambda: fk.kv_quant_scatter_unscaled(k, k, sl, kc, vc), "GPU")


@pytest.mark.parametrize("fn", ["dense", "partials", "unscaled", "sparse"])
def test_decode_geometry_mismatches_raise(fn):
    def call(**over):
        a, kw = decode_args(**over)
        if fn == "dense":
            return fk.paged_decode_attn_fp8(**a, **kw)
        if fn == "partials":
            return fk.paged_decode_partials(**a, **kw)
        if fn == "unscaled":
            a.pop("k_scale"), a.pop("v_scale")
            return fk.paged_decode_attn_unscaled(**a, **kw)
        bt = a["block_tables"]
        return fk.sparse_decode_attn_fp8(**a, block_valid=torch.zeros_like(bt), **kw)

    expect(lambda: call(context_lens=torch.zeros(B + 1, dtype=torch.int32)), "entries for")
    expect(lambda: call(block_tables=torch.zeros((B - 1, 2), dtype=torch.int32)), "rows for")
    expect(lambda: call(max_context=33), "cover")
    expect(lambda: call(v_cache=torch.zeros((S + 16, H, D), dtype=torch.uint8)), "share shape")
    expect(lambda: call(num_kv_heads=H + 1), "cache geometry")
    if fn != "unscaled":
        kp = torch.zeros((H, S + 16)).t()
        expect(lambda: call(k_scale=kp, v_scale=kp), "scale plane covers")
    expect(lambda: call(block_tables=torch.zeros((B, 2), dtype=torch.int64)), "int32")
    expect(lambda: call(), "GPU")


def test_prefill_geometry_mismatches_raise():
    def call(q_lens=None, **over):
        a, kw = decode_args(**over)
        a["q"] = torch.zeros((B, 16, HQ, D), dtype=torch.bfloat16)
        ql = torch.zeros(B, dtype=torch.int32) if q_lens is None else q_lens
        return fk.prefill_attn_fp8(**a, q_lens=ql, **kw)

    expect(lambda: call(q_lens=torch.zeros(B - 1, dtype=torch.int32)), "entries for")
    expect(lambda: call(context_lens=torch.zeros(B + 1, dtype=torch.int32)), "entries for")
    expect(lambda: call(block_tables=torch.zeros((B - 1, 2), dtype=torch.int32)), "rows for")
    expect(lambda: call(max_context=40), "cover")
    kp = torch.zeros((H, S // 2)).t()
    expect(lambda: call(k_scale=kp, v_scale=kp), "scale plane covers")
    expect(lambda: call(), "GPU")


def test_block_shaped_views_are_accepted():
    """[NB, bs, H, D] codes with [NB, bs, H] scale views of the same pool
    pass the geometry checks (and stop at the device check)."""
    kc = torch.zeros((S // BS, BS, H, D), dtype=torch.uint8)
    kp = torch.zeros((S // BS, BS, H))
    a = store_args(k_cache=kc, v_cache=kc.clone(), k_scale=kp, v_scale=kp.clone())
    expect(lambda: fk.kv_quant_scatter(**a), "GPU")
    bad = torch.zeros((S // BS - 1, BS, H))
    a = store_args(k_cache=kc, v_cache=kc.clone(), k_scale=bad, v_scale=bad.clone())
    expect(lambda: fk.kv_quant_scatter(**a), "scale plane covers")
