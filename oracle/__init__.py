"""CPU oracle for the FP8 E4M3 paged KV cache -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its binding in ``fp8_e4m3_paged_kv_amd``) never touches it, and the two share
no code.

The arithmetic lives in plain C (``oracle/*.c``, built into
``oracle/liboracle.so``); this module only marshals numpy arrays. Every
function cites, in the C sources, the page passage it follows.

Arrays: bf16 data is passed as ``numpy.uint16`` bit patterns; strided views
are accepted as they are (their element strides are passed to C).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = ["e4m3.c", "quant.c", "attn.c", "index.c"]

E4M3 = 0
E5M2 = 1
KEYS_MXFP4 = 0
KEYS_E4M3 = 1

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so (strict IEEE:
    no contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp"]
    cmd += [os.path.join(_HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    D = ctypes.c_double
    lib.fo_decode.argtypes = [I, ctypes.c_uint]
    lib.fo_decode.restype = D
    lib.fo_encode.argtypes = [I, ctypes.c_float]
    lib.fo_encode.restype = ctypes.c_uint
    lib.fo_fmt_max.argtypes = [I]
    lib.fo_fmt_max.restype = D
    lib.fo_encode_array.argtypes = [I, P, I64, P]
    lib.fo_decode_array.argtypes = [I, P, I64, P]
    lib.fo_quantize_row.argtypes = [I, P, I64, P, P]
    lib.fo_quantize_rows_bf16.argtypes = [I, P, I64, I64, I64, P, P]
    lib.fo_kv_quant_scatter_bf16.argtypes = [P, I64, I64, P, I64, I64,
                                             I64, I64, I64, P, I64,
                                             P, P, I64, I64, P, P, I64, I64]
    lib.fo_kv_scatter_unscaled_bf16.argtypes = [I, P, I64, I64, P, I64, I64,
                                                I64, I64, I64, P, I64,
                                                P, P, I64, I64]
    lib.fo_attend_dense.argtypes = [P, P, P, I64, I64, D, P]
    lib.fo_paged_decode_attn.argtypes = [I, P, I64, I64, I64, P, P, I64, I64,
                                         P, P, I64, I64, P, I64, P,
                                         I64, I64, I64, I64, I64, I64, D, I64,
                                         P, I64, P]
    lib.fo_sparse_decode_attn.argtypes = [I, P, I64, I64, I64, P, P, I64, I64,
                                          P, P, I64, I64, P, I64, P, I64, P,
                                          I64, I64, I64, I64, I64, I64, D,
                                          P, I64, P]
    lib.fo_e2m1_value.argtypes = [ctypes.c_uint]
    lib.fo_e2m1_value.restype = D
    lib.fo_e8m0_value.argtypes = [ctypes.c_uint]
    lib.fo_e8m0_value.restype = D
    lib.fo_mxfp4_encode_group.argtypes = [P, P, P]
    lib.fo_index_keys_mxfp4.argtypes = [P, I64, I64, I64, P, I64, P, I64]
    lib.fo_index_keys_pool.argtypes = [P, I64, I64, I64, I64, P]
    lib.fo_bf16_rne.argtypes = [D]
    lib.fo_bf16_rne.restype = ctypes.c_uint16
    lib.fo_index_keys_build_bf16.argtypes = [P, I64, I64, I64, I64, P]
    lib.fo_index_score.argtypes = [I, P, I64, I64, I64, P, I64, I64, I64,
                                   P, I64, I64, P, I64, I64,
                                   I64, I64, I64, I64, I64, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _estrides(a: np.ndarray):
    return [s // a.itemsize for s in a.strides]


def fmt_max(fmt: int = E4M3) -> float:
    return _load().fo_fmt_max(fmt)


def decode(codes, fmt: int = E4M3) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    _load().fo_decode_array(fmt, _ptr(c), c.size, _ptr(out))
    return out


def encode(values, fmt: int = E4M3) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    out = np.empty(v.shape, dtype=np.uint8)
    _load().fo_encode_array(fmt, _ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize_rows(x, fmt: int = E4M3):
    """Quantize each row of a float32 [N, D] array: (codes uint8 [N, D],
    scales float32 [N])."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    n, d = x.shape
    codes = np.empty((n, d), dtype=np.uint8)
    scales = np.empty((n,), dtype=np.float32)
    lib = _load()
    for i in range(n):
        lib.fo_quantize_row(fmt, _ptr(x[i]), d, _ptr(codes[i]),
                            scales[i:].ctypes.data)
    return codes, scales


def quantize_rows_bf16(x_bits, fmt: int = E4M3, threads: int = 1):
    """Quantize the rows of a uint16 (bf16 bits) [N, D] array with rows of
    unit inner stride: (codes uint8 [N, D], scales float32 [N]). With
    threads > 1 the rows are split into contiguous chunks, one per thread."""
    x = np.asarray(x_bits)
    assert x.dtype == np.uint16 and x.ndim == 2 and x.strides[1] == 2
    n, d = x.shape
    codes = np.empty((n, d), dtype=np.uint8)
    scales = np.empty((n,), dtype=np.float32)
    lib = _load()
    xs = x.strides[0] // 2

    def run(lo, hi):
        if hi > lo:
            lib.fo_quantize_rows_bf16(fmt, _ptr(x[lo:]), hi - lo, d, xs,
                                      _ptr(codes[lo:]), _ptr(scales[lo:]))
    if threads <= 1 or n < 2 * threads:
        run(0, n)
    else:
        from concurrent.futures import ThreadPoolExecutor
        step = (n + threads - 1) // threads
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda i: run(i, min(n, i + step)),
                        range(0, n, step)))
    return codes, scales


def kv_quant_scatter_bf16(k, v, slot_ids, k_cache, v_cache, k_scale, v_scale,
                          num_slots=None):
    """In-place quantize + scatter.

    k, v       uint16 (bf16 bits) views [T, H, D], last stride 1, any other
               strides (K and V each keep their own).
    slot_ids   int64 [T]; <0 or >= num_slots writes nothing.
    k_cache, v_cache  uint8 [S, H, D] views (same strides for both).
    k_scale, v_scale  float32 [S, H] views (same strides for both).
    """
    assert k.dtype == np.uint16 and v.dtype == np.uint16
    assert k.shape == v.shape and k.ndim == 3
    T, H, D = k.shape
    ks, vs = _estrides(k), _estrides(v)
    assert ks[2] == 1 and vs[2] == 1
    slots = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int64))
    assert slots.shape == (T,)
    cs, ss = _estrides(k_cache), _estrides(k_scale)
    assert _estrides(v_cache) == cs and _estrides(v_scale) == ss and cs[2] == 1
    if num_slots is None:
        num_slots = k_cache.shape[0]
    _load().fo_kv_quant_scatter_bf16(
        _ptr(k), ks[0], ks[1], _ptr(v), vs[0], vs[1], T, H, D,
        _ptr(slots), num_slots, _ptr(k_cache), _ptr(v_cache), cs[0], cs[1],
        _ptr(k_scale), _ptr(v_scale), ss[0], ss[1])


def kv_scatter_unscaled_bf16(fmt, k, v, slot_ids, k_cache, v_cache, num_slots=None):
    """In-place unscaled encode + scatter (no scale planes): every element is
    encoded by itself in fmt (E4M3 or E5M2), saturating. Views as in
    kv_quant_scatter_bf16."""
    assert k.dtype == np.uint16 and v.dtype == np.uint16
    assert k.shape == v.shape and k.ndim == 3
    T, H, D = k.shape
    ks, vs = _estrides(k), _estrides(v)
    assert ks[2] == 1 and vs[2] == 1
    slots = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int64))
    assert slots.shape == (T,)
    cs = _estrides(k_cache)
    assert _estrides(v_cache) == cs and cs[2] == 1
    if num_slots is None:
        num_slots = k_cache.shape[0]
    _load().fo_kv_scatter_unscaled_bf16(
        int(fmt), _ptr(k), ks[0], ks[1], _ptr(v), vs[0], vs[1], T, H, D,
        _ptr(slots), num_slots, _ptr(k_cache), _ptr(v_cache), cs[0], cs[1])


def attend_dense(q, keys, vals, scale):
    q = np.ascontiguousarray(q, dtype=np.float64)
    keys = np.ascontiguousarray(keys, dtype=np.float64)
    vals = np.ascontiguousarray(vals, dtype=np.float64)
    n, d = keys.shape
    out = np.empty((d,), dtype=np.float64)
    _load().fo_attend_dense(_ptr(q), _ptr(keys), _ptr(vals), n, d, scale,
                            _ptr(out))
    return out


def paged_decode_attn(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                      context_lens, num_kv_heads, block_size, softmax_scale,
                      partition_tokens=0, rows=None, fmt: int = E4M3):
    """Paged GQA decode attention in double.

    q            uint16 (bf16 bits) [B, R, Hq, D] view, last stride 1.
    k/v_cache    uint8 [S, Hkv, D] views; k/v_scale float32 [S, Hkv] views.
    block_tables int32 [B, max_blocks] (row stride taken from the view).
    context_lens int32 [B].
    rows         optional list of flat row ids (b*R + r)*Hq + hq; output is
                 then [len(rows), D], else [B, R, Hq, D].
    """
    assert q.dtype == np.uint16 and q.ndim == 4
    B, R, Hq, D = q.shape
    qs = _estrides(q)
    assert qs[3] == 1
    cs, ss = _estrides(k_cache), _estrides(k_scale)
    assert _estrides(v_cache) == cs and _estrides(v_scale) == ss
    bt = np.asarray(block_tables, dtype=np.int32)
    assert bt.strides[1] == 4
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if rows is None:
        sel, nsel = None, 0
        out = np.empty((B, R, Hq, D), dtype=np.float64)
    else:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nsel = sel.size
        out = np.empty((nsel, D), dtype=np.float64)
    _load().fo_paged_decode_attn(
        fmt, _ptr(q), qs[0], qs[1], qs[2], _ptr(k_cache), _ptr(v_cache),
        cs[0], cs[1], _ptr(k_scale), _ptr(v_scale), ss[0], ss[1],
        _ptr(bt), bt.strides[0] // 4, _ptr(cl), B, R, Hq, num_kv_heads, D,
        block_size, float(softmax_scale), int(partition_tokens),
        None if sel is None else _ptr(sel), nsel, _ptr(out))
    return out


def sparse_decode_attn(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       block_valid, context_lens, num_kv_heads, block_size,
                       softmax_scale, rows=None, fmt: int = E4M3):
    """Decode attention over selected blocks, in double.

    block_tables int32 [B, max_sel]: the selected blocks in position order.
    block_valid  int32 [B, max_sel]: keys of each selected block, from its
                 start (0 .. block_size).
    context_lens int32 [B]: virtual positions (i * block_size + offset) of
                 the request; row r of R sees positions 0 .. len - R + r.
    Other arguments as in paged_decode_attn.
    """
    assert q.dtype == np.uint16 and q.ndim == 4
    B, R, Hq, D = q.shape
    qs = _estrides(q)
    assert qs[3] == 1
    cs, ss = _estrides(k_cache), _estrides(k_scale)
    assert _estrides(v_cache) == cs and _estrides(v_scale) == ss
    bt = np.asarray(block_tables, dtype=np.int32)
    bv = np.asarray(block_valid, dtype=np.int32)
    assert bt.strides[1] == 4 and bv.strides[1] == 4 and bv.shape == bt.shape
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if rows is None:
        sel, nsel = None, 0
        out = np.empty((B, R, Hq, D), dtype=np.float64)
    else:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nsel = sel.size
        out = np.empty((nsel, D), dtype=np.float64)
    _load().fo_sparse_decode_attn(
        fmt, _ptr(q), qs[0], qs[1], qs[2], _ptr(k_cache), _ptr(v_cache),
        cs[0], cs[1], _ptr(k_scale), _ptr(v_scale), ss[0], ss[1],
        _ptr(bt), bt.strides[0] // 4, _ptr(bv), bv.strides[0] // 4, _ptr(cl),
        B, R, Hq, num_kv_heads, D, block_size, float(softmax_scale),
        None if sel is None else _ptr(sel), nsel, _ptr(out))
    return out


# ---------------------------------------------------------------- index keys
def e2m1_value(code: int) -> float:
    return _load().fo_e2m1_value(code)


def e8m0_value(code: int) -> float:
    return _load().fo_e8m0_value(code)


def mxfp4_encode_group(x):
    """One group of 32 float32 values -> (exponent code, 16 packed bytes)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    assert x.shape == (32,)
    packed = np.zeros(16, np.uint8)
    e = np.zeros(1, np.uint8)
    _load().fo_mxfp4_encode_group(_ptr(x), _ptr(packed), _ptr(e))
    return int(e[0]), packed


def index_keys_mxfp4(keys_bits):
    """bf16 bits [N, D] (rows of unit inner stride) -> (packed uint8
    [N, D/2], exponent codes uint8 [N, D/32])."""
    k = np.asarray(keys_bits)
    assert k.dtype == np.uint16 and k.ndim == 2 and k.strides[1] == 2
    n, d = k.shape
    assert d % 32 == 0
    packed = np.zeros((n, d // 2), np.uint8)
    exps = np.zeros((n, d // 32), np.uint8)
    _load().fo_index_keys_mxfp4(_ptr(k), n, d, k.strides[0] // 2, _ptr(packed),
                                d // 2, _ptr(exps), d // 32)
    return packed, exps


def index_keys_e4m3(keys_bits, threads: int = 1):
    """bf16 bits [N, D] -> (E4M3 codes uint8 [N, D], fp32 scales [N]): the
    per-row quantizer of the KV cache applied to the keys."""
    return quantize_rows_bf16(keys_bits, E4M3, threads)


def index_keys_pool(raw_bits, g0, g1):
    """Compressed keys g0 .. g1-1 (float64 [g1 - g0, D]) of one request's
    raw bf16 keys [L, D] (bits): the mean of each group of 4 consecutive
    raw keys, L2-normalized (0 for an all-zero mean)."""
    r = np.asarray(raw_bits)
    assert r.dtype == np.uint16 and r.ndim == 2 and r.strides[1] == 2
    L, D = r.shape
    assert 0 <= g0 <= g1 and 4 * g1 <= L
    out = np.empty((g1 - g0, D), np.float64)
    _load().fo_index_keys_pool(_ptr(r), r.strides[0] // 2, D, g0, g1, _ptr(out))
    return out


def bf16_rne(x) -> np.ndarray:
    """bf16 bits (uint16) of each float64 value, rounded once to nearest,
    ties to even."""
    x = np.asarray(x, dtype=np.float64)
    f = _load().fo_bf16_rne
    return np.array([f(float(v)) for v in x.reshape(-1)], np.uint16).reshape(x.shape)


def index_keys_build(raw_bits, g0, g1, key_format):
    """Compressed keys g0 .. g1-1 of one request's raw bf16 keys [L, D]
    (bits), built end to end: pooled and normalized in double, rounded once
    to bf16, then encoded. Returns the bf16 bits [g1 - g0, D] and, for
    KEYS_MXFP4 / KEYS_E4M3, the (codes, scales) of those keys."""
    r = np.asarray(raw_bits)
    assert r.dtype == np.uint16 and r.ndim == 2 and r.strides[1] == 2
    L, D = r.shape
    assert 0 <= g0 <= g1 and 4 * g1 <= L and D <= 512
    kb = np.empty((g1 - g0, D), np.uint16)
    _load().fo_index_keys_build_bf16(_ptr(r), r.strides[0] // 2, D, g0, g1, _ptr(kb))
    if key_format == KEYS_MXFP4:
        return kb, index_keys_mxfp4(kb)
    if key_format == KEYS_E4M3:
        return kb, index_keys_e4m3(kb)
    return kb, None


def index_score(q_bits, w, key_format, codes, scales):
    """score [B, R, N] (float64) = sum_h w[b,r,h] * relu(q[b,r,h,:] . k^[b,n,:]).

    q_bits  uint16 (bf16 bits) [B, R, H, D] view, last stride 1.
    w       float32 [B, R, H] view.
    codes   uint8 [B, N, D] (E4M3) or [B, N, D/2] (MXFP4), last stride 1.
    scales  float32 [B, N] (E4M3) or uint8 [B, N, D/32] (MXFP4 exponents).
    """
    q = np.asarray(q_bits)
    assert q.dtype == np.uint16 and q.ndim == 4 and q.strides[3] == 2
    B, R, H, D = q.shape
    w = np.asarray(w, dtype=np.float32)
    assert w.shape == (B, R, H)
    qs, ws = _estrides(q), _estrides(w)
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.ndim == 3 and codes.strides[2] == 1
    N = codes.shape[1]
    if key_format == KEYS_MXFP4:
        scales = np.asarray(scales, dtype=np.uint8)
        assert scales.shape == (B, N, D // 32) and scales.strides[2] == 1
        sb, ss = scales.strides[0], scales.strides[1]
    else:
        scales = np.asarray(scales, dtype=np.float32)
        assert scales.shape == (B, N)
        sb, ss = scales.strides[0] // 4, scales.strides[1] // 4
    out = np.empty((B, R, N), np.float64)
    _load().fo_index_score(int(key_format), _ptr(q), qs[0], qs[1], qs[2],
                           _ptr(w), ws[0], ws[1], ws[2],
                           _ptr(codes), codes.strides[0], codes.strides[1],
                           _ptr(scales), sb, ss, B, R, H, D, N, _ptr(out))
    return out
