"""Pins of the compressed-index oracle (CPU): the MXFP4 key codec and the
index scorer ("fix(qwen4-exp): register the QSA FP8 scale planes for KV
offload", ROCm/ATOM #2655, description: compressed-index bullet and the
stacked-scorer paragraph).

Each pin holds outside the oracle:
* E2M1 code values = the OCP MX closed forms (1 sign, 2 exponent bits with
  bias 1, 1 mantissa bit); E8M0 code values = torch's float8_e8m0fnu;
* the group exponent is the smallest one that does not clip, checked
  against the bound 6 * 2^(e-1) < amax <= 6 * 2^e;
* every element is the nearest representable value to x / 2^e (brute force
  over all 16 codes, ties to the even code), and the reconstruction error
  is within half the local grid step;
* the scorer equals closed forms (unit-vector keys), is linear in w and
  equivariant under key permutations, applies ReLU per head (a head whose
  dots are all negative contributes nothing), and matches a float64 torch
  evaluation on keys dequantized by torch / by the table pins.
The nibble order and the zero-group code are conventions: parity unpinned
beyond oracle = kernel self-consistency.
"""
import numpy as np
import pytest
import torch

import oracle

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_is_the_ocp_format():
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        want = -mag if s else mag
        got = oracle.e2m1_value(c)
        assert got == want and np.signbit(got) == bool(s), c
    assert [oracle.e2m1_value(c) for c in range(8)] == E2M1
    assert max(abs(oracle.e2m1_value(c)) for c in range(16)) == 6.0


def test_e8m0_table_matches_torch():
    codes = torch.arange(0, 255, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.e8m0_value(int(c)) for c in codes])
    assert np.array_equal(got, ref)


def brute_code(v):
    """Nearest of the 16 E2M1 codes to v by the table above, ties to the
    even code, sign of v kept (so -0 and tiny negatives get the sign bit)."""
    best, bd = None, None
    for c in range(8):
        d = abs(E2M1[c] - abs(v))
        if bd is None or d < bd or (d == bd and c % 2 == 0 and best % 2 == 1):
            best, bd = c, d
    return best | (8 if np.signbit(v) else 0)


def unpack(packed):
    return [(int(b) >> (4 * t)) & 15 for b in packed for t in (0, 1)]


def groups(seed, n):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        scale = 2.0 ** g.integers(-20, 20)
        x = (g.standard_normal(32) * scale).astype(np.float32)
        if i % 5 == 0:
            x[g.integers(0, 32)] *= 30           # one outlier
        if i % 7 == 0:
            x[:16] = 0.0
        out.append(x)
    # exact boundary cases: amax = 6 * 2^k, just above, powers of two, ties
    k = 3
    out.append(np.full(32, 6 * 2.0 ** k, np.float32))
    out.append(np.full(32, np.nextafter(np.float32(6 * 2.0 ** k), np.float32(np.inf)), np.float32))
    out.append(np.array([2.0 ** (i % 8 - 4) for i in range(32)], np.float32))
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, np.float32)
    out.append(np.where(np.arange(32) % 2 == 0, t, -t).astype(np.float32))
    out.append(np.zeros(32, np.float32))
    out.append(np.array([-0.0] * 31 + [1.0], np.float32))
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_mxfp4_group_exponent_never_clips_and_is_minimal(seed):
    for x in groups(seed, 200):
        e_code, packed = oracle.mxfp4_encode_group(x)
        amax = float(np.max(np.abs(x.astype(np.float64))))
        if amax == 0.0:
            assert e_code == 127 and all(c & 7 == 0 for c in unpack(packed))
            continue
        e = e_code - 127
        assert amax <= 6.0 * 2.0 ** e, "group clips"
        assert amax > 6.0 * 2.0 ** (e - 1), "exponent not the smallest"


@pytest.mark.parametrize("seed", [0, 1])
def test_mxfp4_elements_are_nearest_ties_to_even(seed):
    for x in groups(seed, 200):
        e_code, packed = oracle.mxfp4_encode_group(x)
        scale = 2.0 ** (e_code - 127)
        codes = unpack(packed)
        for i, c in enumerate(codes):
            v = float(np.float64(x[i]) / scale)
            assert c == brute_code(v), (i, v, c)
            # reconstruction within half the grid step around v
            rec = oracle.e2m1_value(c) * scale
            step = {0: .5, 1: .5, 2: .5, 3: .5, 4: 1, 5: 1, 6: 2, 7: 2}[c & 7] * scale
            assert abs(rec - float(x[i])) <= step / 2 + 1e-300


def test_mxfp4_closed_forms():
    # amax = 6 * 2^3 exactly: no clip at e = 3, every element is code 7
    e, p = oracle.mxfp4_encode_group(np.full(32, 48.0, np.float32))
    assert e == 127 + 3 and unpack(p) == [7] * 32
    # powers of two within the grid's range (1/2 .. 4 under a maximum of 4)
    # are exact
    x = np.array([2.0 ** (i % 4 - 1) for i in range(32)], np.float32)
    e, p = oracle.mxfp4_encode_group(x)
    rec = [oracle.e2m1_value(c) * 2.0 ** (e - 127) for c in unpack(p)]
    assert np.array_equal(np.array(rec, np.float32), x)
    # ties at the grid midpoints go to the even code
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, np.float32)
    e, p = oracle.mxfp4_encode_group(t)
    assert e == 127 and unpack(p)[:8] == [0, 2, 2, 4, 4, 6, 6, 7]
    # nibble order: element 0 in the low nibble of byte 0 (convention)
    x = np.zeros(32, np.float32)
    x[0], x[1] = 1.0, 6.0
    e, p = oracle.mxfp4_encode_group(x)
    assert e == 127 and p[0] == (2 | (7 << 4))


def test_index_keys_mxfp4_matches_groups():
    g = np.random.default_rng(4)
    keys = torch.from_numpy(g.standard_normal((5, 128)).astype(np.float32)).to(torch.bfloat16)
    bits = keys.view(torch.int16).numpy().view(np.uint16)
    packed, exps = oracle.index_keys_mxfp4(bits)
    for i in range(5):
        for grp in range(4):
            e, p = oracle.mxfp4_encode_group(keys[i, grp * 32:(grp + 1) * 32].float().numpy())
            assert exps[i, grp] == e and np.array_equal(packed[i, grp * 16:(grp + 1) * 16], p)


# ------------------------------------------------------------------- scorer
def rand_case(seed, B=2, R=3, H=4, D=64, N=9):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, R, H, D, generator=g).to(torch.bfloat16)
    w = torch.rand(B, R, H, generator=g)
    keys = torch.randn(B, N, D, generator=g)
    keys = (keys / keys.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    return q, w, keys


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def encode_keys(keys, fmt):
    B, N, D = keys.shape
    flat = bits(keys.reshape(B * N, D))
    if fmt == oracle.KEYS_MXFP4:
        p, e = oracle.index_keys_mxfp4(flat)
        return p.reshape(B, N, D // 2), e.reshape(B, N, D // 32)
    c, s = oracle.index_keys_e4m3(flat)
    return c.reshape(B, N, D), s.reshape(B, N)


def dequant_independent(codes, scales, fmt, D):
    """Dequantize without the oracle: torch's float8_e4m3fn view times the
    scale, or the pinned E2M1 table times 2^(e-127)."""
    if fmt == oracle.KEYS_E4M3:
        v = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64)
        return v * torch.from_numpy(scales.astype(np.float64))[..., None]
    lo = codes & 15
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], codes.shape[1], D)
    table = np.array([oracle.e2m1_value(c) for c in range(16)])
    val = table[nib]
    exp = np.repeat(scales.astype(np.float64) - 127, 32, axis=-1)
    return torch.from_numpy(val * np.exp2(exp))


@pytest.mark.parametrize("fmt", [oracle.KEYS_E4M3, oracle.KEYS_MXFP4])
def test_scorer_matches_float64_torch(fmt):
    q, w, keys = rand_case(7)
    codes, scales = encode_keys(keys, fmt)
    got = oracle.index_score(bits(q), w.numpy(), fmt, codes, scales)
    kd = dequant_independent(codes, scales, fmt, q.shape[-1])
    dots = torch.einsum("brhd,bnd->brhn", q.to(torch.float64), kd)
    ref = (w.to(torch.float64)[..., None] * torch.relu(dots)).sum(dim=2).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_scorer_unit_vector_keys_closed_form():
    """Keys with one nonzero element c at dim i: the score is
    sum_h w_h * max(0, q_h[i] * c^), with c^ that element dequantized
    independently of the oracle."""
    B, R, H, D, N = 1, 2, 3, 64, 5
    q, w, _ = rand_case(3, B, R, H, D, N)
    keys = torch.zeros(B, N, D)
    idx = [0, 7, 31, 32, 63]
    for n, i in enumerate(idx):
        keys[0, n, i] = 0.5 * (n + 1) * (-1) ** n
    keys = keys.to(torch.bfloat16)
    for fmt in (oracle.KEYS_E4M3, oracle.KEYS_MXFP4):
        codes, scales = encode_keys(keys, fmt)
        got = oracle.index_score(bits(q), w.numpy(), fmt, codes, scales)
        kd = dequant_independent(codes, scales, fmt, D).numpy()
        qf = q.float().numpy().astype(np.float64)
        for n, i in enumerate(idx):
            c = kd[0, n, i]
            assert np.count_nonzero(kd[0, n]) == 1
            want = (w.numpy().astype(np.float64)[0] * np.maximum(qf[0, :, :, i] * c, 0)).sum(axis=1)
            assert np.allclose(got[0, :, n], want, rtol=1e-13, atol=0), fmt


def test_scorer_relu_linearity_and_permutation():
    q, w, keys = rand_case(11)
    fmt = oracle.KEYS_E4M3
    codes, scales = encode_keys(keys, fmt)
    base = oracle.index_score(bits(q), w.numpy(), fmt, codes, scales)
    # linear in w (a factor of 2 is exact in fp32)
    w2 = (w * 2).numpy()
    assert np.array_equal(oracle.index_score(bits(q), w2, fmt, codes, scales), 2 * base)
    # key permutation permutes the scores
    perm = np.array([4, 0, 8, 1, 7, 2, 6, 3, 5])
    pb = oracle.index_score(bits(q), w.numpy(), fmt, codes[:, perm], scales[:, perm])
    assert np.allclose(pb, base[:, :, perm], rtol=1e-12)
    # ReLU per head: with all-positive keys and head 0's q all negative,
    # head 0's dots are all negative and its weight changes nothing
    kpos = keys.float().abs().to(torch.bfloat16)
    cpos, spos = encode_keys(kpos, fmt)
    qn = q.clone()
    qn[:, :, 0] = -q[:, :, 0].float().abs().to(torch.bfloat16)
    wa, wb = w.clone(), w.clone()
    wa[:, :, 0], wb[:, :, 0] = 0.0, 5.0
    sa = oracle.index_score(bits(qn), wa.numpy(), fmt, cpos, spos)
    sb = oracle.index_score(bits(qn), wb.numpy(), fmt, cpos, spos)
    assert np.array_equal(sa, sb)
    # and a head with positive dots does change it
    wc = w.clone()
    wc[:, :, 1] += 1.0
    assert np.all(oracle.index_score(bits(qn), wc.numpy(), fmt, cpos, spos) >= sa)


# ---------------------------------------------------------------- key builder
def pool_torch(raw_bits, g0, g1):
    x = torch.from_numpy(raw_bits.astype(np.int32) << 16).view(torch.float32).double()
    m = x[4 * g0:4 * g1].reshape(g1 - g0, 4, -1).mean(dim=1)
    return torch.nn.functional.normalize(m, dim=1).numpy()


def bf16_bits_of(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_pooling_matches_torch_mean_and_normalize():
    g = torch.Generator().manual_seed(3)
    raw = bf16_bits_of(torch.randn((4 * 37, 128), generator=g).numpy())
    got = oracle.index_keys_pool(raw, 0, 37)
    assert np.abs(got - pool_torch(raw, 0, 37)).max() < 1e-15
    assert np.allclose(np.linalg.norm(got, axis=1), 1.0, atol=1e-15)


def test_pooling_closed_forms():
    x = np.zeros((8, 128), np.float32)
    x[0:4, 5] = 3.0
    x[0:4, 9] = -4.0                     # four identical keys -> (0.6, -0.8)
    x[4:8] = 0.0                         # an all-zero group -> 0
    got = oracle.index_keys_pool(bf16_bits_of(x), 0, 2)
    want = np.zeros((2, 128))
    want[0, 5], want[0, 9] = 0.6, -0.8
    assert np.abs(got - want).max() < 1e-15
    # scaling every raw key by 2 changes nothing
    g = torch.Generator().manual_seed(4)
    r = torch.randn((16, 128), generator=g).numpy()
    a = oracle.index_keys_pool(bf16_bits_of(r), 0, 4)
    b = oracle.index_keys_pool(bf16_bits_of(2 * r), 0, 4)
    assert np.array_equal(a, b)


def test_groups_follow_positions_not_chunks():
    """A group straddling two prefill chunks is the group of its positions:
    building [0, 5) and [5, 9) equals building [0, 9)."""
    g = torch.Generator().manual_seed(5)
    raw = bf16_bits_of(torch.randn((36, 128), generator=g).numpy())
    whole = oracle.index_keys_pool(raw, 0, 9)
    parts = np.concatenate([oracle.index_keys_pool(raw, 0, 5), oracle.index_keys_pool(raw, 5, 9)])
    assert np.array_equal(whole, parts)
    # a group's value depends on its four rows only
    raw2 = raw.copy()
    raw2[20:24] = bf16_bits_of(np.full((4, 128), 7.0, np.float32))
    diff = np.abs(oracle.index_keys_pool(raw2, 0, 9) - whole).max(axis=1)
    assert np.all(diff[[0, 1, 2, 3, 4, 6, 7, 8]] == 0) and diff[5] > 0


# ------------------------------------------- bf16 rounding of the pooled keys
def bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_bf16_rne_matches_torch_on_float_inputs():
    """Inputs that are exact floats: torch's float32 -> bfloat16 cast (round
    to nearest even) is the reference. Every midpoint between consecutive
    bf16 values of a few binades, its float neighbours, log-uniform values
    of both signs, and bf16 subnormals."""
    base = np.arange(0x3E00, 0x4100, dtype=np.uint32)          # 0.125 .. 8
    lo = (base << 16).view(np.float32)
    mids = ((base << 16) | 0x8000).view(np.float32)            # exact midpoints
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    g = np.random.default_rng(7)
    logu = (np.exp(g.uniform(-80, 80, 20000)) * g.choice([-1, 1], 20000)).astype(np.float32)
    sub = (np.arange(1, 300, dtype=np.float64) * 2.0 ** -134).astype(np.float32)
    x = np.concatenate([lo, mids, up, dn, -mids, logu, sub, -sub, [0.0, -0.0]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(x.astype(np.float64))
    assert np.array_equal(got, want), int((got != want).sum())


def test_bf16_rne_rounds_once_from_double():
    """Doubles within a float ulp of a bf16 midpoint round to the side they
    lie on (a detour through float would make them ties)."""
    base = np.arange(0x3F00, 0x4000, dtype=np.uint32)          # 0.5 .. 2
    mid = bf16_value(base) + 0.5 * (bf16_value(base + 1) - bf16_value(base))
    eps = mid * 2.0 ** -40
    assert np.array_equal(oracle.bf16_rne(mid + eps), base + 1)
    assert np.array_equal(oracle.bf16_rne(mid - eps), base)
    # exact ties go to the even last bit
    even = np.where(base % 2 == 0, base, base + 1)
    assert np.array_equal(oracle.bf16_rne(mid), even)


def test_index_keys_build_is_pool_then_torch_rounding_then_encode():
    """End to end: the built bf16 keys equal torch's float64 mean and
    normalization rounded to bf16 (wherever a detour through float cannot
    change the rounding), and the codes equal the encoders' on those keys."""
    g = torch.Generator().manual_seed(8)
    raw = bf16_bits_of(torch.randn((4 * 300, 128), generator=g).numpy())
    want64 = pool_torch(raw, 0, 300)
    want = torch.from_numpy(want64).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # exclude values within 2^-20 (relative) of a bf16 midpoint
    lo = bf16_value(want)
    step = np.abs(bf16_value(want + np.uint16(1)) - lo)
    near = np.abs(np.abs(want64 - lo) - 0.5 * step) <= 2.0 ** -20 * np.abs(want64)
    for fmt in (oracle.KEYS_MXFP4, oracle.KEYS_E4M3):
        kb, enc = oracle.index_keys_build(raw, 0, 300, fmt)
        assert np.array_equal(kb[~near], want[~near])
        ref = oracle.index_keys_mxfp4(kb) if fmt == oracle.KEYS_MXFP4 else oracle.index_keys_e4m3(kb)
        for a, b in zip(enc, ref):
            assert np.array_equal(np.asarray(a), np.asarray(b))
