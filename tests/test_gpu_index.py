"""GPU parity of the compressed-index key encoders and the index scorer
against the oracle ("fix(qwen4-exp): register the QSA FP8 scale planes for
KV offload", ROCm/ATOM #2655, description: compressed-index bullet and the
stacked decode scorer paragraph).

Bars:
* key codes (E4M3 codes + fp32 scales; MXFP4 nibbles + E8M0 codes) equal
  the oracle's bit for bit;
* the widened keys are exact: a one-hot query reads back every E2M1 code at
  every exponent as exactly E2M1 * 2^e;
* scores: |got - ref| <= 2^-16 * sum_h |w_h| * sum_d |q_hd * k^_nd| per
  element, the forward error bound of any-order fp32 summation of the
  <= 145 terms each score adds (products of bf16 q and the exactly widened
  keys are exact in fp32), with ref the oracle's float64 score.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_paged_kv_amd as fk
from fp8_e4m3_paged_kv_amd import synth

from gpu_cases import bf16_bits, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
MX, E4 = fk.KEYS_MXFP4, fk.KEYS_E4M3
TOL = 2.0 ** -16

E2M1 = np.array([oracle.e2m1_value(c) for c in range(16)])


def dequant_keys(fmt, codes, scales):
    """k^ [B, N, 128] float64 from host codes/scales, by the oracle's
    code tables."""
    codes = np.asarray(codes)
    if fmt == MX:
        nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(
            codes.shape[:-1] + (128,))
        exps = np.asarray(scales).astype(np.int64)
        sc = np.ldexp(1.0, exps - 127)                      # [.., 4]
        return E2M1[nib] * np.repeat(sc, 32, axis=-1)
    table = oracle.decode(np.arange(256, dtype=np.uint8))
    return table[codes] * np.asarray(scales, np.float64)[..., None]


def score_bound(q_bits, w, kh):
    q = oracle.bf16_to_f32(q_bits).astype(np.float64)      # [B, R, H, D]
    B, R, H, D = q.shape
    aq = np.abs(q).reshape(B, R * H, D)
    ak = np.abs(kh)                                        # [B, N, D]
    s = np.matmul(aq, ak.transpose(0, 2, 1)).reshape(B, R, H, -1)
    return (np.abs(np.asarray(w, np.float64))[..., None] * s).sum(axis=2)


def check_scores(got, q, w, fmt, codes, scales, what):
    qb = bf16_bits(q)
    wh = w.cpu().numpy()
    ch, sh = codes.cpu().numpy(), scales.cpu().numpy()
    ref = oracle.index_score(qb, wh, fmt, ch, sh)
    kh = dequant_keys(fmt, ch, sh)
    bound = TOL * score_bound(qb, wh, kh) + 1e-37
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
    worst = float((err / bound).max()) if err.size else 0.0
    log(f"  {what}: max |err| {err.max() if err.size else 0:.3e}, "
        f"worst err/bound {worst:.3f}")
    assert np.all(err <= bound), what


def encode(keys, fmt):
    codes, scales = fk.index_keys_quantize(keys, fmt)
    torch.cuda.synchronize()
    return codes, scales


def oracle_keys(keys, fmt):
    kb = bf16_bits(keys.reshape(-1, 128))
    if fmt == MX:
        return oracle.index_keys_mxfp4(kb)
    return oracle.index_keys_e4m3(kb)


def edge_keys():
    """Rows exercising ties, group boundaries, zeros, signed zeros, bf16
    subnormals and the largest bf16 values."""
    rows = []
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    g = np.concatenate([ties, -ties, ties * 0.5, -ties * 0.5])   # amax 6 -> e = 0
    rows.append(np.concatenate([g, g * 2.0 ** -20, g * 2.0 ** 90, -g * 2.0 ** -120]))
    rows.append(np.zeros(128, np.float32))                     # all-zero groups
    r = np.zeros(128, np.float32)
    r[3], r[40], r[77], r[100] = 4.0, -6.0, 3.0 * 2.0 ** -130, 1.0e-40
    rows.append(r)                                             # lone values / subnormals
    r = np.full(128, -0.0, np.float32)
    r[::7] = 0.0
    rows.append(r)                                             # signed zeros
    big = float(torch.finfo(torch.bfloat16).max)
    rows.append(np.where(np.arange(128) % 2 == 0, big, -big / 3).astype(np.float32))
    r = np.linspace(-1.0, 1.0, 128, dtype=np.float32)
    r[0:32] *= 6.0 * 2.0 ** -3 / np.abs(r[0:32]).max()        # amax exactly 6 * 2^e
    r[32:64] *= (6.0 * 2.0 ** 5) * (1 + 2 ** -7) / np.abs(r[32:64]).max()  # just above
    rows.append(r)
    sub = np.array([2.0 ** -133, -2.0 ** -130, 2.0 ** -127, 3 * 2.0 ** -128], np.float32)
    rows.append(np.tile(sub, 32))                              # all-subnormal row
    x = torch.tensor(np.stack(rows)).to(torch.bfloat16)
    return x


@pytest.mark.parametrize("fmt", [MX, E4])
def test_key_codes_bit_exact(fmt):
    case = synth.index_case(2, 1, 1, 333, seed=41)
    keys = torch.cat([case.keys.reshape(-1, 128), edge_keys(),
                      synth.normal_bf16((64, 128), synth.gen(5), std=300.0)])
    log(f"index keys fmt={fmt}: {keys.shape[0]} keys")
    codes, scales = encode(keys.to(DEV), fmt)
    rc, rs = oracle_keys(keys, fmt)
    assert np.array_equal(codes.cpu().numpy(), rc)
    if fmt == MX:
        assert np.array_equal(scales.cpu().numpy(), rs)
    else:
        assert np.array_equal(scales.cpu().numpy().view(np.uint32),
                              np.asarray(rs, np.float32).view(np.uint32))


def test_mxfp4_codes_every_bf16_value_at_unit_exponent():
    """Every finite bf16 value in [-6, 6], both zeros and the subnormals
    included, encoded with its group's exponent at 0 (each group of 32
    opens with 6) and compared with the oracle: the E2M1 rounding
    (midpoints to the even code, sign kept) checked exhaustively."""
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).float()
    vals = vals[torch.isfinite(vals) & (vals.abs() <= 6.0)]
    per_group = 31
    n_groups = -(-vals.numel() // per_group)
    n_groups += (-n_groups) % 4                      # whole keys of 4 groups
    body = torch.zeros(n_groups * per_group)
    body[:vals.numel()] = vals
    groups = torch.cat([torch.full((n_groups, 1), 6.0), body.view(n_groups, per_group)], 1)
    keys = groups.reshape(-1, 128).to(torch.bfloat16)
    log(f"mxfp4 exhaustive: {vals.numel()} values in {keys.shape[0]} keys")
    codes, scales = encode(keys.to(DEV), MX)
    rc, rs = oracle_keys(keys, MX)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.all(rs == 127)
    bad = np.flatnonzero(codes.cpu().numpy() != rc)
    assert bad.size == 0, f"{bad.size} code bytes differ, e.g. at {bad[:4]}"


@pytest.mark.parametrize("fmt", [MX, E4])
def test_key_codes_strided_rows(fmt):
    """Keys read from every other row of a wider tensor; codes written into
    padded rows (the padding must stay untouched)."""
    base = synth.normal_bf16((50, 256), synth.gen(8)).to(DEV)
    keys = base[:, 64:192]
    nbytes = 64 if fmt == MX else 128
    codes_buf = torch.full((50, nbytes + 32), 0x5A, dtype=torch.uint8, device=DEV)
    codes = codes_buf[:, :nbytes]
    if fmt == MX:
        sbuf = torch.full((50, 8), 0x5A, dtype=torch.uint8, device=DEV)
        scales = sbuf[:, 2:6]
    else:
        sbuf = torch.full((50, 2), -3.0, device=DEV)
        scales = sbuf[:, 1]
    lib = fk.lib()
    fk._check(lib.fp8kv_index_keys_quantize(
        keys.data_ptr(), keys.stride(0), 50, 128, fmt, codes.data_ptr(),
        codes.stride(0), scales.data_ptr(), scales.stride(0),
        torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    rc, rs = oracle_keys(keys.cpu(), fmt)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert torch.all(codes_buf[:, nbytes:] == 0x5A)
    if fmt == MX:
        assert np.array_equal(scales.cpu().numpy(), rs)
        assert torch.all(sbuf[:, :2] == 0x5A) and torch.all(sbuf[:, 6:] == 0x5A)
    else:
        assert np.array_equal(scales.cpu().numpy(), np.asarray(rs, np.float32))
        assert torch.all(sbuf[:, 0] == -3.0)


def widen_case(exps):
    """Keys n with exponent code exps[n] in all 4 groups and nibbles cycling
    through all 16 codes at every position; 256 one-hot query rows (head 0,
    dim d, sign +-), so row (d, sign) reads back max(0, +-k^[n, d])."""
    N = exps.size
    j = np.arange(64)
    n = np.arange(N)[:, None]
    lo = (j[None, :] + n) % 16
    hi = (j[None, :] * 3 + n + 7) % 16
    packed = (lo | (hi << 4)).astype(np.uint8)[None]           # [1, N, 64]
    ex = np.repeat(exps[:, None], 4, axis=1)[None]            # [1, N, 4]
    q = torch.zeros((1, 256, 1, 128), dtype=torch.float32)
    for d in range(128):
        q[0, 2 * d, 0, d] = 1.0
        q[0, 2 * d + 1, 0, d] = -1.0
    q = q.to(torch.bfloat16).to(DEV)
    w = torch.ones((1, 256, 1), device=DEV)
    out = fk.index_score_mxfp4(q, w, MX, torch.tensor(packed).to(DEV),
                               torch.tensor(ex).to(DEV))
    torch.cuda.synchronize()
    kh = dequant_keys(MX, packed, ex)[0]                      # [N, 128]
    want = np.empty((256, N))
    want[0::2] = np.maximum(kh.T, 0.0)
    want[1::2] = np.maximum(-kh.T, 0.0)
    return out[0].cpu().numpy().astype(np.float64), want


def test_mxfp4_widening_exact_for_every_code_and_exponent():
    """Exponent codes 2..252: every E2M1 * 2^e is a finite normal bf16."""
    got, want = widen_case(np.arange(2, 253, dtype=np.uint8))
    assert np.array_equal(got, want)


def test_mxfp4_widening_subnormal_exponents():
    """Exponent codes 0 and 1, where E2M1 * 2^e falls to bf16 subnormals."""
    got, want = widen_case(np.array([0, 1, 0, 1], dtype=np.uint8))
    bad = got != want
    if bad.any():
        log(f"  subnormal widening: {int(bad.sum())} mismatches, e.g. "
            f"got {got[bad][:4]} want {want[bad][:4]}")
    assert not bad.any()


@pytest.mark.parametrize("fmt", [MX, E4])
@pytest.mark.parametrize("B,R,H,N,chunk", [
    (2, 37, 16, 333, 0),        # ragged rows and keys, library chunking
    (3, 5, 16, 200, 48),        # several chunks with a tail
    (1, 1, 4, 17, 16),          # one row, 4 heads, a 1-key tail tile
    (2, 70, 1, 64, 32),         # one head: 16 rows per MFMA tile
    (1, 300, 1, 100, 0),        # one head, rows across 3 workgroups of 128
    (1, 256, 16, 1000, 0),      # the verify-sized row count
    (2, 37, 8, 333, 0),         # 2 rows x 8 heads per MFMA tile, ragged rows
    (1, 70, 8, 96, 32),         # 8 heads: rows across 2 workgroups of 64
    (2, 4, 4, 500, 0),          # 4 verify rows x 4 heads: one MFMA tile
    (1, 130, 4, 333, 0),        # 4 heads: rows across 2 workgroups of 128
    (2, 45, 2, 200, 48),        # 8 rows x 2 heads per tile
    (1, 33, 3, 77, 16),         # 3 heads padded to 4
    (1, 19, 5, 64, 0),          # 5 heads padded to 8
    (1, 11, 12, 64, 0),         # 12 heads padded to 16
])
def test_scores_match_oracle(fmt, B, R, H, N, chunk):
    case = synth.index_case(B, R, H, N, seed=B * 1000 + R + N)
    log(f"index score fmt={fmt} B={B} R={R} H={H} N={N} chunk={chunk}")
    codes, scales = encode(case.keys.to(DEV), fmt)
    q, w = case.q.to(DEV), case.w.to(DEV)
    out = fk.index_score_mxfp4(q, w, fmt, codes, scales, key_chunk=chunk)
    torch.cuda.synchronize()
    check_scores(out, q, w, fmt, codes, scales, f"B{B} R{R} H{H} N{N}")


@pytest.mark.parametrize("H", [16, 4, 1])
@pytest.mark.parametrize("fmt", [MX, E4])
def test_scores_strided_views_and_signed_weights(fmt, H):
    """q and w as non-contiguous views, negative weights, keys with padded
    rows, out with a padded row stride: only the addressed bytes matter."""
    B, R, N = 2, 9, 130
    case = synth.index_case(B, R, H, N, seed=77)
    qbig = torch.zeros((B, R, H + 3, 136), dtype=torch.bfloat16)
    qbig[:, :, 1:H + 1, :128] = case.q
    q = qbig.to(DEV)[:, :, 1:H + 1, :128]
    wbig = torch.zeros((B, R, 2 * H))
    wbig[:, :, ::2] = case.w - 0.5
    w = wbig.to(DEV)[:, :, ::2]
    codes, scales = encode(case.keys.to(DEV), fmt)
    cpad = torch.zeros((B, N, codes.shape[2] + 16), dtype=torch.uint8, device=DEV)
    cpad[:, :, :codes.shape[2]] = codes
    cview = cpad[:, :, :codes.shape[2]]
    obuf = torch.full((B, R, N + 20), 7.0, device=DEV)
    out = obuf[:, :, :N]
    fk.index_score_mxfp4(q, w, fmt, cview, scales, out=out)
    torch.cuda.synchronize()
    assert torch.all(obuf[:, :, N:] == 7.0)
    check_scores(out, q.contiguous(), w.contiguous(), fmt, codes, scales, "strided")


@pytest.mark.parametrize("H,N,chunk", [
    (4, 333, 0),      # library chunking, ragged last chunk
    (4, 1000, 512),   # waves start 0, 128, 256, 384 keys in; a 488-key last chunk
    (4, 200, 48),     # chunks of 48 keys: a 32-key pair and a lone 16-key tile
    (2, 1000, 160),   # starts 0, 128, 96, 64 (wrapped); a 40-key last chunk
    (2, 700, 320),    # starts 0, 128, 256, 64
    (1, 77, 16),      # one head, 16-key chunks (a single tile per chunk)
    (3, 130, 64),     # 3 heads padded to 4
])
@pytest.mark.parametrize("fmt", [MX, E4])
def test_scores_rotated_chunks_on_a_64k_row_pitch(fmt, H, N, chunk):
    """A row pitch of 16,384 floats (64 KiB) at 4 heads or fewer makes wave
    w of a workgroup start 128 w keys into its key chunk and wrap around:
    every score is still written once, within the bound, and nothing past
    N in a row is touched."""
    B, R = 2, 37
    case = synth.index_case(B, R, H, N, seed=500 + N + H)
    log(f"index score rotated fmt={fmt} H={H} N={N} chunk={chunk}")
    codes, scales = encode(case.keys.to(DEV), fmt)
    q, w = case.q.to(DEV), case.w.to(DEV)
    obuf = torch.full((B, R, 16384), 7.0, device=DEV)
    out = obuf[:, :, :N]
    fk.index_score_mxfp4(q, w, fmt, codes, scales, out=out, key_chunk=chunk)
    torch.cuda.synchronize()
    assert torch.all(obuf[:, :, N:] == 7.0)
    check_scores(out, q, w, fmt, codes, scales, f"rotated H{H} N{N} chunk{chunk}")


def test_negative_dots_contribute_nothing():
    """Keys = -q direction for every head: every dot is negative and every
    score is exactly 0 (ReLU per head before the head sum)."""
    B, R, H, N = 1, 8, 16, 48
    g = synth.gen(3)
    q = torch.rand((B, R, H, 128), generator=g).to(torch.bfloat16)
    keys = -torch.rand((B, N, 128), generator=g).to(torch.bfloat16)
    w = torch.rand((B, R, H), generator=g)
    for fmt in (MX, E4):
        codes, scales = encode(keys.to(DEV), fmt)
        out = fk.index_score_mxfp4(q.to(DEV), w.to(DEV), fmt, codes, scales)
        torch.cuda.synchronize()
        assert torch.all(out == 0)


@pytest.mark.parametrize("fmt,H", [(MX, 16), (E4, 16), (MX, 4), (E4, 4)])
def test_index_workload_full_size_sampled(fmt, H):
    """8 requests x 256 rows x 16 (or 4) heads x 65,536 keys, the
    benchmark's launches (library-chosen chunks); key codes of two requests
    are checked bit for bit, and the oracle rescores 10 rows (every lane
    group and store slot of the stacking) x 2048 keys of two requests."""
    case = synth.index_workload(seed=4, device=DEV, heads=H)
    codes, scales = encode(case.keys, fmt)
    out = fk.index_score_mxfp4(case.q, case.w, fmt, codes, scales)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    for b in (0, 7):
        rc, rs = oracle_keys(case.keys[b].cpu(), fmt)
        assert np.array_equal(codes[b].cpu().numpy(), rc)
    rows = torch.tensor([0, 1, 2, 3, 64, 100, 127, 128, 200, 255])
    keys = torch.arange(0, 65536, 32)
    for b in (1, 6):
        sub_q = case.q[b:b + 1, rows]
        sub_w = case.w[b:b + 1, rows]
        sub_c = codes[b:b + 1, keys.to(DEV)]
        sub_s = scales[b:b + 1, keys.to(DEV)]
        got = out[b:b + 1][:, rows.to(DEV)][:, :, keys.to(DEV)]
        check_scores(got, sub_q, sub_w, fmt, sub_c, sub_s, f"full-size request {b}")


# ---------------------------------------------------------------- key builder
def build_keys(raw, g0, g1, fmt, N=None):
    B = raw.shape[0]
    N = g1 if N is None else N
    nbytes = {MX: 64, E4: 128, fk.KEYS_BF16: 256}[fmt]
    codes = torch.full((B, N, nbytes), 0x5A, dtype=torch.uint8, device=DEV)
    scales = (torch.full((B, N, 4), 0x5A, dtype=torch.uint8, device=DEV) if fmt == MX
              else torch.full((B, N), -3.0, device=DEV) if fmt == E4 else None)
    fk.index_keys_build(raw, g0, g1, fmt, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def bf16_keys_of(codes):
    """BF16-format builder output [B, N, 256 bytes] -> bf16 bits [B, N, 128]."""
    return codes.cpu().numpy().view(np.uint16)


def check_pooled(bits, raw, g0, g1, what):
    """Every pooled key is the correctly rounded bf16 of the exact normalized
    mean, or its neighbour when the exact value lies within 2^-16 (relative)
    of a rounding midpoint (the fp32 mean and norm are accurate to a few
    ulps)."""
    got = oracle.bf16_to_f32(bits).astype(np.float64)
    want = oracle.index_keys_pool(bf16_bits(raw), g0, g1)
    mag = np.abs(want)
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0)
    err = np.abs(got - want)
    assert np.all(err <= 0.5 * ulp + 2.0 ** -16 * mag), what
    rne = oracle.bf16_to_f32(bf16_bits(torch.from_numpy(want).to(torch.bfloat16)))
    off = int((got != rne).sum())
    log(f"  {what}: {off} of {got.size} values off the correctly rounded bf16")
    assert off <= max(4, got.size // 10000)


def test_builder_pools_and_normalizes():
    g = synth.gen(60)
    raw = synth.normal_bf16((2, 4 * 300 + 3, 128), g)
    raw[0, 40:44] = 0                                        # an all-zero group
    raw[1, 8:12] = synth.normal_bf16((4, 128), g, std=1e-30)  # tiny magnitudes
    raw = raw.to(DEV)
    codes, _ = build_keys(raw, 0, 300, fk.KEYS_BF16)
    bits = bf16_keys_of(codes)
    for b in range(2):
        check_pooled(bits[b], raw[b].cpu(), 0, 300, f"request {b}")
    assert np.all(bits[0, 10] == 0)


@pytest.mark.parametrize("fmt", [MX, E4])
def test_builder_codes_equal_the_encoding_of_its_bf16_keys(fmt):
    raw = synth.normal_bf16((3, 4 * 257, 128), synth.gen(61)).to(DEV)
    kb, _ = build_keys(raw, 0, 257, fk.KEYS_BF16)
    codes, scales = build_keys(raw, 0, 257, fmt)
    for b in range(3):
        rc, rs = oracle_keys(torch.from_numpy(bf16_keys_of(kb)[b].view(np.int16)).view(torch.bfloat16), fmt)
        assert np.array_equal(codes[b].cpu().numpy(), rc)
        if fmt == MX:
            assert np.array_equal(scales[b].cpu().numpy(), rs)
        else:
            assert np.array_equal(scales[b].cpu().numpy().view(np.uint32),
                                  np.asarray(rs, np.float32).view(np.uint32))


@pytest.mark.parametrize("fmt", [MX, E4, fk.KEYS_BF16])
def test_builder_chunked_equals_whole(fmt):
    """Two calls [0, 77) and [77, 200) -- a raw chunk boundary inside group
    77 -- write exactly what one call [0, 200) writes, and nothing else."""
    raw = synth.normal_bf16((2, 4 * 200 + 1, 128), synth.gen(62)).to(DEV)
    whole = build_keys(raw, 0, 200, fmt, N=210)
    B = 2
    nbytes = whole[0].shape[2]
    codes = torch.full((B, 210, nbytes), 0x5A, dtype=torch.uint8, device=DEV)
    scales = (torch.full((B, 210, 4), 0x5A, dtype=torch.uint8, device=DEV) if fmt == MX
              else torch.full((B, 210), -3.0, device=DEV) if fmt == E4 else None)
    fk.index_keys_build(raw, 0, 77, fmt, codes, scales)
    fk.index_keys_build(raw, 77, 200, fmt, codes, scales)
    torch.cuda.synchronize()
    assert torch.equal(codes, whole[0])
    assert torch.all(codes[:, 200:] == 0x5A)
    if scales is not None:
        assert torch.equal(scales, whole[1])


def test_builder_index_workload_full_size_sampled():
    """8 requests x 262,144 raw keys -> 65,536 compressed keys each (the
    index workload's key recipe), MXFP4; sampled keys checked."""
    raw = synth.normal_bf16((8, 4 * 65536, 128), synth.gen(63, DEV), device=DEV)
    kb, _ = build_keys(raw, 0, 65536, fk.KEYS_BF16)
    codes, scales = build_keys(raw, 0, 65536, MX)
    pick = torch.arange(0, 65536, 97)
    for b in (0, 5):
        sub = raw[b].view(65536, 4, 128)[pick.to(DEV)].reshape(-1, 128).cpu()
        check_pooled(bf16_keys_of(kb)[b][pick.numpy()], sub, 0, pick.numel(), f"request {b}")
        rc, rs = oracle_keys(torch.from_numpy(bf16_keys_of(kb)[b][pick.numpy()].view(np.int16)).view(torch.bfloat16), MX)
        assert np.array_equal(codes[b][pick.to(DEV)].cpu().numpy(), rc)
        assert np.array_equal(scales[b][pick.to(DEV)].cpu().numpy(), rs)


@pytest.mark.parametrize("fmt", [MX, E4])
def test_builder_end_to_end_full_size(fmt):
    """The index workload's keys (8 requests x 262,144 raw keys -> 65,536
    compressed keys each) against the oracle end to end: pool and normalize
    in double, one rounding to bf16, encode. Every key whose bf16 values the
    kernel rounds like the oracle has bit-identical codes and scales; the
    keys that differ are counted and logged, and every value that differs
    is one bf16 step away with the exact pooled value within 2^-16
    (relative) of the midpoint between the two (the fp32 mean and norm are
    accurate to a few fp32 ulps)."""
    from concurrent.futures import ThreadPoolExecutor
    B, N = 8, 65536
    raw = synth.normal_bf16((B, 4 * N, 128), synth.gen(63, DEV), device=DEV)
    kb, _ = build_keys(raw, 0, N, fk.KEYS_BF16)
    codes, scales = build_keys(raw, 0, N, fmt)
    raw_h = bf16_bits(raw)
    del raw
    kb_h = bf16_keys_of(kb)
    codes_h = codes.cpu().numpy()
    scales_h = scales.cpu().numpy()

    def one(b):
        okb, (oc, osc) = oracle.index_keys_build(raw_h[b], 0, N, fmt)
        pooled = oracle.index_keys_pool(raw_h[b], 0, N)
        diff = kb_h[b] != okb
        dk = diff.any(axis=1)
        same = ~dk
        ok_codes = np.array_equal(codes_h[b][same], oc[same])
        if fmt == MX:
            ok_scales = np.array_equal(scales_h[b][same], osc[same])
        else:
            ok_scales = np.array_equal(scales_h[b][same].view(np.uint32),
                                       np.asarray(osc, np.float32)[same].view(np.uint32))
        gv = oracle.bf16_to_f32(kb_h[b][diff]).astype(np.float64)
        ov = oracle.bf16_to_f32(okb[diff]).astype(np.float64)
        steps = np.abs(kb_h[b][diff].astype(np.int32) - okb[diff].astype(np.int32))
        x = pooled[diff]
        in_band = np.abs(x - 0.5 * (gv + ov)) <= TOL * np.abs(x)
        return (int(dk.sum()), int(diff.sum()), ok_codes, ok_scales,
                bool(np.all(steps == 1)), bool(np.all(in_band)))

    with ThreadPoolExecutor(max_workers=8) as ex:
        res = list(ex.map(one, range(B)))
    keys_off = sum(r[0] for r in res)
    vals_off = sum(r[1] for r in res)
    log(f"  builder end to end, format {fmt}: {keys_off} of {B * N} keys "
        f"({vals_off} of {B * N * 128} bf16 values) differ from the oracle's "
        f"one-rounding result; all others bit-exact")
    for b, r in enumerate(res):
        assert r[2] and r[3], f"request {b}: codes or scales differ on an equal key"
        assert r[4] and r[5], f"request {b}: a differing value is outside the midpoint band"
    assert vals_off <= B * N * 128 // 10000
