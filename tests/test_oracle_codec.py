"""Pins of the oracle's FP8 codec against facts fixed outside it.

* torch's float8_e4m3fn / float8_e5m2 dtypes (an independent library
  implementation of the OCP formats) for every code's value and for RNE
  casts inside the finite range;
* closed forms the pages state: e4m3 max 448 and its 0.0156 (2^-6) normal
  floor (sglang-jax #1776, "Three design points"), and the worst-case
  relative errors "~6% vs ~12.5%" (same section), whose exact suprema on the
  normal range are 1/17 and 1/9.
"""
import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(256, dtype=np.uint8)


def torch_decode(codes, fmt):
    dt = torch.float8_e4m3fn if fmt == oracle.E4M3 else torch.float8_e5m2
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(dt).double().numpy()


def torch_encode(values, fmt):
    dt = torch.float8_e4m3fn if fmt == oracle.E4M3 else torch.float8_e5m2
    t = torch.from_numpy(np.asarray(values, np.float32))
    return t.to(dt).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_table_matches_torch(fmt):
    ours = oracle.decode(ALL, fmt)
    ref = torch_decode(ALL, fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # signed zeros too
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_closed_forms():
    v = oracle.decode(ALL)
    assert oracle.fmt_max(oracle.E4M3) == 448.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    # the smallest normal, the pages' "0.0156" floor
    assert v[0x08] == 2.0 ** -6 == 0.015625
    assert v[0x01] == 2.0 ** -9          # smallest subnormal
    nan_codes = set(np.flatnonzero(np.isnan(v)).tolist())
    assert nan_codes == {0x7F, 0xFF}      # no infinities in e4m3
    finite = v[~np.isnan(v)]
    assert len(np.unique(finite)) == 253  # +-0 coincide
    assert oracle.fmt_max(oracle.E5M2) == 57344.0


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_decode_roundtrip(fmt):
    v = oracle.decode(ALL, fmt)
    ok = np.isfinite(v)
    back = oracle.encode(v[ok].astype(np.float32), fmt)
    assert np.array_equal(back, ALL[ok])


def _sweep_values(fmt, n_random=200_000, seed=0):
    """Every code value, every midpoint between neighbours, the fp32
    neighbours of each midpoint, and log-uniform random values."""
    v = oracle.decode(ALL, fmt)
    mx = oracle.fmt_max(fmt)
    pos = np.unique(v[(v >= 0) & np.isfinite(v)])
    mids = (pos[:-1] + pos[1:]) / 2.0
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)  # exact in fp32
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    rng = np.random.default_rng(seed)
    rnd = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(mx),
                             n_random)).astype(np.float32)
    vals = np.concatenate([pos.astype(np.float32), mids32, up, dn, rnd,
                           np.array([0.0, 2.0 ** -12, 2.0 ** -11], np.float32)])
    vals = vals[vals <= mx]
    return np.concatenate([vals, -vals])


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_matches_torch_rne(fmt):
    vals = _sweep_values(fmt)
    ours = oracle.encode(vals, fmt)
    ref = torch_encode(vals, fmt)
    bad = np.flatnonzero(ours != ref)
    assert bad.size == 0, (vals[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_ties_go_to_even_code():
    # midpoint of 1.0 (0x38) and 1.125 (0x39) -> even 0x38
    assert oracle.encode([1.0625])[0] == 0x38
    # midpoint of 1.125 (0x39) and 1.25 (0x3A) -> even 0x3A
    assert oracle.encode([1.1875])[0] == 0x3A
    # subnormal boundaries: 2^-10 -> 0, (7*2^-9 + 2^-6)/2 -> 2^-6 (0x08)
    assert oracle.encode([2.0 ** -10])[0] == 0x00
    assert oracle.encode([7.5 * 2.0 ** -9])[0] == 0x08
    assert oracle.encode([-0.0])[0] == 0x80


@pytest.mark.parametrize("fmt,code", [(oracle.E4M3, 0x7E), (oracle.E5M2, 0x7B)])
def test_saturation(fmt, code):
    big = np.array([oracle.fmt_max(fmt) * 1.01, 1e30, np.float32(3e38)],
                   np.float32)
    assert np.all(oracle.encode(big, fmt) == code)
    assert np.all(oracle.encode(-big, fmt) == (code | 0x80))


@pytest.mark.parametrize("fmt,sup,bound", [(oracle.E4M3, 1.0 / 17.0, 2 ** -4),
                                           (oracle.E5M2, 1.0 / 9.0, 2 ** -3)])
def test_worst_relative_error(fmt, sup, bound):
    """On the normal range the largest relative error of encode/decode is
    attained at the first midpoint above a power of two: exactly 1/17 for
    e4m3 ("~6%") and 1/9 for e5m2 ("~12.5%" is the 2^-3 bound)."""
    v = oracle.decode(ALL, fmt)
    pos = np.unique(v[(v > 0) & np.isfinite(v)])
    min_normal = 2.0 ** -6 if fmt == oracle.E4M3 else 2.0 ** -14
    vals = _sweep_values(fmt)
    vals = vals[(vals >= min_normal) & (vals <= pos.max())]
    rec = oracle.decode(oracle.encode(vals, fmt), fmt)
    rel = np.abs(rec - vals.astype(np.float64)) / np.abs(vals)
    assert rel.max() <= bound
    assert rel.max() == pytest.approx(sup, rel=1e-12)


def test_encode_is_monotone():
    x = np.sort(_sweep_values(oracle.E4M3))
    dec = oracle.decode(oracle.encode(x))
    assert np.all(np.diff(dec) >= 0)
