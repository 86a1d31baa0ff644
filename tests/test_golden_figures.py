"""The numbers the pages print (tests/golden/page_figures.json, each with its
citation) against the oracle's codec and the closed forms of the format:
a wrong bias, mantissa width or byte accounting moves one of them."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "page_figures.json")))


def finite_values(fmt):
    v = oracle.decode(np.arange(256, dtype=np.uint8), fmt)
    return v[np.isfinite(v)]


def test_e4m3_range_and_floor():
    assert oracle.fmt_max(oracle.E4M3) == GOLDEN["e4m3_max"]["value"]
    v = finite_values(oracle.E4M3)
    min_normal = 2.0 ** -6
    assert min_normal in v and min_normal - min_normal / 8 in v   # largest subnormal below it
    assert round(min_normal, 4) == GOLDEN["e4m3_floor"]["value"]


@pytest.mark.parametrize("fmt,key,mbits", [(oracle.E4M3, "worst_rel_error_e4m3", 3),
                                           (oracle.E5M2, "worst_rel_error_e5m2", 2)])
def test_worst_relative_error_is_the_printed_bound(fmt, key, mbits):
    # half a spacing over the rounded value peaks at the bottom of a binade:
    # exactly 2^-(m+1) (0.0625 for e4m3, 0.125 for e5m2); over the input
    # value it is 1/(2^(m+1)+1) (1/17, 1/9)
    printed = GOLDEN[key]["value"]
    v = np.unique(np.abs(finite_values(fmt)))
    normal = v[v >= 2.0 ** (-6 if fmt == oracle.E4M3 else -14)]
    mids = (normal[:-1] + normal[1:]) / 2
    over_code = np.max((mids - normal[:-1]) / normal[:-1])
    over_input = np.max((mids - normal[:-1]) / mids)
    assert over_code == 2.0 ** -(mbits + 1)
    assert abs(over_input - 1 / (2 ** (mbits + 1) + 1)) < 1e-12
    assert round(over_code, 2 if mbits == 3 else 3) == printed


def test_scale_sidecar_fraction():
    D = 128
    codes, scale = D, 4                      # bytes per (token, KV head) row
    frac = scale / codes
    assert frac == 0.03125 and round(frac, 2) == GOLDEN["scale_sidecar_fraction_d128"]["value"]
    assert (codes + scale) / (2 * D) < 0.52  # halves the 16-bit row, sidecar included


def test_measured_error_ratio_is_the_mantissa_bit():
    m = GOLDEN["measured_rel_l2_tpu"]
    for phase in ("prefill", "decode"):
        ratio = m[f"e5m2_{phase}"] / m[f"e4m3_{phase}"]
        assert 1.8 < ratio < 2.2              # one mantissa bit: ~2x


def test_capacity_with_a_bf16_indexer():
    g = GOLDEN["indexer_fraction_and_capacity"]
    f = g["indexer_fraction"]                # share of the bf16 cache bytes
    capacity = 1.0 / ((1 - f) / 2 + f)       # fp8 body, bf16 indexer
    assert round(capacity, 2) == g["capacity"]
    assert 1.0 / 0.5 == g["capacity_without_indexer"]


def test_page_buffer_halves():
    g = GOLDEN["page_buffer_mib"]
    assert g["bf16"] / g["e4m3"] == 2.0
