"""Property-based pins of the CPU oracle (hypothesis): on random tiny inputs
the oracle must agree with the exact pure-Python brute force of
tests/_brute.py, which uses different algorithms (bucket enumeration, exact
rational nearest search, per-operation rational rounding).  CPU only.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from tests import _brute as brute

SETTINGS = settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
FINITE_BF16 = st.integers(0, 0xFFFF).filter(lambda b: (b >> 7) & 0xFF != 0xFF)


@st.composite
def routing(draw, max_rows=12, max_k=4, max_e=8):
    e = draw(st.integers(1, max_e))
    k = draw(st.integers(1, max_k))
    n = draw(st.integers(0, max_rows))
    ids = draw(st.lists(st.integers(-3, e + 2), min_size=n * k, max_size=n * k))
    return np.array(ids, dtype=np.int32).reshape(n, k), e


@SETTINGS
@given(routing(), st.integers(-20, 40), st.integers(0, 3))
def test_mask_matches_brute(case, count, tp_rank):
    ids, _ = case
    got = oracle.mask_routing_padding(ids, count, tp_rank)
    want = np.array(brute.mask(ids.tolist(), count, tp_rank), dtype=np.int32).reshape(ids.shape)
    np.testing.assert_array_equal(got, want)


@SETTINGS
@given(routing())
def test_indices_match_brute(case):
    ids, e = case
    got = oracle.create_indices(ids, e)
    want = brute.indices(ids.reshape(-1).tolist(), e)
    for key in ("token_expert_order", "restore_token_order", "expert_start_indices", "expert_ids",
                "expert_usage_stats"):
        np.testing.assert_array_equal(got[key].astype(np.int64), np.array(want[key], dtype=np.int64), err_msg=key)
    assert got["n_routed"] == want["n_routed"]


@SETTINGS
@given(routing(), st.integers(1, 9))
def test_scales_offset_matches_brute(case, align):
    ids, e = case
    got = oracle.create_indices(ids, e, scales_align=align)["scales_offset"]
    np.testing.assert_array_equal(got.astype(np.int64), np.array(brute.scales_offset(ids.reshape(-1).tolist(), e, align)))


@st.composite
def bf16_block(draw):
    """32 finite bf16 patterns, often sharing a narrow exponent range so that
    ties and saturation against the block scale are common."""
    if draw(st.booleans()):
        return draw(st.lists(FINITE_BF16, min_size=32, max_size=32))
    exp = draw(st.integers(0, 254))
    lo = max(0, exp - 4)
    elems = st.tuples(st.integers(0, 1), st.integers(lo, exp), st.integers(0, 127)).map(
        lambda t: (t[0] << 15) | (t[1] << 7) | t[2])
    return draw(st.lists(elems, min_size=32, max_size=32))


@SETTINGS
@given(bf16_block())
def test_mxfp4_block_matches_brute(block):
    q, s = oracle.mxfp4_quantize(np.array([block], dtype=np.uint16))
    scale, nibs = brute.mxfp4_block(block)
    assert int(s[0, 0]) == scale
    assert [int(b) for b in q[0]] == [nibs[2 * m] | (nibs[2 * m + 1] << 4) for m in range(16)]


@SETTINGS
@given(bf16_block())
def test_mxfp4_even_scale_matches_brute(block):
    _, s = oracle.mxfp4_quantize(np.array([block], dtype=np.uint16), even=True)
    assert int(s[0, 0]) == brute.even_scale_byte(block)


@st.composite
def combine_case(draw):
    n = draw(st.integers(1, 4))
    k = draw(st.integers(1, 4))
    e = draw(st.integers(1, 4))
    h = 8
    ids = np.array(draw(st.lists(st.integers(-1, e), min_size=n * k, max_size=n * k)), dtype=np.int32).reshape(n, k)
    w = np.array(draw(st.lists(st.floats(-4.0, 4.0, width=32, allow_subnormal=False), min_size=n * k,
                               max_size=n * k)), dtype=np.float32).reshape(n, k)
    rows = max(int(((ids >= 0) & (ids < e)).sum()), 1)
    ybits = np.array(draw(st.lists(FINITE_BF16.filter(lambda b: ((b >> 7) & 0xFF) < 0xF0), min_size=rows * h,
                                   max_size=rows * h)), dtype=np.uint16).reshape(rows, h)
    return ids, e, w, ybits


@SETTINGS
@given(combine_case())
def test_combine_matches_brute(case):
    ids, e, w, ybits = case
    k = ids.shape[1]
    r = oracle.create_indices(ids, e)
    out = oracle.combine(ybits, w, r["restore_token_order"], k)
    ylist = ybits.tolist()
    for t in range(ids.shape[0]):
        want = brute.combine_row(w[t].tolist(), ylist, r["restore_token_order"][t * k:(t + 1) * k].tolist())
        for c, wv in enumerate(want):
            assert brute.bf16_value(int(out[t, c]))[0] == wv
