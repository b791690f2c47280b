"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a hand-worked example (tests/golden/),
a closed form, an invariant, or the exact pure-Python brute force in
tests/_brute.py.  CPU only.
"""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _brute as brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SENT = 0xFFFFFFFF


def to_bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ mask
@pytest.mark.parametrize("count_case", ["zero", "one", "n_minus_1", "n", "n_plus_5", "neg3"])
@pytest.mark.parametrize("tp_rank", [0, 1, 2])
def test_mask_against_brute(count_case, tp_rank):
    g = np.random.default_rng(11)
    n, k = 13, 3
    ids = g.integers(-2, 9, size=(n, k)).astype(np.int32)
    c = {"zero": 0, "one": 1, "n_minus_1": n - 1, "n": n, "n_plus_5": n + 5, "neg3": -3}[count_case]
    c += tp_rank * n  # count is in the global frame
    got = oracle.mask_routing_padding(ids, c, tp_rank)
    want = np.array(brute.mask(ids.tolist(), c, tp_rank), dtype=np.int32)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(ids, ids.copy())  # input untouched


def test_mask_tp_offset_frame():
    # global count 20 with N = 8: rank 0 keeps all 8 rows, rank 1 keeps 8, rank 2 keeps 4, rank 3 none.
    ids = np.arange(16, dtype=np.int32).reshape(8, 2)
    kept = [int((oracle.mask_routing_padding(ids, 20, r) >= 0).all(axis=1).sum()) for r in range(4)]
    assert kept == [8, 8, 4, 0]


# ------------------------------------------------------------------ worked example
def test_worked_example_whole_path():
    d = json.load(open(os.path.join(GOLDEN, "worked_example_path.json")))
    ids = np.array(d["routing_map"], dtype=np.int32)
    m = oracle.mask_routing_padding(ids, d["real_token_count"], d["tp_rank"])
    np.testing.assert_array_equal(m, np.array(d["masked"]))
    r = oracle.create_indices(m, d["n_experts"])
    for key in ("token_expert_order", "restore_token_order", "expert_start_indices", "expert_ids",
                "expert_usage_stats"):
        np.testing.assert_array_equal(r[key].astype(np.int64), np.array(d[key], dtype=np.int64), err_msg=key)
    x = np.arange(3 * 8, dtype=np.uint16).reshape(3, 8)
    out = oracle.dispatch(x, r["token_expert_order"], d["top_k"], r["n_routed"])
    np.testing.assert_array_equal(out, x[d["dispatch_source_rows"]])


# ------------------------------------------------------------------ indices
def _tiny_ids(g, n, k, e, kind):
    if kind == "uniform":
        return g.integers(0, e, size=(n, k))
    if kind == "garbage":
        pool = np.array([-1, -7, e, e + 3, 2 ** 31 - 1, -2 ** 31] + list(range(e)))
        return g.choice(pool, size=(n, k))
    if kind == "one_expert":
        return np.full((n, k), e - 1)
    if kind == "all_unrouted":
        return np.full((n, k), -1)
    raise ValueError(kind)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("kind", ["uniform", "garbage", "one_expert", "all_unrouted"])
def test_indices_against_brute(seed, kind):
    g = np.random.default_rng(100 + seed)
    e = int(g.integers(1, 9))
    k = int(g.choice([1, 2, 3, e]))
    n = int(g.integers(0, 17))
    ids = _tiny_ids(g, n, k, e, kind).astype(np.int32)
    got = oracle.create_indices(ids, e)
    want = brute.indices(ids.reshape(-1).tolist(), e)
    for key in ("token_expert_order", "restore_token_order", "expert_start_indices", "expert_ids",
                "expert_usage_stats"):
        np.testing.assert_array_equal(got[key].astype(np.int64), np.array(want[key], dtype=np.int64),
                                      err_msg=key)
    assert got["n_routed"] == want["n_routed"]


def check_index_invariants(ids_masked, n_experts, r, expect_routed=None):
    f = ids_masked.reshape(-1).astype(np.int64)
    s = f.size
    teo, res = r["token_expert_order"], r["restore_token_order"]
    esi, eids, stats = r["expert_start_indices"], r["expert_ids"], r["expert_usage_stats"]
    v = r["n_routed"]
    routed = (f >= 0) & (f < n_experts)
    assert v == int(routed.sum())
    if expect_routed is not None:
        assert v == expect_routed
    # restore inverts token_expert_order; unrouted slots never appear
    assert np.all(teo[v:] == SENT)
    pos = teo[:v].astype(np.int64)
    assert np.all(routed[pos])
    assert np.array_equal(res[pos], np.arange(v))
    assert np.all(res[~routed] == SENT)
    # CSR over active experts
    a = int(stats[1])
    assert esi[0] == 0 and np.all(np.diff(esi.astype(np.int64)) >= 0) and esi[a] == v
    assert np.all(esi[a:] == v)
    assert np.all(np.diff(eids[:a]) > 0) and np.all(eids[a:] == -1)
    seg_len = np.diff(esi[: a + 1].astype(np.int64))
    assert np.all(seg_len > 0)
    assert stats[0] == (seg_len.max() if a else 0)
    for j in range(a):
        seg = pos[esi[j]:esi[j + 1]]
        assert np.all(f[seg] == eids[j])
        assert np.all(np.diff(seg) > 0)  # stable: ascending slot index


@pytest.mark.parametrize("cfg", range(len(workloads.WORKLOADS)))
def test_indices_invariants_on_workloads(cfg):
    w = workloads.WORKLOADS[cfg]
    ids, _, real = workloads.make_routing(w, cfg)
    m = oracle.mask_routing_padding(ids, real)
    r = oracle.create_indices(m, w.n_experts)
    check_index_invariants(m, w.n_experts, r, expect_routed=real * w.top_k)
    # masked rows never appear in the order
    assert np.all(r["token_expert_order"][: r["n_routed"]] // w.top_k < real)
    if w.routing == "hotcold":
        assert int(r["expert_usage_stats"][1]) == w.n_experts - w.n_cold


# ------------------------------------------------------------------ dispatch
def test_dispatch_token_major_closed_form():
    g = np.random.default_rng(5)
    n, k, e, h = 40, 3, 6, 16
    ids = g.integers(-1, e, size=(n, k)).astype(np.int32)
    r = oracle.create_indices(ids, e)
    x = g.integers(0, 1 << 16, size=(n, h)).astype(np.uint16)
    out = oracle.dispatch(x, r["token_expert_order"], k, r["n_routed"])
    assert out.shape == (r["n_routed"], h)
    res = r["restore_token_order"].reshape(n, k)
    for t in range(n):
        for j in range(k):
            if res[t, j] != SENT:
                np.testing.assert_array_equal(out[res[t, j]], x[t])


# ------------------------------------------------------------------ MXFP4
def test_mxfp4_hand_vectors():
    d = json.load(open(os.path.join(GOLDEN, "mxfp4_vectors.json")))
    for v in d["vectors"]:
        blk = np.zeros(32, np.uint16)
        if "bits" in v:
            for i, b in enumerate(v["bits"]):
                blk[i] = int(b, 16)
        else:
            vals = [1.0] * 32 if v["values"] == "ones32" else v["values"]
            blk[: len(vals)] = to_bf16_bits(vals)
        q, s = oracle.mxfp4_quantize(blk[None])
        head = [int(h, 16) for h in v["payload_head"]]
        assert s[0, 0] == int(v["scale"], 16), v["why"]
        assert list(q[0, : len(head)]) == head, v["why"]


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]


@pytest.mark.parametrize("se", [0, -127, -126, -100, -10, 7, 100, 125])
def test_mxfp4_element_map_exhaustive(se):
    """Every finite bf16 value that keeps the block exponent at ``se`` (anchor
    2**(se+2) in element 0) maps to the nearest E2M1 code, ties to even,
    exactly as an exact rational nearest search says (element 1 = high nibble,
    element 2 = low nibble)."""
    allb = _all_finite_bf16()
    vals = oracle.bf16_bits_to_f32(allb).astype(np.float64)
    lim = 2.0 ** (se + 3)
    sel = allb[np.abs(vals) < lim]
    if se != 0:  # other exponents: a seeded sample keeps the brute force fast
        sel = np.random.default_rng(se + 1000).choice(sel, size=min(sel.size, 3000), replace=False)
    anchor = to_bf16_bits([2.0 ** (se + 2)])[0]
    blocks = np.zeros((sel.size, 32), np.uint16)
    blocks[:, 0] = anchor
    blocks[:, 1] = sel
    blocks[:, 2] = sel
    q, s = oracle.mxfp4_quantize(blocks)
    assert np.all(s[:, 0] == se + 127)
    unit = Fraction(2) ** se
    for i, b in enumerate(sel.tolist()):
        v, sgn = brute.bf16_value(b)
        a = abs(v) / unit
        best, bd = None, None
        for code, gval in enumerate(brute.E2M1):
            dd = abs(a - gval)
            if best is None or dd < bd or (dd == bd and code % 2 == 0):
                best, bd = code, dd
        nib = best | (8 if sgn else 0)
        assert (q[i, 0] >> 4) == nib, (hex(b), se)
        assert (q[i, 1] & 0xF) == nib, (hex(b), se)


@pytest.mark.parametrize("seed", range(4))
def test_mxfp4_rows_against_brute(seed):
    g = np.random.default_rng(200 + seed)
    t, h = 3, 96
    f = g.standard_normal((t, h)).astype(np.float32)
    f[0, 5] *= 1e3
    f[1, 40:64] = 0.0
    f[1, 70] = -0.0
    f[2, :32] *= 1e-39          # subnormal-range block
    f[2, 32:64] = np.float32(2.0 ** -133)
    bits = to_bf16_bits(f.reshape(-1)).reshape(t, h)
    q, s = oracle.mxfp4_quantize(bits)
    for r in range(t):
        pq, ps = brute.mxfp4_row(bits[r].tolist())
        assert list(q[r]) == pq
        assert list(s[r]) == ps


@pytest.mark.parametrize("seed", range(3))
def test_mxfp4_round_trip_on_representable_blocks(seed):
    g = np.random.default_rng(300 + seed)
    nblk = 400
    codes = g.integers(0, 8, size=(nblk, 32))
    signs = np.where(g.random((nblk, 32)) < 0.5, -1.0, 1.0)
    sexp = g.integers(-120, 121, size=(nblk, 1))
    vals = signs * oracle.moe_oracle.E2M1_GRID[codes] * np.ldexp(1.0, sexp)
    vals[codes == 0] = 0.0   # keep zeros positive so the decoded value is bitwise the same
    bits = to_bf16_bits(vals.reshape(-1)).reshape(nblk, 32)
    assert np.array_equal(oracle.bf16_bits_to_f32(bits).astype(np.float64), vals)
    q, s = oracle.mxfp4_quantize(bits)
    back = oracle.mxfp4_dequantize(q, s).reshape(nblk, 32)
    np.testing.assert_array_equal(back, vals)


def test_mxfp4_dispatch_copies_identical():
    g = np.random.default_rng(9)
    n, k, e, h = 20, 4, 5, 64
    ids = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    r = oracle.create_indices(ids, e)
    x = to_bf16_bits(g.standard_normal(n * h)).reshape(n, h)
    q, s = oracle.dispatch_mxfp4(x, r["token_expert_order"], k, r["n_routed"])
    q1, s1 = oracle.mxfp4_quantize(x)
    res = r["restore_token_order"].reshape(n, k)
    for t in range(n):
        for j in range(k):
            np.testing.assert_array_equal(q[res[t, j]], q1[t])
            np.testing.assert_array_equal(s[res[t, j]], s1[t])


# ------------------------------------------------------------------ combine
def _combine_vs_brute(y_bits, w, restore, k):
    out = oracle.combine(y_bits, w, restore, k)
    n = w.shape[0]
    ylist = y_bits.tolist()
    for t in range(n):
        want = brute.combine_row(w[t].tolist(), ylist, restore[t * k:(t + 1) * k].tolist())
        for c, wv in enumerate(want):
            got_v, got_s = brute.bf16_value(int(out[t, c]))
            assert got_v == wv, (t, c)
            if wv == 0:
                assert got_s == 0  # the sum over an empty or cancelling set is +0


@pytest.mark.parametrize("seed", range(5))
def test_combine_against_brute(seed):
    g = np.random.default_rng(400 + seed)
    n, k, h = 5, int(g.integers(1, 5)), 12
    s = n * k
    ids = g.integers(-1, 3, size=(n, k)).astype(np.int32)
    r = oracle.create_indices(ids, 3)
    v = r["n_routed"]
    y = to_bf16_bits(g.standard_normal(max(v, 1) * h) * np.exp(g.normal(0, 4, max(v, 1) * h))).reshape(-1, h)
    w = g.random((n, k)).astype(np.float32)
    w[0, 0] = -w[0, 0]
    _combine_vs_brute(y, w, r["restore_token_order"], k)
    assert s == r["restore_token_order"].size


def test_combine_identity_k1():
    g = np.random.default_rng(7)
    n, h = 9, 40
    y = to_bf16_bits(g.standard_normal(n * h)).reshape(n, h)
    y[y == 0x8000] = 0
    w = np.ones((n, 1), np.float32)
    restore = np.arange(n, dtype=np.uint32)
    np.testing.assert_array_equal(oracle.combine(y, w, restore, 1), y)


def test_combine_one_hot_selects_row():
    g = np.random.default_rng(8)
    n, k, h = 6, 4, 16
    y = to_bf16_bits(g.standard_normal(n * k * h)).reshape(n * k, h)
    y[y == 0x8000] = 0
    restore = g.permutation(n * k).astype(np.uint32)
    w = np.zeros((n, k), np.float32)
    hot = g.integers(0, k, size=n)
    w[np.arange(n), hot] = 1.0
    out = oracle.combine(y, w, restore, k)
    for t in range(n):
        want = y[restore[t * k + hot[t]]]
        # zero-weight terms add +0 or -0 to the sum; +0 + x == x for x != 0
        np.testing.assert_array_equal(out[t][want != 0], want[want != 0])


def test_combine_no_fused_multiply_add():
    """w1*y1 is inexact in fp32; with separate rounding the two terms cancel
    to +0, whereas a fused multiply-add would leave 2**-30 (bf16 0x3080)."""
    w = np.array([[-(1 + 2.0 ** -23), 1 + 2.0 ** -23]], np.float32)
    y = to_bf16_bits([1 + 2.0 ** -7, 1 + 2.0 ** -7]).reshape(2, 1)
    restore = np.array([0, 1], np.uint32)
    out = oracle.combine(y, w, restore, 2)
    assert out[0, 0] == 0x0000
    exact_fused = Fraction(float(np.float32(-(1 + 2.0 ** -23)))) * Fraction(1 + 2.0 ** -7)
    exact_fused = brute.f32(exact_fused) + Fraction(float(np.float32(1 + 2.0 ** -23))) * Fraction(1 + 2.0 ** -7)
    assert exact_fused == Fraction(2) ** -30
    _combine_vs_brute(y, w, restore, 2)


def test_combine_fixed_order():
    """+1, +2**-30, -1 in slot order sums to +0; any other order leaves 2**-30."""
    w = np.ones((1, 3), np.float32)
    y = to_bf16_bits([1.0, 2.0 ** -30, -1.0]).reshape(3, 1)
    out = oracle.combine(y, w, np.array([0, 1, 2], np.uint32), 3)
    assert out[0, 0] == 0
    out2 = oracle.combine(y, w, np.array([0, 2, 1], np.uint32), 3)
    assert out2[0, 0] == to_bf16_bits([2.0 ** -30])[0]


def test_combine_unrouted_rows_are_positive_zero():
    y = to_bf16_bits([3.0, -2.0]).reshape(2, 1)
    w = np.ones((3, 2), np.float32)
    restore = np.array([0, SENT, SENT, SENT, 1, SENT], np.uint32)
    out = oracle.combine(y, w, restore, 2)
    assert out.tolist() == [[to_bf16_bits([3.0])[0]], [0], [to_bf16_bits([-2.0])[0]]]


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(12)
    f = (g.standard_normal(200000) * np.exp(g.normal(0, 20, 200000))).astype(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    ties = (np.arange(1, 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, -ties])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16_rne(f), want)


def test_brute_rounding_sanity():
    # the exact fp32 rounding of the brute force agrees with IEEE hardware on products and sums
    g = np.random.default_rng(13)
    a = g.standard_normal(2000).astype(np.float32)
    b = (g.standard_normal(2000) * 1e-3).astype(np.float32)
    for x, y in zip(a.tolist(), b.tolist()):
        assert brute.f32(Fraction(x) * Fraction(y)) == Fraction(float(np.float32(x) * np.float32(y)))
        assert brute.f32(Fraction(x) + Fraction(y)) == Fraction(float(np.float32(x) + np.float32(y)))
    assert struct.calcsize("<f") == 4
