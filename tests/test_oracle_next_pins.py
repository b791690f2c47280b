"""Pins of the oracle's definitions for the extensions of the path: aligned
scale offsets, even-mode MXFP4 scales, packed MXFP4 rows, the combine
epilogue and int64 routing maps.  CPU only."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests import _brute as brute
from tests.test_oracle_pins import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SENT = 0xFFFFFFFF


# ------------------------------------------------------------------ scales_offset
def test_scales_offset_worked_example():
    d = json.load(open(os.path.join(GOLDEN, "worked_example_path.json")))
    m = oracle.mask_routing_padding(np.array(d["routing_map"], np.int32), d["real_token_count"])
    r = oracle.create_indices(m, d["n_experts"], scales_align=4)
    # active experts 0, 2, 3 hold 1, 2, 1 slots -> padded to 4 each
    assert r["scales_offset"].tolist() == [0, 4, 8, 12, 12]


@pytest.mark.parametrize("seed", range(8))
def test_scales_offset_against_brute(seed):
    g = np.random.default_rng(600 + seed)
    e = int(g.integers(1, 12))
    ids = g.integers(-2, e + 2, size=int(g.integers(0, 60))).astype(np.int32)
    align = int(g.choice([1, 2, 3, 8, 128]))
    r = oracle.create_indices(ids, e, scales_align=align)
    assert r["scales_offset"].tolist() == brute.scales_offset(ids.tolist(), e, align)


@pytest.mark.parametrize("cfg", range(len(workloads.WORKLOADS)))
def test_scales_offset_invariants_on_workloads(cfg):
    w = workloads.WORKLOADS[cfg]
    ids, _, real = workloads.make_routing(w, cfg)
    m = oracle.mask_routing_padding(ids, real)
    for align in (1, 32, 128):
        r = oracle.create_indices(m, w.n_experts, scales_align=align)
        a = int(r["expert_usage_stats"][1])
        so = r["scales_offset"].astype(np.int64)
        esi = r["expert_start_indices"].astype(np.int64)
        cnt = np.diff(esi[: a + 1])
        assert so[0] == 0 and np.all(so % align == 0)
        gaps = np.diff(so[: a + 1])
        assert np.all(gaps >= cnt) and np.all(gaps < cnt + align)
        assert np.all(so[a:] == so[a])
        if align == 1:
            np.testing.assert_array_equal(so, esi)


# ------------------------------------------------------------------ even-mode MXFP4
def _block(v):
    blk = np.zeros(32, np.uint16)
    if "bits" in v:
        for i, b in enumerate(v["bits"]):
            blk[i] = int(b, 16)
    else:
        blk[: len(v["values"])] = to_bf16_bits(v["values"])
    return blk


def test_even_hand_vectors():
    d = json.load(open(os.path.join(GOLDEN, "mxfp4_vectors.json")))
    for v in d["even_vectors"]:
        q, s = oracle.mxfp4_quantize(_block(v)[None], even=True)
        head = [int(h, 16) for h in v["payload_head"]]
        assert s[0, 0] == int(v["scale"], 16), v["why"]
        assert list(q[0, : len(head)]) == head, v["why"]


def test_even_scale_exhaustive_over_block_maxima():
    """Every finite bf16 value as the block maximum: the oracle's even-mode
    scale byte equals the exact round-then-floor definition."""
    b = np.arange(1 << 15, dtype=np.uint32).astype(np.uint16)   # non-negative patterns
    b = b[((b >> 7) & 0xFF) != 0xFF]
    blocks = np.zeros((b.size, 32), np.uint16)
    blocks[:, 0] = b
    _, s = oracle.mxfp4_quantize(blocks, even=True)
    for i, bits in enumerate(b.tolist()):
        assert s[i, 0] == brute.even_scale_byte([bits] + [0] * 31), hex(bits)


def test_even_differs_from_floor_only_by_one_binade():
    g = np.random.default_rng(33)
    x = to_bf16_bits(g.standard_normal(64 * 32) * np.exp(g.normal(0, 3, 64 * 32))).reshape(64, 32)
    _, s_floor = oracle.mxfp4_quantize(x)
    _, s_even = oracle.mxfp4_quantize(x, even=True)
    d = s_even.astype(int) - s_floor.astype(int)
    assert set(np.unique(d)) <= {0, 1}
    # a block max whose scaled value would be >= 7 moves up a binade, everything else stays
    amax = np.abs(oracle.bf16_bits_to_f32(x).astype(np.float64)).max(axis=1)
    scaled = amax * np.ldexp(1.0, 127 - s_floor[:, 0].astype(int))
    np.testing.assert_array_equal(d[:, 0] == 1, scaled >= 7.0)


@pytest.mark.parametrize("seed", range(3))
def test_even_rows_against_brute(seed):
    g = np.random.default_rng(700 + seed)
    x = to_bf16_bits(g.standard_normal(2 * 96) * np.exp(g.normal(0, 2, 2 * 96))).reshape(2, 96)
    q, s = oracle.mxfp4_quantize(x, even=True)
    for r in range(2):
        for b in range(3):
            blk = x[r, 32 * b: 32 * b + 32].tolist()
            sb = brute.even_scale_byte(blk)
            assert s[r, b] == sb
            unit = Fraction(2) ** (sb - 127)
            for i, bits in enumerate(blk):
                v, sgn = brute.bf16_value(bits)
                a = abs(v) / unit
                best, bd = None, None
                for code, gv in enumerate(brute.E2M1):
                    dd = abs(a - gv)
                    if best is None or dd < bd or (dd == bd and code % 2 == 0):
                        best, bd = code, dd
                nib = (q[r, 16 * b + i // 2] >> (4 * (i % 2))) & 0xF
                assert nib == (best | (8 if sgn else 0))


def test_packed_rows_are_payload_then_scales():
    g = np.random.default_rng(34)
    n, k, e, h = 12, 3, 5, 512
    ids = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    r = oracle.create_indices(ids, e)
    x = to_bf16_bits(g.standard_normal(n * h)).reshape(n, h)
    q, s = oracle.dispatch_mxfp4(x, r["token_expert_order"], k, r["n_routed"])
    packed = oracle.dispatch_mxfp4(x, r["token_expert_order"], k, r["n_routed"], packed=True)
    assert packed.shape == (r["n_routed"], h // 2 + h // 32)
    for p in range(r["n_routed"]):
        assert bytes(packed[p]) == bytes(q[p]) + bytes(s[p])


# ------------------------------------------------------------------ combine epilogue
@pytest.mark.parametrize("seed", range(4))
def test_combine_epilogue_against_brute(seed):
    g = np.random.default_rng(800 + seed)
    n, k, h = 4, 3, 10
    ids = g.integers(-1, 3, size=(n, k)).astype(np.int32)
    r = oracle.create_indices(ids, 3)
    v = max(r["n_routed"], 1)
    y = to_bf16_bits(g.standard_normal(v * h)).reshape(v, h)
    w = g.random((n, k)).astype(np.float32)
    res = to_bf16_bits(g.standard_normal(n * h) * 4).reshape(n, h)
    scale = float(np.float32(g.choice([1.0, 2.5, -0.7, 1e-3])))
    for residual in (None, res):
        out = oracle.combine_epilogue(y, w, r["restore_token_order"], k, scale, residual)
        for t in range(n):
            want = brute.combine_epilogue_row(w[t].tolist(), y.tolist(), r["restore_token_order"][t * k:(t + 1) * k].tolist(),
                                              scale, None if residual is None else residual[t].tolist())
            for c in range(h):
                assert brute.bf16_value(int(out[t, c]))[0] == want[c]


def test_combine_epilogue_identity_and_rounding_order():
    g = np.random.default_rng(35)
    n, k, h = 6, 2, 16
    y = to_bf16_bits(g.standard_normal(n * k * h)).reshape(n * k, h)
    w = g.random((n, k)).astype(np.float32)
    restore = g.permutation(n * k).astype(np.uint32)
    np.testing.assert_array_equal(oracle.combine_epilogue(y, w, restore, k, 1.0, None),
                                  oracle.combine(y, w, restore, k))
    # scale then residual, each rounded: 3 * (1 + 2^-23) rounds before +(-3) is added
    yy = to_bf16_bits([1.0]).reshape(1, 1)
    ww = np.array([[1 + 2.0 ** -23]], np.float32)
    rr = to_bf16_bits([-3.0]).reshape(1, 1)
    out = oracle.combine_epilogue(yy, ww, np.array([0], np.uint32), 1, 3.0, rr)
    exact = Fraction(3) * Fraction(float(ww[0, 0])) - 3
    assert brute.bf16_value(int(out[0, 0]))[0] == brute.bf16(brute.f32(Fraction(3) * Fraction(float(ww[0, 0]))) - 3)
    assert exact != 0 and brute.bf16_value(int(out[0, 0]))[0] == brute.bf16(Fraction(2) ** -21)


# ------------------------------------------------------------------ int64 routing map
def test_int64_ids_equal_int32_after_clipping_garbage():
    g = np.random.default_rng(36)
    e = 10
    ids64 = g.choice(np.array([-1, -(2 ** 40), 2 ** 31, 2 ** 40, e, 3, 7, 0, 9], np.int64), size=(50, 4))
    m64 = oracle.mask_routing_padding(ids64, 40)
    r64 = oracle.create_indices(m64, e)
    ids32 = np.where((ids64 >= 0) & (ids64 < e), ids64, -1).astype(np.int32)
    r32 = oracle.create_indices(oracle.mask_routing_padding(ids32, 40), e)
    for key in ("token_expert_order", "restore_token_order", "expert_start_indices", "expert_ids",
                "expert_usage_stats"):
        np.testing.assert_array_equal(r64[key], r32[key])
    assert m64.dtype == np.int64 and np.all(m64[40:] == -1)
