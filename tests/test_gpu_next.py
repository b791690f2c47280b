"""GPU parity of the extensions: aligned scale offsets, int64 routing maps,
even-mode and packed MXFP4 dispatch, the fused combine epilogue, and the
fused mask + index call."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _oracle_threads as oracle_threads
from tests.gpu_common import SENT, bf16_from_bits, check_indices, gpu_available, i32, u16, u32

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]
mod = pytest.importorskip("expert_grouping_dispatch_amd") if gpu_available() else None
DEV = "cuda"


def _indices(d_ids, e, align=None):
    s = d_ids.numel()
    idx = mod.alloc_indices(s, e, DEV, scales_offset=align is not None)
    mod.moe_create_indices(d_ids, e, idx["token_expert_order"], idx["expert_start_indices"],
                           idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"],
                           idx["workspace"], idx["scales_offset"], align or 1)
    torch.cuda.synchronize()
    return idx


@pytest.mark.parametrize("cfg", range(len(workloads.WORKLOADS)))
@pytest.mark.parametrize("align", [1, 16, 128, 1000])
def test_scales_offset_on_workloads(cfg, align):
    w = workloads.WORKLOADS[cfg]
    ids, _, real = workloads.make_routing(w, cfg)
    m = oracle.mask_routing_padding(ids, real)
    idx = _indices(torch.from_numpy(m).to(DEV), w.n_experts, align)
    ref = oracle.create_indices(m, w.n_experts, scales_align=align)
    check_indices(idx, ref)
    np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])


@pytest.mark.parametrize("n,k,e", [(0, 4, 16), (50, 3, 1), (1000, 8, 1024), (20000, 8, 256)])
def test_scales_offset_edges(n, k, e):
    g = np.random.default_rng(n + e)
    ids = g.integers(-3, e + 3, size=(n, k)).astype(np.int32)
    idx = _indices(torch.from_numpy(ids).to(DEV), e, 64)
    ref = oracle.create_indices(ids, e, scales_align=64)
    check_indices(idx, ref)
    np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])


@pytest.mark.parametrize("n,k,e,real", [(300, 4, 16, 211), (20000, 8, 256, 17000), (2, 2, 3, 5)])
def test_int64_routing_map(n, k, e, real):
    g = np.random.default_rng(n)
    pool = np.array([-1, -(2 ** 40), 2 ** 31, 2 ** 33 + 1, e, -5] + list(range(e)), np.int64)
    ids = g.choice(pool, size=(n, k))
    d_ids = torch.from_numpy(ids).to(DEV)
    cnt = torch.tensor([real], dtype=torch.int32, device=DEV)
    mod.moe_mask_padding(d_ids, cnt, 0)
    m = oracle.mask_routing_padding(ids, real)
    np.testing.assert_array_equal(d_ids.cpu().numpy(), m)
    idx = _indices(d_ids, e, 32)
    ref = oracle.create_indices(m, e, scales_align=32)
    check_indices(idx, ref)
    np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])


def _mxfp4_case(xb, ids, e, k, flags):
    n, h = xb.shape
    x = bf16_from_bits(xb, DEV)
    ref = oracle.create_indices(ids, e)
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    packed = bool(flags & mod.MXFP4_PACKED_ROWS)
    q, sc = mod.alloc_dispatch_mxfp4(n * k, h, DEV, packed=packed)
    mod.moe_dispatch_mxfp4(x, k, restore, q, sc, flags=flags)
    torch.cuda.synchronize()
    v = ref["n_routed"]
    want = oracle.dispatch_mxfp4(xb, ref["token_expert_order"], k, v,
                                 even=bool(flags & mod.MXFP4_EVEN_SCALE), packed=packed)
    if packed:
        np.testing.assert_array_equal(q[:v].cpu().numpy(), want)
    else:
        np.testing.assert_array_equal(q[:v].cpu().numpy(), want[0])
        np.testing.assert_array_equal(sc[:v].cpu().numpy(), want[1])


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_mxfp4_modes_on_decode_workload(flags):
    w = workloads.WORKLOADS[3]
    ids, _, real = workloads.make_routing(w, 3)
    x, _ = workloads.make_dense(w, 3, DEV, y_rows=1)
    _mxfp4_case(u16(x), oracle.mask_routing_padding(ids, real), w.n_experts, w.top_k, flags)


@pytest.mark.parametrize("flags", [1, 3])
def test_mxfp4_even_special_blocks(flags):
    g = np.random.default_rng(51)
    h = 1024
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[((allb >> 7) & 0xFF) != 0xFF]
    rows = [np.zeros(h, np.uint16), np.full(h, 0x7F7F, np.uint16), g.choice(finite, size=h).astype(np.uint16)]
    # block maxima right around the even-mode threshold (mantissa 0x5F / 0x60 / 0x7F)
    for mant in (0x5F, 0x60, 0x7F, 0x00):
        r = g.integers(0, 0x3F00, size=h).astype(np.uint16)
        r[::32] = ((g.integers(100, 160, size=h // 32) << 7) | mant).astype(np.uint16)
        rows.append(r)
    for s in range(5):
        f = g.standard_normal(h).astype(np.float32)
        f[::32] *= 10.0 ** (s * 5 - 12)
        rows.append(oracle.f32_to_bf16_rne(f))
    xb = np.stack(rows)
    n = xb.shape[0]
    ids = (np.stack([np.arange(3) + t for t in range(n)]) % 5).astype(np.int32)
    _mxfp4_case(xb, ids, 5, 3, flags)


def _every_finite_blocks(seed, h):
    """Blocks of 32 bf16 values covering every finite pattern under every
    block maximum exponent B (0..254): each block holds one anchor of
    exponent B plus 31 patterns of exponent <= B, both signs, so each finite
    value is quantized against every scale that a block containing it can
    have."""
    g = np.random.default_rng(seed)
    mags = np.arange(0x7F80, dtype=np.uint16)
    blocks = []
    for b in range(255):
        vals = np.concatenate([mags[: (b + 1) << 7], mags[: (b + 1) << 7] | 0x8000]).astype(np.uint16)
        g.shuffle(vals)
        n = -(-vals.size // 31)
        vals = np.concatenate([vals, g.choice(vals, n * 31 - vals.size)]).reshape(n, 31)
        anchor = ((np.uint16(b) << 7) | (g.integers(0, 2, n) << 15)).astype(np.uint16)
        blk = np.concatenate([anchor[:, None], vals], axis=1)
        blocks.append(np.take_along_axis(blk, np.argsort(g.random((n, 32)), axis=1), axis=1))
    allb = np.concatenate(blocks)
    allb = np.concatenate([allb, allb[: (-allb.shape[0]) % (h // 32)]])
    return allb.reshape(-1, h)


@pytest.mark.parametrize("flags", [0, 1])
def test_mxfp4_every_finite_value_under_every_scale(flags):
    """8.6M elements: the element rounding and the scale rule, bit-exact,
    over the whole finite bf16 domain."""
    xb = _every_finite_blocks(7 + flags, 8192)
    ids = np.zeros((xb.shape[0], 1), np.int32)
    _mxfp4_case(xb, ids, 1, 1, flags)


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_mxfp4_every_finite_value_wide_output(flags):
    """The four-lanes-per-block MXFP4 kernel (outputs of 256 MiB or more with
    top_k <= 8): every finite bf16 value under every block scale, in both
    scale modes and both layouts, bit-exact against the oracle.  8000 tokens
    tile the distinct rows of the exhaustive blocks, and each token goes to
    all 8 experts (in a seeded order), so every row is written 8 times.  x
    holds 131 MB, under the 256 MiB from which that kernel loads x
    non-temporally, so this case takes its plain loads."""
    even, packed = bool(flags & mod.MXFP4_EVEN_SCALE), bool(flags & mod.MXFP4_PACKED_ROWS)
    xu = _every_finite_blocks(7 + int(even), 8192)
    n, k, e, h = 8000, 8, 8, 8192
    assert n * k * (h // 32) * 17 >= 256 << 20
    print(f"[parity] MXFP4 wide output, every finite value, flags={flags}", flush=True)
    x = bf16_from_bits(xu[np.arange(n) % xu.shape[0]], DEV)
    g = np.random.default_rng(300 + flags)
    ids = np.argsort(g.random((n, e)), axis=1)[:, :k].astype(np.int32)
    ref = oracle.create_indices(ids, e)
    v = ref["n_routed"]
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    q, sc = mod.alloc_dispatch_mxfp4(n * k, h, DEV, packed=packed)
    mod.moe_dispatch_mxfp4(x, k, restore, q, sc, flags=flags)
    torch.cuda.synchronize()
    pq, ps = oracle_threads.mxfp4_quantize_rows(xu, even)
    want = torch.from_numpy(np.concatenate([pq, ps], axis=1) if packed else pq).to(DEV)
    want_s = None if packed else torch.from_numpy(ps).to(DEV)
    src = torch.from_numpy((ref["token_expert_order"][:v].astype(np.int64) // k) % xu.shape[0]).to(DEV)
    block = 16384
    for p0 in range(0, v, block):
        sl = slice(p0, min(v, p0 + block))
        assert torch.equal(q[sl], want[src[sl]]), p0
        if want_s is not None:
            assert torch.equal(sc[sl], want_s[src[sl]]), p0


@pytest.mark.parametrize("n, flags", [(16383, 0), (16384, 0), (16384, 1), (16384, 2), (16384, 3)])
def test_mxfp4_wide_output_at_the_non_temporal_load_switch(n, flags):
    """The four-lanes-per-block kernel loads x non-temporally once x holds
    256 MiB: 16,383 tokens of 8192 elements fall one row short (plain loads),
    16,384 hold exactly 256 MiB (non-temporal loads, in both scale modes and
    both layouts).  Every routed row of 400 sampled tokens, payload and scale
    bytes, against the oracle."""
    k, e, h = 8, 64, 8192
    even, packed = bool(flags & mod.MXFP4_EVEN_SCALE), bool(flags & mod.MXFP4_PACKED_ROWS)
    assert (n * h * 2 >= 256 << 20) == (n == 16384)
    assert n * k * (h // 32) * 17 >= 256 << 20
    print(f"[parity] MXFP4 wide output at the load switch, n={n} flags={flags}", flush=True)
    g = np.random.default_rng(500 + n + 10 * flags)
    ids = np.argsort(g.random((n, e), dtype=np.float32), axis=1)[:, :k].astype(np.int32)
    ref = oracle.create_indices(ids, e)
    gen = torch.Generator(device=DEV).manual_seed(600 + n + 10 * flags)
    x = (torch.randn((n, h), generator=gen, device=DEV) * 4).to(torch.bfloat16)
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    q, sc = mod.alloc_dispatch_mxfp4(n * k, h, DEV, packed=packed)
    mod.moe_dispatch_mxfp4(x, k, restore, q, sc, flags=flags)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([g.integers(0, n, size=398), [0, n - 1]]))
    pq, ps = oracle.mxfp4_quantize(u16(x[torch.from_numpy(toks).to(DEV)]), even=even)
    pos = ref["restore_token_order"].reshape(n, k)[toks].astype(np.int64)   # k distinct experts: all routed
    d_pos = torch.from_numpy(pos.reshape(-1)).to(DEV)
    if packed:
        np.testing.assert_array_equal(q[d_pos].cpu().numpy(), np.repeat(np.concatenate([pq, ps], axis=1), k, axis=0))
    else:
        np.testing.assert_array_equal(q[d_pos].cpu().numpy(), np.repeat(pq, k, axis=0))
        np.testing.assert_array_equal(sc[d_pos].cpu().numpy(), np.repeat(ps, k, axis=0))


def test_mxfp4_packed_full_size_sampled():
    """The outlier workload in even + packed mode, checked on sampled rows."""
    w = workloads.WORKLOADS[2]
    ids, _, real = workloads.make_routing(w, 2)
    x, _ = workloads.make_dense(w, 2, DEV, y_rows=1)
    m = oracle.mask_routing_padding(ids, real)
    ref = oracle.create_indices(m, w.n_experts)
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    s, h, k = w.n_slots, w.hidden, w.top_k
    q, _ = mod.alloc_dispatch_mxfp4(s, h, DEV, packed=True)
    mod.moe_dispatch_mxfp4(x, k, restore, q, None, flags=mod.MXFP4_EVEN_SCALE | mod.MXFP4_PACKED_ROWS)
    torch.cuda.synchronize()
    g = np.random.default_rng(2)
    pos = np.unique(g.integers(0, ref["n_routed"], size=600))
    src = ref["token_expert_order"][pos].astype(np.int64) // k
    xs = u16(x[torch.from_numpy(src).to(DEV)])
    pq, ps = oracle.mxfp4_quantize(xs, even=True)
    np.testing.assert_array_equal(q[torch.from_numpy(pos).to(DEV)].cpu().numpy(), np.concatenate([pq, ps], axis=1))


def _combine_epi_case(n, k, e, h, scale, with_residual, seed):
    g = np.random.default_rng(seed)
    ids = g.integers(-1, e, size=(n, k)).astype(np.int32)
    ref = oracle.create_indices(ids, e)
    v = max(ref["n_routed"], 1)
    yb = oracle.f32_to_bf16_rne((g.standard_normal((v, h)) * np.exp(g.normal(0, 2, (v, h)))).astype(np.float32))
    rb = oracle.f32_to_bf16_rne((g.standard_normal((n, h)) * 3).astype(np.float32)) if with_residual else None
    w = g.random((n, k)).astype(np.float32)
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    out = torch.empty((n, h), dtype=torch.bfloat16, device=DEV)
    mod.moe_combine_epilogue(bf16_from_bits(yb, DEV), torch.from_numpy(w).to(DEV), restore, k, out, scale,
                             None if rb is None else bf16_from_bits(rb, DEV))
    torch.cuda.synchronize()
    want = oracle.combine_epilogue(yb, w, ref["restore_token_order"], k, scale, rb)
    np.testing.assert_array_equal(u16(out), want)


@pytest.mark.parametrize("scale", [1.0, 2.5, -0.75, 1e-30])
@pytest.mark.parametrize("with_residual", [False, True])
@pytest.mark.parametrize("k", [1, 8, 11])
def test_combine_epilogue(scale, with_residual, k):
    _combine_epi_case(300, k, 16, 7168 // 7, scale, with_residual, 60 + k)


def test_combine_epilogue_whole_rows_sampled():
    """top_k = 8 with over 1 GiB of routed y rows (9400 tokens, H = 7168),
    which the whole-row combine kernel takes: the epilogue with a residual on
    64 sampled tokens (real and fully unrouted ones) against the oracle."""
    n, k, e, h, scale = 9400, 8, 64, 7168, 0.75
    print(f"[parity] combine epilogue n={n} k={k} h={h}", flush=True)
    g = np.random.default_rng(777)
    ids = g.integers(0, e, size=(n, k)).astype(np.int32)
    ids[g.choice(n, 40, replace=False)] = -1
    ref = oracle.create_indices(ids, e)
    v = ref["n_routed"]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(778)
    y = torch.randn((v, h), generator=gen, device=DEV).to(torch.bfloat16)
    res = (torch.randn((n, h), generator=gen, device=DEV) * 3).to(torch.bfloat16)
    w = g.random((n, k)).astype(np.float32)
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    out = torch.empty((n, h), dtype=torch.bfloat16, device=DEV)
    mod.moe_combine_epilogue(y, torch.from_numpy(w).to(DEV), restore, k, out, scale, res)
    torch.cuda.synchronize()
    unrouted = np.flatnonzero((ids < 0).all(axis=1))
    tok = np.unique(np.concatenate([g.choice(n, 56, replace=False), unrouted[:8]]))
    pos = ref["restore_token_order"].reshape(n, k)[tok]
    routed = pos != SENT
    rows = np.unique(pos[routed]).astype(np.int64)
    ysub = u16(y[torch.from_numpy(rows).to(DEV)])
    local = np.full(pos.shape, SENT, dtype=np.uint32)
    local[routed] = np.searchsorted(rows, pos[routed]).astype(np.uint32)
    want = oracle.combine_epilogue(ysub, w[tok], local.reshape(-1), k, scale,
                                   u16(res[torch.from_numpy(tok).to(DEV)]))
    np.testing.assert_array_equal(u16(out[torch.from_numpy(tok).to(DEV)]), want)


@pytest.mark.parametrize("cfg", [3, 1])   # decode; mixtral_prefill, whose y and output take plain stores
def test_combine_epilogue_matches_combine_at_identity(cfg):
    w = workloads.WORKLOADS[cfg]
    ids, wts, real = workloads.make_routing(w, cfg)
    x, y = workloads.make_dense(w, cfg, DEV)
    print(f"[parity] combine epilogue at identity and with a residual: {w.name}", flush=True)
    m = oracle.mask_routing_padding(ids, real)
    ref = oracle.create_indices(m, w.n_experts)
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    d_w = torch.from_numpy(wts).to(DEV)
    a = torch.empty((w.n_rows, w.hidden), dtype=torch.bfloat16, device=DEV)
    b = torch.empty_like(a)
    mod.moe_combine(y, d_w, restore, w.top_k, a)
    mod.moe_combine_epilogue(y, d_w, restore, w.top_k, b, 1.0, None)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    res = x.clone()
    mod.moe_combine_epilogue(y, d_w, restore, w.top_k, b, 0.5, res)
    torch.cuda.synchronize()
    want = oracle.combine_epilogue(u16(y), wts, ref["restore_token_order"], w.top_k, 0.5, u16(res))
    np.testing.assert_array_equal(u16(b), want)


# ---------------------------------------------------------------- fused mask + indices
def _fused(ids, real, tp_rank, e, align=None):
    d_map = torch.from_numpy(np.ascontiguousarray(ids)).to(DEV)
    cnt = torch.tensor([real], dtype=torch.int32, device=DEV)
    idx = mod.alloc_indices(d_map.numel(), e, DEV, scales_offset=align is not None)
    mod.moe_mask_create_indices(d_map, cnt, tp_rank, e, idx["token_expert_order"], idx["expert_start_indices"],
                                idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"],
                                idx["workspace"], idx["scales_offset"], align or 1)
    torch.cuda.synchronize()
    return d_map, idx


def _check_fused(ids, real, tp_rank, e, align=None):
    d_map, idx = _fused(ids, real, tp_rank, e, align)
    m = oracle.mask_routing_padding(ids, real, tp_rank)
    np.testing.assert_array_equal(d_map.cpu().numpy(), m)
    ref = oracle.create_indices(m, e, scales_align=align)
    check_indices(idx, ref)
    if align is not None:
        np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])
    assert mod.index_workspace_error(idx["workspace"]) == 0


@pytest.mark.parametrize("cfg", range(len(workloads.WORKLOADS)))
def test_fused_mask_indices_on_workloads(cfg):
    w = workloads.WORKLOADS[cfg]
    ids, _, real = workloads.make_routing(w, cfg)
    _check_fused(ids, real, 0, w.n_experts)


@pytest.mark.parametrize("n,k,e,real,tp_rank", [
    (256, 8, 256, 97, 0),            # one workgroup (2048 slots)
    (257, 8, 256, 97, 0),            # two chunks
    (3000, 4, 16, 0, 0),             # everything masked
    (3000, 4, 16, 3000, 0),          # nothing masked
    (3000, 4, 16, -7, 0),
    (3000, 4, 16, 3000 + 1234, 1),   # second shard: boundary 1234
    (3000, 4, 16, 2 ** 31 - 1, 715827),
    (40000, 8, 1024, 39999, 0),
    (1, 1, 1, 1, 0),
    (0, 4, 8, 0, 0),
])
def test_fused_mask_indices_edges(n, k, e, real, tp_rank):
    g = np.random.default_rng(n + k + e)
    ids = g.integers(-2, e + 2, size=(n, k)).astype(np.int32)
    _check_fused(ids, real, tp_rank, e)


# The one-workgroup index pass launches the fewest whole waves that hold the
# slots (2 per lane): each side of every wave-count step, up to the largest
# one-workgroup input (2048 slots) and the first two-chunk input.
@pytest.mark.parametrize("s", [1, 128, 129, 256, 257, 512, 513, 1024, 1025, 2047, 2048, 2049])
@pytest.mark.parametrize("e", [8, 1024])
def test_indices_one_workgroup_sizes(s, e):
    g = np.random.default_rng(s * 7 + e)
    ids = g.integers(-1, e + 1, size=(s, 1)).astype(np.int32)
    print(f"[parity] one-workgroup indices: S={s} E={e}", flush=True)
    d = torch.from_numpy(ids.reshape(-1)).to(DEV)
    idx = mod.alloc_indices(s, e, DEV, scales_offset=True)
    mod.moe_create_indices(d, e, idx["token_expert_order"], idx["expert_start_indices"], idx["restore_token_order"],
                           idx["expert_ids"], idx["expert_usage_stats"], idx["workspace"], idx["scales_offset"], 16)
    torch.cuda.synchronize()
    ref = oracle.create_indices(ids, e, scales_align=16)
    check_indices(idx, ref)
    np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])
    # the one-call mask + indices on the same slots as rows of 1, masking the last third
    _check_fused(ids, s - s // 3, 0, e, 16)


# The one-launch few-expert index pass: 2 to 32 chunks of 1024 slots with at
# most 8 experts, 2 to 16 chunks with 9 to 16 (8 or 16 counted experts; 8, 16
# or 32 groups per wave), and just past each limit (33 and 17 chunks, 17
# experts); int32 and int64 maps with unrouted and out-of-range ids; the
# separate and the one-call forms.
@pytest.mark.parametrize("s, k, e", [(2049, 1, 1), (2050, 2, 8), (5000, 1, 12), (8199, 1, 8), (16384, 2, 8),
                                     (16384, 1, 16), (16385, 1, 16), (24000, 3, 9), (32768, 2, 8),
                                     (32769, 1, 8), (20000, 4, 17)])
@pytest.mark.parametrize("dtype", [np.int32, np.int64])
def test_index_few_expert_path(s, k, e, dtype):
    n = s // k
    g = np.random.default_rng(s * 31 + e)
    pool = [-1, -5, e, e + 5] + list(range(e)) * 3
    if dtype == np.int64:
        pool += [-(2 ** 40), 2 ** 31, 2 ** 33 + 1]
    ids = g.choice(np.array(pool, np.int64), size=(n, k)).astype(dtype)
    print(f"[parity] few-expert indices: S={s} k={k} E={e} {np.dtype(dtype).name}", flush=True)
    idx = _indices(torch.from_numpy(ids).to(DEV), e, 16)
    ref = oracle.create_indices(ids, e, scales_align=16)
    check_indices(idx, ref)
    np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])
    # masking from inside a chunk, and everything masked
    _check_fused(ids, n - n // 3 - 5, 0, e, 16)
    _check_fused(ids, 0, 0, e)


@pytest.mark.parametrize("seed", range(4))
def test_index_random_shapes_around_the_few_expert_limits(seed):
    """Seeded random inputs on both sides of the few-expert pass's limits
    (experts 1-17, 1 to 40,000 slots, top_k 1-8), int32 and int64 maps,
    uniform, skewed and garbage ids, separate and one-call forms with random
    counts and scale alignments: every index output against the oracle."""
    g = np.random.default_rng(4200 + seed)
    for c in range(50):
        e = int(g.choice([1, 2, 3, 5, 7, 8, 9, 12, 15, 16, 17]))
        k = int(g.choice([1, 2, 3, 4, 6, 8]))
        s = int(g.choice([g.integers(1, 2049), g.integers(2049, 16385), g.integers(16385, 32770),
                          g.integers(32769, 40000)]))
        n = max(1, s // k)
        dt = np.int64 if g.random() < 0.3 else np.int32
        kind = str(g.choice(["uniform", "skew", "garbage"]))
        if kind == "uniform":
            ids = g.integers(0, e, size=(n, k))
        elif kind == "skew":
            ids = np.minimum(g.geometric(0.5, size=(n, k)) - 1, e - 1)
        else:
            pool = [-1, -7, e, e + 3] + list(range(e)) + ([2 ** 33 + 1, -(2 ** 40)] if dt == np.int64 else [])
            ids = g.choice(np.array(pool, np.int64), size=(n, k))
        ids = ids.astype(dt)
        real = int(g.choice([n, n - 1, 0, int(g.integers(0, n + 1)), n + 5]))
        align = int(g.choice([1, 16, 128]))
        print(f"[parity] few-expert sweep seed={seed} case={c}: n={n} k={k} e={e} {np.dtype(dt).name} {kind} "
              f"real={real}", flush=True)
        if g.random() < 0.5:
            _check_fused(ids, real, 0, e, align)
        else:
            idx = _indices(torch.from_numpy(ids).to(DEV).view(-1), e, align)
            ref = oracle.create_indices(ids, e, scales_align=align)
            check_indices(idx, ref)
            np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])
            assert mod.index_workspace_error(idx["workspace"]) == 0


@pytest.mark.parametrize("s, e", [(32768, 8), (16384, 16)])
def test_index_few_expert_path_one_expert(s, e):
    """Every slot on one expert: the largest counts the pass keeps per wave."""
    ids = np.full((s, 1), e - 1, np.int32)
    idx = _indices(torch.from_numpy(ids).to(DEV), e)
    check_indices(idx, oracle.create_indices(ids, e))


@pytest.mark.parametrize("align", [1, 128])
def test_fused_mask_indices_int64_and_offsets(align):
    n, k, e, real = 5000, 8, 256, 4321
    g = np.random.default_rng(7)
    pool = np.array([-1, 2 ** 33 + 1, e, -(2 ** 40)] + list(range(e)), np.int64)
    ids = g.choice(pool, size=(n, k))
    _check_fused(ids, real, 0, e, align)


def test_fused_equals_separate_calls():
    """Same map bytes and index outputs as moe_mask_padding then moe_create_indices."""
    w = workloads.WORKLOADS[4]
    ids, _, real = workloads.make_routing(w, 4)
    d_map, fused = _fused(ids, real, 0, w.n_experts)
    d_sep = torch.from_numpy(ids).to(DEV)
    mod.moe_mask_padding(d_sep, torch.tensor([real], dtype=torch.int32, device=DEV), 0)
    sep = _indices(d_sep, w.n_experts)
    assert torch.equal(d_map, d_sep)
    for key in ("token_expert_order", "expert_start_indices", "restore_token_order", "expert_ids",
                "expert_usage_stats"):
        assert torch.equal(fused[key].view(torch.int32), sep[key].view(torch.int32)), key
