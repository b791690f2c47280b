"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact on the masked routing map, every index output, bf16 dispatch rows
and MXFP4 payload / scale bytes; combine within 1 bf16 ulp (and bit-exact
in practice: the kernel does the same fp32 operations in the same order).
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _oracle_threads as oracle_threads
from tests.gpu_common import (SENT, bf16_from_bits, bf16_ulp_distance, check_indices, gpu_available, i32,
                              run_path, u16, u32)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

mod = pytest.importorskip("expert_grouping_dispatch_amd") if gpu_available() else None
DEV = "cuda"


def _oracle_front(ids, real, n_experts, tp_rank=0):
    m = oracle.mask_routing_padding(ids, real, tp_rank)
    return m, oracle.create_indices(m, n_experts)


def _check_combine(got_bits, want_bits, exact=True):
    d = bf16_ulp_distance(got_bits, want_bits)
    assert int(d.max(initial=0)) <= 1, f"combine off by {int(d.max())} ulp"
    if exact:
        assert int((got_bits != want_bits).sum()) == 0, "combine not bit-exact"


def _full_check(ids, w, real, n_experts, x, y, variants, tp_rank=0):
    """Everything compared element by element."""
    n, k = ids.shape
    res = run_path(mod, ids, real, n_experts, x, y, w, variants, tp_rank)
    m, ref = _oracle_front(ids, real, n_experts, tp_rank)
    np.testing.assert_array_equal(i32(res["ids"]), m)
    check_indices(res, ref)
    v = ref["n_routed"]
    xb = u16(x)
    if "bf16" in variants:
        want = oracle.dispatch(xb, ref["token_expert_order"], k, v)
        np.testing.assert_array_equal(u16(res["dispatch"][:v]), want)
    if "mxfp4" in variants:
        wq, ws = oracle.dispatch_mxfp4(xb, ref["token_expert_order"], k, v)
        np.testing.assert_array_equal(res["q"][:v].cpu().numpy(), wq)
        np.testing.assert_array_equal(res["scales"][:v].cpu().numpy(), ws)
    if y is not None:
        want = oracle.combine(u16(y), w, ref["restore_token_order"], k)
        _check_combine(u16(res["combine"]), want)
    return res, ref


# ---------------------------------------------------------------- workloads
@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_workload_full(cfg):
    w = workloads.WORKLOADS[cfg]
    ids, wts, real = workloads.make_routing(w, cfg)
    x, y = workloads.make_dense(w, cfg, DEV)
    print(f"[parity] workload {w.name} full", flush=True)
    _full_check(ids, wts, real, w.n_experts, x, y, ("bf16", "mxfp4"))


def _sample_positions(esi, a, v, g, n=512):
    edges = np.concatenate([esi[:a], np.maximum(esi[1:a + 1].astype(np.int64) - 1, 0)]).astype(np.int64)
    rnd = g.integers(0, v, size=n)
    return np.unique(np.concatenate([edges, rnd, [0, v - 1]]))


@pytest.mark.parametrize("cfg", [2, 4])
def test_workload_full_size_sampled(cfg):
    """Full-size workloads in the launch configuration the bench times:
    indices compared in full, dispatch / MXFP4 / combine on sampled rows."""
    w = workloads.WORKLOADS[cfg]
    ids, wts, real = workloads.make_routing(w, cfg)
    x, y = workloads.make_dense(w, cfg, DEV)
    print(f"[parity] workload {w.name} full size, sampled rows", flush=True)
    res = run_path(mod, ids, real, w.n_experts, x, y, wts, ("bf16", "mxfp4"))
    m, ref = _oracle_front(ids, real, w.n_experts)
    np.testing.assert_array_equal(i32(res["ids"]), m)
    check_indices(res, ref)
    k, v = w.top_k, ref["n_routed"]
    g = np.random.default_rng(cfg)
    pos = _sample_positions(ref["expert_start_indices"], int(ref["expert_usage_stats"][1]), v, g)
    src = ref["token_expert_order"][pos].astype(np.int64) // k
    xs = u16(x[torch.from_numpy(src).to(DEV)])
    pidx = torch.from_numpy(pos).to(DEV)
    np.testing.assert_array_equal(u16(res["dispatch"][pidx]), xs)
    wq, wsc = oracle.mxfp4_quantize(xs)
    np.testing.assert_array_equal(res["q"][pidx].cpu().numpy(), wq)
    np.testing.assert_array_equal(res["scales"][pidx].cpu().numpy(), wsc)
    # combine on sampled tokens (including masked rows when there are any)
    toks = np.unique(np.concatenate([g.integers(0, w.n_rows, size=256), [0, w.n_rows - 1, real - 1,
                                                                          min(real, w.n_rows - 1)]]))
    rs = ref["restore_token_order"].reshape(w.n_rows, k)[toks]
    used = np.unique(rs[rs != SENT]).astype(np.int64)
    ysub = u16(y[torch.from_numpy(used).to(DEV)])
    remap = np.full(rs.shape, SENT, np.uint32)
    remap[rs != SENT] = np.searchsorted(used, rs[rs != SENT].astype(np.int64))
    want = oracle.combine(ysub, wts[toks], remap.reshape(-1), k)
    got = u16(res["combine"][torch.from_numpy(toks).to(DEV)])
    _check_combine(got, want)
    # property at full size: rows with nothing routed are +0
    if real < w.n_rows:
        assert int(res["combine"][real:].view(torch.int16).abs().max()) == 0


@pytest.mark.parametrize("cfg", [2, 4])
def test_workload_full_size_every_row_bf16(cfg):
    """Full-size workloads, every routed bf16 dispatch row: row p is
    x[teo[p] // k] (the oracle's dispatch, a row gather, evaluated on the GPU
    with the oracle's token_expert_order)."""
    w = workloads.WORKLOADS[cfg]
    ids, wts, real = workloads.make_routing(w, cfg)
    x, _ = workloads.make_dense(w, cfg, DEV, y_rows=1)
    print(f"[parity] workload {w.name} full size, every bf16 row", flush=True)
    res = run_path(mod, ids, real, w.n_experts, x, None, wts, ("bf16",))
    _, ref = _oracle_front(ids, real, w.n_experts)
    check_indices(res, ref)
    k, v = w.top_k, ref["n_routed"]
    teo = torch.from_numpy(ref["token_expert_order"][:v].astype(np.int64)).to(DEV)
    block = 32768
    for p0 in range(0, v, block):
        sl = slice(p0, min(v, p0 + block))
        assert torch.equal(res["dispatch"][sl].view(torch.int16), x[teo[sl] // k].view(torch.int16)), p0


@pytest.mark.parametrize("cfg", [2, 4])
def test_workload_full_size_every_row_mxfp4(cfg):
    """Full-size workloads, every routed MXFP4 row (payload and scale bytes)
    against the oracle: each real token is quantized once by
    oracle.mxfp4_quantize (row chunks on host threads) and compared with the
    rows at each of its routed positions.  deepseek_v3_prefill (125 MB of
    output) runs the eager one-lane-per-block kernel, the stress workload
    (1.9 GB) the four-lanes-per-block kernel with non-temporal loads (x of
    939 MB)."""
    w = workloads.WORKLOADS[cfg]
    ids, wts, real = workloads.make_routing(w, cfg)
    x, _ = workloads.make_dense(w, cfg, DEV, y_rows=1)
    print(f"[parity] workload {w.name} full size, every MXFP4 row", flush=True)
    res = run_path(mod, ids, real, w.n_experts, x, None, wts, ("mxfp4",))
    _, ref = _oracle_front(ids, real, w.n_experts)
    check_indices(res, ref)
    n, k = w.n_rows, w.top_k
    # every routed slot belongs to a real token (padding rows are masked)
    assert np.all(ref["restore_token_order"].reshape(n, k)[real:] == SENT)
    wq, wsc = oracle_threads.mxfp4_quantize_rows(u16(x[:real]))
    rest = torch.from_numpy(ref["restore_token_order"].astype(np.int64)).to(DEV).view(n, k)
    sent = torch.tensor(SENT, dtype=torch.int64, device=DEV)
    block = 4096
    for t0 in range(0, real, block):
        t1 = min(real, t0 + block)
        r = rest[t0:t1]
        routed = r != sent
        tok = torch.arange(t1 - t0, device=DEV).view(-1, 1).expand(-1, k)[routed]
        pos = r[routed]
        eq = torch.from_numpy(wq[t0:t1]).to(DEV)
        es = torch.from_numpy(wsc[t0:t1]).to(DEV)
        assert torch.equal(res["q"][pos], eq[tok]), t0
        assert torch.equal(res["scales"][pos], es[tok]), t0


@pytest.mark.parametrize("cfg", [2, 4])
def test_workload_full_size_every_row_combine(cfg):
    """Full-size workloads, every combine output row against oracle.combine:
    the y rows each chunk of tokens reads are gathered on the GPU at the
    oracle's positions, and the oracle runs on them chunk by chunk on host
    threads (rows with nothing routed included: they come out +0).  The
    stress workload runs the whole-row combine kernel, deepseek_v3_prefill
    the loop-free one."""
    w = workloads.WORKLOADS[cfg]
    ids, wts, real = workloads.make_routing(w, cfg)
    x, y = workloads.make_dense(w, cfg, DEV)
    print(f"[parity] workload {w.name} full size, every combine row", flush=True)
    res = run_path(mod, ids, real, w.n_experts, x, y, wts, ())
    _, ref = _oracle_front(ids, real, w.n_experts)
    check_indices(res, ref)
    n, k = w.n_rows, w.top_k
    rest = ref["restore_token_order"].reshape(n, k)
    got = res["combine"]
    block = 2048

    def one(t0):
        t1 = min(n, t0 + block)
        rs = rest[t0:t1]
        routed = rs != SENT
        mini = np.full(rs.shape, SENT, np.uint32)
        mini[routed] = np.arange(int(routed.sum()), dtype=np.uint32)   # row order of the gathered rows
        want = oracle.combine(gathered[t0], wts[t0:t1], mini.reshape(-1), k)
        return t0, want

    gathered = {}
    with cf.ThreadPoolExecutor(oracle_threads.n_threads()) as ex:
        futs = []
        for t0 in range(0, n, block):
            rs = rest[t0:min(n, t0 + block)]
            used = rs[rs != SENT].astype(np.int64)
            gathered[t0] = u16(y[torch.from_numpy(used).to(DEV)]) if used.size else np.zeros((0, w.hidden), np.uint16)
            futs.append(ex.submit(one, t0))
        for f in futs:
            t0, want = f.result()
            t1 = t0 + want.shape[0]
            _check_combine(u16(got[t0:t1]), want)
            del gathered[t0]


# ---------------------------------------------------------------- edge cases
def _rand_case(seed, n, k, e, h, kind="uniform", real=None):
    g = np.random.default_rng(seed)
    if kind == "uniform":
        ids = g.integers(0, e, size=(n, k))
    elif kind == "distinct":
        ids = np.argsort(g.random((n, e)), axis=1)[:, :k]
    elif kind == "garbage":
        pool = np.array([-1, -9, e, e + 5, 2 ** 31 - 1, -2 ** 31] + list(range(e)))
        ids = g.choice(pool, size=(n, k))
    elif kind == "one_expert":
        ids = np.full((n, k), e // 2)
    elif kind == "half_empty":  # only even experts used -> zero-token experts in between
        ids = 2 * g.integers(0, max(1, e // 2), size=(n, k))
    else:
        raise ValueError(kind)
    w = g.random((n, k)).astype(np.float32)
    x = bf16_from_bits(oracle.f32_to_bf16_rne(g.standard_normal((n, h)).astype(np.float32)), DEV)
    y = bf16_from_bits(oracle.f32_to_bf16_rne(g.standard_normal((n * k, h)).astype(np.float32)), DEV)
    return ids.astype(np.int32), w, (n if real is None else real), x, y


@pytest.mark.parametrize("real_case", ["zero", "one", "n_minus_1", "n", "n_plus_5", "neg3"])
@pytest.mark.parametrize("tp_rank", [0, 1])
def test_real_count_edges(real_case, tp_rank):
    n, k, e, h = 300, 4, 16, 64
    real = {"zero": 0, "one": 1, "n_minus_1": n - 1, "n": n, "n_plus_5": n + 5, "neg3": -3}[real_case]
    real += tp_rank * n
    ids, w, _, x, y = _rand_case(1, n, k, e, h, "garbage")
    _full_check(ids, w, real, e, x, y, ("bf16", "mxfp4"), tp_rank)


@pytest.mark.parametrize("real, tp_rank", [(2 ** 31 - 1, 0), (2 ** 31 - 1, 2 ** 31 - 1), (-2 ** 31, 0),
                                           (-2 ** 31, 5), (2 ** 31 - 1, 7158278), (150 + 300 * 7158278, 7158278)])
def test_count_and_rank_extremes(real, tp_rank):
    """The boundary count - tp_rank * N taken in 64 bits, clamped to [0, N]."""
    n, k, e, h = 300, 4, 16, 64
    ids, w, _, x, y = _rand_case(1, n, k, e, h, "garbage")
    _full_check(ids, w, real, e, x, y, ("bf16", "mxfp4"), tp_rank)


CASES = {
    # name: (seed, n, k, e, h, kind)
    "k1": (2, 500, 1, 8, 32, "uniform"),
    "k_equals_e": (3, 200, 8, 8, 64, "distinct"),
    "duplicates": (4, 333, 6, 5, 32, "uniform"),
    "garbage_ids": (5, 257, 3, 7, 96, "garbage"),
    "one_expert": (6, 1500, 4, 64, 32, "one_expert"),
    "zero_token_experts": (7, 2000, 4, 256, 64, "half_empty"),
    "e1": (8, 100, 2, 1, 32, "uniform"),
    "e1024": (9, 3000, 8, 1024, 32, "distinct"),
    "k64": (10, 90, 64, 128, 32, "distinct"),
    "k100": (11, 40, 100, 300, 32, "distinct"),
    "ragged_chunks": (12, 3 * 4096 // 4 + 77, 4, 32, 32, "uniform"),
    "many_chunks_skewed": (13, 40000, 8, 256, 32, "one_expert"),
    "many_chunks": (14, 70000, 8, 256, 32, "distinct"),
    "h8_bf16_only": (15, 64, 2, 4, 8, "uniform"),
    "h_large": (16, 20, 2, 4, 16384, "uniform"),
    "h_ragged_vectors": (17, 30, 3, 6, 32 * 37, "uniform"),
    "k1024_e1024": (18, 6, 1024, 1024, 32, "distinct"),
    # every register-resident slot count (k <= 8) and the first slot-list k
    "k3_h96": (19, 311, 3, 9, 96, "distinct"),
    "k5": (20, 301, 5, 12, 160, "distinct"),
    "k7": (21, 299, 7, 13, 224, "uniform"),
    "k9": (22, 205, 9, 40, 64, "distinct"),
    "k16_garbage": (23, 190, 16, 33, 96, "garbage"),
    "h24_bf16_only": (24, 77, 4, 6, 24, "uniform"),
    "h32_one_block": (25, 150, 2, 8, 32, "uniform"),
    # around the one-workgroup limit of the index stage (2048 slots) and two chunks
    "s2048_one_workgroup": (26, 256, 8, 256, 32, "distinct"),
    "s2049_two_chunks": (27, 2049, 1, 16, 32, "uniform"),
    "s4097": (28, 4097, 1, 300, 32, "uniform"),
    # few rows: each row is cut across several workgroups (ragged last part; slot-list top_k)
    "split_rows_ragged": (29, 100, 3, 20, 8000, "uniform"),
    "split_rows_k10": (30, 50, 10, 64, 4096, "distinct"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_edge_case(name):
    seed, n, k, e, h, kind = CASES[name]
    ids, w, real, x, y = _rand_case(seed, n, k, e, h, kind)
    variants = ("bf16",) if h % 32 else ("bf16", "mxfp4")
    print(f"[parity] edge {name}: n={n} k={k} e={e} h={h}", flush=True)
    _full_check(ids, w, real, e, x, y, variants)


def test_empty_input():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    ids = np.zeros((0, 4), np.int32)
    res = run_path(mod, ids, 0, 16, x, y, np.zeros((0, 4), np.float32))
    assert u32(res["expert_start_indices"]).tolist() == [0] * 17
    assert i32(res["expert_ids"]).tolist() == [-1] * 16
    assert u32(res["expert_usage_stats"]).tolist() == [0, 0]


def test_mxfp4_special_blocks():
    """Zero / negative-zero / subnormal / largest-finite / tie blocks, bit-exact."""
    g = np.random.default_rng(21)
    h = 32 * 64
    rows = []
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[((allb >> 7) & 0xFF) != 0xFF]
    rows.append(np.zeros(h, np.uint16))
    rows.append(np.full(h, 0x8000, np.uint16))
    rows.append(g.integers(0, 0x80, size=h).astype(np.uint16))                # subnormals
    rows.append((g.integers(0, 0x80, size=h) | 0x8000).astype(np.uint16))
    rows.append(np.full(h, 0x7F7F, np.uint16))                                 # max finite
    rows.append(g.choice(finite, size=h).astype(np.uint16))                    # every exponent
    ties = oracle.f32_to_bf16_rne(np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.0, 1.0, 0.5,
                                            -0.25, -2.5, -5.0, 0.0] * 2, np.float32))
    rows.append(np.tile(ties, h // 32))
    for s in range(6):  # mixed-magnitude blocks with one large outlier each
        f = g.standard_normal(h).astype(np.float32)
        f[::32] *= 10.0 ** (s * 6 - 15)
        rows.append(oracle.f32_to_bf16_rne(f))
    xb = np.stack(rows)
    n = xb.shape[0]
    x = bf16_from_bits(xb, DEV)
    ids = np.stack([np.arange(3) + t for t in range(n)]).astype(np.int32) % 5
    res = run_path(mod, ids, n, 5, x, None, np.ones((n, 3), np.float32), ("mxfp4",))
    ref = oracle.create_indices(ids, 5)
    wq, ws = oracle.dispatch_mxfp4(xb, ref["token_expert_order"], 3, ref["n_routed"])
    np.testing.assert_array_equal(res["scales"].cpu().numpy(), ws)
    np.testing.assert_array_equal(res["q"].cpu().numpy(), wq)


def test_combine_no_fma_and_fixed_order():
    """Two cancelling products that a fused multiply-add would leave as 2^-30,
    and +1, +2^-30, -1 that only the fixed j order sums to +0."""
    h = 8
    w = np.array([[-(1 + 2.0 ** -23), 1 + 2.0 ** -23, 0.0], [1.0, 1.0, 1.0]], np.float32)
    yv = np.zeros((6, h), np.float32)
    yv[0] = yv[1] = 1 + 2.0 ** -7
    yv[3], yv[4], yv[5] = 1.0, 2.0 ** -30, -1.0
    y = bf16_from_bits(oracle.f32_to_bf16_rne(yv), DEV)
    restore = torch.from_numpy(np.array([0, 1, SENT, 3, 4, 5], np.uint32).view(np.int32)).to(DEV).view(torch.uint32)
    out = torch.empty((2, h), dtype=torch.bfloat16, device=DEV)
    mod.moe_combine(y, torch.from_numpy(w).to(DEV), restore, 3, out)
    got = u16(out)
    want = oracle.combine(u16(y), w, u32(restore), 3)
    assert np.all(want == 0)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("h", [32, 2048])
def test_positions_outside_buffer_are_skipped(h):
    """Output (dispatch) and input (combine) buffers shorter than the routed
    rows: positions past them are skipped.  h = 2048 also cuts rows across
    workgroups."""
    n, k, e = 50, 2, 4
    ids, w, real, x, y = _rand_case(30, n, k, e, h)
    ref = oracle.create_indices(ids, e)
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    limit = 37
    out = torch.zeros((limit, h), dtype=torch.bfloat16, device=DEV)
    mod.moe_dispatch(x, k, restore, out)
    want = oracle.dispatch(u16(x), ref["token_expert_order"], k, ref["n_routed"])[:limit]
    np.testing.assert_array_equal(u16(out), want)
    q = torch.zeros((limit, h // 2), dtype=torch.uint8, device=DEV)
    sc = torch.zeros((limit, h // 32), dtype=torch.uint8, device=DEV)
    mod.moe_dispatch_mxfp4(x, k, restore, q, sc)
    wq, wsc = oracle.dispatch_mxfp4(u16(x), ref["token_expert_order"], k, ref["n_routed"])
    np.testing.assert_array_equal(q.cpu().numpy(), wq[:limit])
    np.testing.assert_array_equal(sc.cpu().numpy(), wsc[:limit])
    comb = torch.empty((n, h), dtype=torch.bfloat16, device=DEV)
    mod.moe_combine(y[:limit], torch.from_numpy(w).to(DEV), restore, k, comb)
    r2 = ref["restore_token_order"].copy()
    r2[(r2 != SENT) & (r2 >= limit)] = SENT
    _check_combine(u16(comb), oracle.combine(u16(y[:limit]), w, r2, k))


def test_deterministic_under_skew():
    w = workloads.WORKLOADS[2]
    ids, wts, real = workloads.make_routing(w, 2)
    w_small = workloads.scaled(w, hidden=64)
    x, y = workloads.make_dense(w_small, 2, DEV)
    a = run_path(mod, ids, real, w.n_experts, x, y, wts)
    b = run_path(mod, ids, real, w.n_experts, x, y, wts)
    for key in ("token_expert_order", "restore_token_order", "expert_start_indices"):
        assert torch.equal(a[key].view(torch.int32), b[key].view(torch.int32))
    assert torch.equal(a["combine"].view(torch.int16), b["combine"].view(torch.int16))
    assert torch.equal(a["q"], b["q"])


@pytest.mark.parametrize("n, e", [(30000, 256), (40000, 1024)])   # count-table sums / lookback
def test_index_error_word_clear(n, e):
    ids, w, real, x, y = _rand_case(40, n, 8, e, 32, "distinct")
    res = run_path(mod, ids, real, e, x, y, w, ("bf16",))
    assert mod.index_workspace_error(res["workspace"]) == 0


# The multi-chunk index paths: up to 512 chunks whose count table (chunks x
# (E+1 rounded up to a multiple of 8) 16-bit counts) holds at most 2^17
# entries, every workgroup sums the table; larger inputs chain the chunks by
# lookback.  Both sides of each limit, with unrouted ids and the separate and
# one-call forms.
@pytest.mark.parametrize("s, e", [
    (496 * 2048, 256), (496 * 2048 + 1, 256),       # 496 * 264 entries; 497 rows are too many
    (512 * 2048, 8), (512 * 2048 + 1, 8),           # 512 chunks; 513 are too many
    (127 * 2048, 1024), (127 * 2048 + 1, 1024),     # 127 * 1032 entries; 128 rows are too many
    (65536, 1024), (65537, 1024),                   # the 1024-slot chunks of mid-size inputs, then 2048
])
def test_index_paths_around_the_table_limit(s, e):
    g = np.random.default_rng(s + e)
    ids = g.integers(-1, e + 1, size=(s, 1)).astype(np.int32)
    print(f"[parity] multi-chunk indices: S={s} E={e}", flush=True)
    d = torch.from_numpy(ids.reshape(-1)).to(DEV)
    idx = mod.alloc_indices(s, e, DEV, scales_offset=True)
    mod.moe_create_indices(d, e, idx["token_expert_order"], idx["expert_start_indices"], idx["restore_token_order"],
                           idx["expert_ids"], idx["expert_usage_stats"], idx["workspace"], idx["scales_offset"], 64)
    torch.cuda.synchronize()
    ref = oracle.create_indices(ids, e, scales_align=64)
    check_indices(idx, ref)
    np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])
    assert mod.index_workspace_error(idx["workspace"]) == 0
    # the one-call mask + indices, masking the last 1000 rows, in the same workspace
    real = s - 1000
    d = torch.from_numpy(ids.reshape(-1)).to(DEV)
    mod.moe_mask_create_indices(d.view(s, 1), torch.tensor([real], dtype=torch.int32, device=DEV), 0, e,
                                idx["token_expert_order"], idx["expert_start_indices"], idx["restore_token_order"],
                                idx["expert_ids"], idx["expert_usage_stats"], idx["workspace"])
    torch.cuda.synchronize()
    m = oracle.mask_routing_padding(ids, real, 0)
    np.testing.assert_array_equal(d.view(s, 1).cpu().numpy(), m)
    check_indices(idx, oracle.create_indices(m, e))


def test_argument_errors_on_device():
    idx = mod.alloc_indices(100, 8, DEV)
    ids = torch.zeros(100, dtype=torch.int32, device=DEV)
    small = idx["workspace"][:16]
    with pytest.raises(mod.MoeError) as e:
        mod.moe_create_indices(ids, 8, idx["token_expert_order"], idx["expert_start_indices"],
                               idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"], small)
    assert e.value.status == 2
    x = torch.zeros((10, 32), dtype=torch.bfloat16, device=DEV)
    q, s = mod.alloc_dispatch_mxfp4(100, 32, DEV)
    with pytest.raises(mod.MoeError) as e:
        mod.moe_dispatch_mxfp4(x, 10, idx["restore_token_order"], q, s, flags=4)
    assert e.value.status == 1


# index paths: count table (8192 slots), one workgroup (2048), lookback (1.12M slots, 547 chunks)
@pytest.mark.parametrize("fused, n, k, e", [(False, 2048, 4, 64), (True, 2048, 4, 64), (False, 256, 8, 64),
                                            (True, 256, 8, 64), (False, 140000, 8, 64), (True, 140000, 8, 64),
                                            (False, 4096, 2, 8), (True, 8192, 2, 8)])   # few-expert pass
def test_graph_replay_with_device_count(fused, n, k, e):
    """Capture mask+indices+dispatch+combine once (mask and indices as two
    calls, or as the one-call entry point); change only the device-side count
    between replays (with eager work in between) and check each replay.  On
    the large input, MXFP4 rows are checked for the first 4096 positions."""
    h = 64
    ids0, w, _, x, y = _rand_case(50, n, k, e, h, "distinct")
    d_ids = torch.from_numpy(ids0).to(DEV)
    d_src = d_ids.clone()
    cnt = torch.tensor([n], dtype=torch.int32, device=DEV)
    d_w = torch.from_numpy(w).to(DEV)
    idx = mod.alloc_indices(n * k, e, DEV)
    disp = mod.alloc_dispatch(n * k, h, DEV)
    q, sc = mod.alloc_dispatch_mxfp4(n * k, h, DEV)
    comb = torch.empty((n, h), dtype=torch.bfloat16, device=DEV)

    def step():
        if fused:
            mod.moe_mask_create_indices(d_ids, cnt, 0, e, idx["token_expert_order"], idx["expert_start_indices"],
                                        idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"],
                                        idx["workspace"])
        else:
            mod.moe_mask_padding(d_ids, cnt, 0)
            mod.moe_create_indices(d_ids, e, idx["token_expert_order"], idx["expert_start_indices"],
                                   idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"],
                                   idx["workspace"])
        mod.moe_dispatch(x, k, idx["restore_token_order"], disp)
        mod.moe_dispatch_mxfp4(x, k, idx["restore_token_order"], q, sc)
        mod.moe_combine(y, d_w, idx["restore_token_order"], k, comb)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
        d_ids.copy_(d_src)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for real in (n * 3 // 4, 7, n, 0, n - 49):
        d_ids.copy_(d_src)  # the mask works in place; restore the unmasked map eagerly
        cnt.fill_(real)
        torch.cuda.synchronize()
        _ = (x.float() * 2).sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        m, ref = _oracle_front(ids0, real, e)
        np.testing.assert_array_equal(i32(d_ids), m)
        res = dict(idx)
        check_indices(res, ref)
        v = ref["n_routed"]
        np.testing.assert_array_equal(u16(disp[:v]), oracle.dispatch(u16(x), ref["token_expert_order"], k, v))
        vq = min(v, 4096)
        wq, wsc = oracle.dispatch_mxfp4(u16(x), ref["token_expert_order"][:vq], k, vq)
        np.testing.assert_array_equal(q[:vq].cpu().numpy(), wq)
        np.testing.assert_array_equal(sc[:vq].cpu().numpy(), wsc)
        _check_combine(u16(comb), oracle.combine(u16(y), w, ref["restore_token_order"], k))
        assert mod.index_workspace_error(idx["workspace"]) == 0, real


@pytest.mark.parametrize("S, E", [((1 << 31) + 4099, 1024), (0xFFFFFFFE, 256)])
def test_indices_beyond_int32_slots(S, E):
    """Past the int32 range (2^31 + 4099 slots, ragged last chunk, E = 1024)
    and at the largest slot count the sentinel allows (2^32 - 2, positions up
    to 2^32 - 3): every property that defines the outputs, checked on the GPU
    in pieces."""
    print(f"[parity] create_indices at S={S} E={E}", flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(20261203)
    ids = torch.randint(-2, E + 6, (S,), generator=gen, device=DEV, dtype=torch.int32)
    idx = mod.alloc_indices(S, E, DEV)
    mod.moe_create_indices(ids, E, idx["token_expert_order"], idx["expert_start_indices"],
                           idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"],
                           idx["workspace"])
    torch.cuda.synchronize()
    assert mod.index_workspace_error(idx["workspace"]) == 0

    def as_i64(t):
        return t.view(torch.int32).to(torch.int64) & 0xFFFFFFFF

    routed = (ids >= 0) & (ids < E)
    counts = torch.zeros(E, dtype=torch.int64, device=DEV)
    step = 1 << 28
    for a in range(0, S, step):
        sl = ids[a:a + step]
        r = routed[a:a + step]
        counts += torch.bincount(sl[r].to(torch.int64), minlength=E)
    v = int(counts.sum().item())
    active = torch.nonzero(counts > 0).flatten()
    na = active.numel()
    esi = as_i64(idx["expert_start_indices"])
    assert int(esi[0]) == 0 and int(esi[na]) == v and bool((esi[na:] == v).all())
    assert torch.equal(esi[1:na + 1] - esi[:na], counts[active])
    assert torch.equal(idx["expert_ids"][:na].to(torch.int64), active)
    assert bool((idx["expert_ids"][na:] == -1).all())
    st = as_i64(idx["expert_usage_stats"])
    assert int(st[0]) == int(counts.max()) and int(st[1]) == na
    teo, res = idx["token_expert_order"], idx["restore_token_order"]
    prev_key = prev_slot = None
    for a in range(0, v, step):
        b = min(v, a + step)
        t = as_i64(teo[a:b])
        assert bool((t < S).all())
        k = ids[t].to(torch.int64)
        assert bool(((k >= 0) & (k < E)).all())
        if prev_key is not None:
            k = torch.cat([prev_key, k])
            t = torch.cat([prev_slot, t])
        dk = k[1:] - k[:-1]
        assert bool((dk >= 0).all())
        assert bool(((t[1:] - t[:-1]) > 0)[dk == 0].all())  # stable within an expert
        prev_key, prev_slot = k[-1:], t[-1:]
        pos = as_i64(res.view(torch.int32)[as_i64(teo[a:b])])
        assert torch.equal(pos, torch.arange(a, b, device=DEV))
    assert bool((as_i64(teo[v:]) == 0xFFFFFFFF).all())
    n_unrouted = 0
    for a in range(0, S, step):
        r = routed[a:a + step]
        rr = as_i64(res[a:a + step])
        assert bool((rr[~r] == 0xFFFFFFFF).all()) and bool((rr[r] < v).all())
        n_unrouted += int((~r).sum())
    assert n_unrouted == S - v


def test_dispatch_rows_beyond_one_item_grid():
    """More (token, part) items than a one-workgroup-per-item bf16 grid takes
    (2^25 + 37 rows of 8 elements, top_k = 1): the workgroups loop over
    tokens.  Every routed row against the oracle."""
    n, k, h, e = (1 << 25) + 37, 1, 8, 64
    print(f"[parity] dispatch bf16 with n={n} k={k} h={h}", flush=True)
    g = np.random.default_rng(4242)
    ids = g.integers(-1, e, size=(n, k), dtype=np.int32)
    ref = oracle.create_indices(ids, e)
    v = ref["n_routed"]
    xb = g.integers(0, 1 << 16, size=(n, h), dtype=np.uint16)
    x = bf16_from_bits(xb, DEV)
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    out = torch.zeros((n * k, h), dtype=torch.bfloat16, device=DEV)
    mod.moe_dispatch(x, k, restore, out)
    np.testing.assert_array_equal(u16(out[:v]), oracle.dispatch(xb, ref["token_expert_order"], k, v))


@pytest.mark.parametrize("n, k, h", [(1500, 12, 2048), (400, 9, 2048), (6000, 8, 1024)])
def test_dispatch_store_regimes(n, k, h):
    """Outputs on both sides of the store-policy bounds of bf16 dispatch:
    under 64 MiB (non-temporal stores, eager x loads) and 64-256 MiB (plain
    stores, x loaded for routed tokens only), through the looping kernel
    (k > 8) and the loop-free one (k = 8).  Every routed row against the
    oracle, with a quarter of the rows unrouted."""
    e = 64
    print(f"[parity] dispatch regimes n={n} k={k} h={h} out={n * k * h * 2 / 2**20:.0f} MiB", flush=True)
    g = np.random.default_rng(n + k)
    ids = g.integers(0, e, size=(n, k)).astype(np.int32)
    ids[g.random(n) < 0.25] = -1
    ref = oracle.create_indices(ids, e)
    v = ref["n_routed"]
    xb = oracle.f32_to_bf16_rne(g.standard_normal((n, h)).astype(np.float32))
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    out = torch.zeros((n * k, h), dtype=torch.bfloat16, device=DEV)
    mod.moe_dispatch(bf16_from_bits(xb, DEV), k, restore, out)
    np.testing.assert_array_equal(u16(out[:v]), oracle.dispatch(xb, ref["token_expert_order"], k, v))


# MXFP4 output sizes (payload and scales, 17 bytes per block) on each side of
# the eager-load window [64, 256) MiB, k <= 8 (eager and lazy forms) and
# k > 8: sampled routed rows against the oracle, a quarter of tokens unrouted.
@pytest.mark.parametrize("n, k, h", [(1500, 8, 7168), (2600, 8, 7168), (9000, 8, 7168), (600, 12, 7168)])
def test_dispatch_mxfp4_load_regimes(n, k, h):
    e = 64
    out_mib = n * k * (h // 32) * 17 / 2 ** 20
    print(f"[parity] MXFP4 regimes n={n} k={k} h={h} out={out_mib:.0f} MiB", flush=True)
    g = np.random.default_rng(n + k + h)
    ids = g.integers(0, e, size=(n, k)).astype(np.int32)
    ids[g.random(n) < 0.25] = -1
    ref = oracle.create_indices(ids, e)
    v = ref["n_routed"]
    xb = oracle.f32_to_bf16_rne(g.standard_normal((n, h)).astype(np.float32))
    restore = torch.from_numpy(ref["restore_token_order"].view(np.int32)).to(DEV).view(torch.uint32)
    q, sc = mod.alloc_dispatch_mxfp4(n * k, h, DEV)
    mod.moe_dispatch_mxfp4(bf16_from_bits(xb, DEV), k, restore, q, sc)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(min(v, 64)), g.integers(0, v, size=192), [v - 1]]))
    teo = ref["token_expert_order"]
    wq, wsc = oracle.dispatch_mxfp4(xb, teo[rows], k, rows.size)
    np.testing.assert_array_equal(q[rows].cpu().numpy(), wq)
    np.testing.assert_array_equal(sc[rows].cpu().numpy(), wsc)


def test_workspace_reuse_across_shapes():
    """One zero-filled workspace serves calls of different sizes, expert
    counts and id widths in any order: nothing an earlier call left in it is
    taken as this call's (small calls first, then a larger footprint)."""
    shapes = [(40000, 8, 256), (10000, 8, 64), (40000, 8, 256), (300, 4, 16), (70000, 8, 1024),
              (9000, 8, 256), (40000, 8, 256), (513, 8, 8), (70000, 8, 1024), (20000, 8, 1000),
              (60000, 8, 3), (4097, 1, 1024), (70000, 8, 1024)]
    g = np.random.default_rng(77)
    shapes += [shapes[j] for j in g.permutation(len(shapes))]
    ws_bytes = max(mod.moe_create_indices_workspace_bytes(n * k, e) for n, k, e in shapes)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    for i, (n, k, e) in enumerate(shapes):
        kind = "distinct" if k <= e and n * e <= 10 ** 7 else "uniform"
        ids, _, _, _, _ = _rand_case(900 + i, n, k, e, 8, kind)
        d_ids = torch.from_numpy(ids).to(DEV)
        if i % 3 == 2:
            d_ids = d_ids.to(torch.int64)
        idx = mod.alloc_indices(n * k, e, DEV)
        mod.moe_create_indices(d_ids, e, idx["token_expert_order"], idx["expert_start_indices"],
                               idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"], ws)
        torch.cuda.synchronize()
        check_indices(idx, oracle.create_indices(ids, e))
        assert mod.index_workspace_error(ws) == 0, (i, n, k, e)


def test_concurrent_streams_with_separate_workspaces():
    """Two paths of different shapes run at once on two streams, each with its
    own workspace and outputs; both match the oracle (the library keeps no
    state outside the buffers it is given)."""
    cases = [(41, 30000, 8, 256, 64, "distinct"), (42, 20000, 4, 64, 96, "uniform")]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for (seed, n, k, e, h, kind), st in zip(cases, streams):
        ids, w, real, x, y = _rand_case(seed, n, k, e, h, kind, real=n - 17)
        runs.append((ids, w, real, e, x, y, st))
    torch.cuda.synchronize()
    results = []
    for _ in range(3):
        outs = []
        for ids, w, real, e, x, y, st in runs:
            with torch.cuda.stream(st):
                outs.append(_launch_path(ids, w, real, e, x, y, st))
        torch.cuda.synchronize()
        results = outs
        for (ids, w, real, e, x, y, st), res in zip(runs, outs):
            m, ref = _oracle_front(ids, real, e)
            np.testing.assert_array_equal(i32(res["ids"]), m)
            check_indices(res, ref)
            n, k = ids.shape
            v = ref["n_routed"]
            np.testing.assert_array_equal(u16(res["dispatch"][:v]),
                                          oracle.dispatch(u16(x), ref["token_expert_order"], k, v))
            wq, wsc = oracle.dispatch_mxfp4(u16(x), ref["token_expert_order"], k, v)
            np.testing.assert_array_equal(res["q"][:v].cpu().numpy(), wq)
            np.testing.assert_array_equal(res["scales"][:v].cpu().numpy(), wsc)
            _check_combine(u16(res["combine"]), oracle.combine(u16(y), w, ref["restore_token_order"], k))
            assert mod.index_workspace_error(res["workspace"]) == 0
    assert len(results) == 2


def _launch_path(ids, w, real, e, x, y, st):
    """Every stage enqueued on the current stream `st`, with no host sync."""
    n, k = ids.shape
    h = x.shape[1]
    s = n * k
    with torch.cuda.stream(st):
        d_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV, non_blocking=False)
        d_cnt = torch.tensor([real], dtype=torch.int32, device=DEV)
        d_w = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(DEV)
        idx = mod.alloc_indices(s, e, DEV)
        mod.moe_mask_padding(d_ids, d_cnt, 0)
        mod.moe_create_indices(d_ids, e, idx["token_expert_order"], idx["expert_start_indices"],
                               idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"],
                               idx["workspace"])
        out = mod.alloc_dispatch(s, h, DEV)
        mod.moe_dispatch(x, k, idx["restore_token_order"], out)
        q, sc = mod.alloc_dispatch_mxfp4(s, h, DEV)
        mod.moe_dispatch_mxfp4(x, k, idx["restore_token_order"], q, sc)
        o = torch.empty((n, h), dtype=torch.bfloat16, device=DEV)
        mod.moe_combine(y, d_w, idx["restore_token_order"], k, o)
    return dict(ids=d_ids, dispatch=out, q=q, scales=sc, combine=o, **idx)


# Count-table rows hold E+1 counts padded to a multiple of 8: each side of
# the padding steps, with 1024-slot chunks (9000 slots) and 2048-slot chunks
# (70000 slots), unrouted ids included.
@pytest.mark.parametrize("e", [1, 6, 7, 8, 15, 16, 17, 255, 1023, 1024])
@pytest.mark.parametrize("s", [9000, 70000])
def test_index_count_table_row_padding(e, s):
    g = np.random.default_rng(e * 7 + s)
    ids = g.integers(-1, e + 1, size=(s, 1)).astype(np.int32)
    print(f"[parity] count-table rows: S={s} E={e}", flush=True)
    d = torch.from_numpy(ids.reshape(-1)).to(DEV)
    idx = mod.alloc_indices(s, e, DEV, scales_offset=True)
    mod.moe_create_indices(d, e, idx["token_expert_order"], idx["expert_start_indices"], idx["restore_token_order"],
                           idx["expert_ids"], idx["expert_usage_stats"], idx["workspace"], idx["scales_offset"], 32)
    torch.cuda.synchronize()
    ref = oracle.create_indices(ids, e, scales_align=32)
    check_indices(idx, ref)
    np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])


# The scan of the bucket totals gives each lane ceil((E+1)/T) consecutive
# buckets, with the reads unrolled to a compile-time bound that depends on
# the path: E+1 on each side of 64, 128, 256 and 320 buckets (320 is the
# most one wave scans alone), and 1024 experts, through the one-workgroup
# pass at 64, 128, 256 and 1024 lanes (100, 200, 400 and 2000 slots) and the
# count-table path at both chunk sizes.  Every index output and the aligned
# offsets, bit-exact.
@pytest.mark.parametrize("e", [63, 64, 127, 128, 255, 256, 319, 320, 1024])
@pytest.mark.parametrize("s", [100, 200, 400, 2000, 9000, 70000])
def test_index_scan_buckets_per_lane(e, s):
    g = np.random.default_rng(e * 11 + s)
    ids = g.integers(-1, e + 1, size=(s, 1)).astype(np.int32)
    print(f"[parity] bucket scan: S={s} E={e}", flush=True)
    d = torch.from_numpy(ids.reshape(-1)).to(DEV)
    idx = mod.alloc_indices(s, e, DEV, scales_offset=True)
    mod.moe_create_indices(d, e, idx["token_expert_order"], idx["expert_start_indices"], idx["restore_token_order"],
                           idx["expert_ids"], idx["expert_usage_stats"], idx["workspace"], idx["scales_offset"], 16)
    torch.cuda.synchronize()
    ref = oracle.create_indices(ids, e, scales_align=16)
    check_indices(idx, ref)
    np.testing.assert_array_equal(u32(idx["scales_offset"]), ref["scales_offset"])


def test_workspace_not_zero_filled_sets_error_word():
    """Misuse, forced from the host: the ticket word of the workspace is not
    zero, so the first chunks are never handed out and later chunks wait for
    them.  The waits are bounded; the call must finish, keep every write
    inside the buffers (canaries after the outputs and the workspace stay
    intact) and set the sticky error word.  The outputs are unspecified."""
    n, k, e = 600000, 2, 16                     # 1.2M slots, 586 chunks: the lookback path
    s = n * k
    ids = np.random.default_rng(5).integers(0, e, size=(n, k)).astype(np.int32)
    d_ids = torch.from_numpy(ids).to(DEV)
    pad = 4096
    canary = 0x5A5A5A5A
    teo = torch.full((s + pad,), canary, dtype=torch.int64, device=DEV).to(torch.int32).view(torch.uint32)
    rest = torch.full((s + pad,), canary, dtype=torch.int64, device=DEV).to(torch.int32).view(torch.uint32)
    esi = torch.empty(e + 1, dtype=torch.uint32, device=DEV)
    eid = torch.empty(e, dtype=torch.int32, device=DEV)
    stats = torch.empty(2, dtype=torch.uint32, device=DEV)
    ws_bytes = mod.moe_create_indices_workspace_bytes(s, e)
    ws = torch.zeros(ws_bytes + 65536, dtype=torch.uint8, device=DEV)
    ws[ws_bytes:] = 0xA5
    ws[:8].view(torch.int32)[1] = 3             # ticket word
    mod.moe_create_indices(d_ids, e, teo[:s], esi, rest[:s], eid, stats, ws[:ws_bytes])
    torch.cuda.synchronize()
    assert mod.index_workspace_error(ws) != 0
    assert bool((teo[s:].view(torch.int32) == canary).all()) and bool((rest[s:].view(torch.int32) == canary).all())
    assert bool((ws[ws_bytes:] == 0xA5).all())


_ARCH_PROBE = r"""
import sys, torch
sys.path.insert(0, {root!r})
import expert_grouping_dispatch_amd as mod
ids = torch.arange(32, dtype=torch.int32, device="cuda").reshape(8, 4) % 5
before = ids.clone()
cnt = torch.tensor([3], dtype=torch.int32, device="cuda")
codes = []
try:
    mod.moe_mask_padding(ids, cnt, 0)
    codes.append(0)
except mod.MoeError as exc:
    codes.append(exc.status)
idx = mod.alloc_indices(32, 5, "cuda")
try:
    mod.moe_create_indices(ids, 5, idx["token_expert_order"], idx["expert_start_indices"],
                           idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"], idx["workspace"])
    codes.append(0)
except mod.MoeError as exc:
    codes.append(exc.status)
torch.cuda.synchronize()
print("codes", codes, "unchanged", bool(torch.equal(ids, before)))
"""


@pytest.mark.parametrize("arch, want", [("gfx942", "codes [3, 3] unchanged True"),
                                        ("gfx950:sramecc+:xnack-", "codes [0, 0] unchanged False")])
def test_device_architecture_check(arch, want):
    """A device that is not gfx950 is rejected before anything is launched;
    the architecture name is stood in for through MOE_ROUTE_ASSUME_ARCH, in a
    fresh process (the check is made once per device and process)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, MOE_ROUTE_ASSUME_ARCH=arch)
    r = subprocess.run([sys.executable, "-c", _ARCH_PROBE.format(root=root)], env=env, capture_output=True,
                       text=True, timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    assert want in r.stdout, r.stdout


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(seed):
    """Seeded random shapes through the whole path, element by element against
    the oracle: row counts across the one-workgroup / multi-chunk boundary and
    the split-row range, every top_k path, expert counts, hidden sizes (some
    not a multiple of 32: bf16 only), counts outside [0, N] and garbage ids."""
    g = np.random.default_rng(9000 + seed)
    k = int(g.choice([1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16, 33]))
    n = int(g.integers(1, max(2, 24000 // k)))
    e = int(g.choice([1, 2, 7, 8, 64, 255, 256, 300, 1024]))
    h = int(g.choice([8, 24, 32, 96, 256, 1000, 2048, 4096]))
    kind = str(g.choice(["uniform", "garbage", "distinct" if k <= e else "uniform", "half_empty"]))
    real = int(g.choice([n, n - 1, 0, n // 2, n + 3, -5]))
    ids, w, _, x, y = _rand_case(9000 + seed, n, k, e, h, kind)
    variants = ("bf16",) if h % 32 else ("bf16", "mxfp4")
    print(f"[parity] random seed={seed}: n={n} k={k} e={e} h={h} kind={kind} real={real}", flush=True)
    _full_check(ids, w, real, e, x, y, variants)
