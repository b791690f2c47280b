"""The seeded synthetic inputs follow their recipe (CPU only).

Every parity test and the bench draw their inputs from ``workloads``; these
checks pin the recipe itself: the shapes of the five workloads, distinct
experts per real token, the hot / cold split of the stress routing, the Zipf
skew, garbage ids in padding rows, softmax router weights, the outlier rows
of the DeepSeek-shaped activations, and that every draw is reproducible.
"""
import numpy as np
import pytest
import torch

import workloads

SHAPES = {  # name: (N, R, H, E, k)
    "tiny": (64, 64, 256, 8, 2),
    "mixtral_prefill": (8192, 7000, 4096, 8, 2),
    "deepseek_v3_prefill": (4096, 4096, 7168, 256, 8),
    "decode": (256, 97, 7168, 256, 8),
    "large_prefill_stress": (65536, 61440, 7168, 256, 8),
}


def _routing(name):
    cfg = [w.name for w in workloads.WORKLOADS].index(name)
    w = workloads.WORKLOADS[cfg]
    ids, wts, real = workloads.make_routing(w, cfg)
    return cfg, w, ids, wts, real


def test_workload_shapes():
    assert [w.name for w in workloads.WORKLOADS] == list(SHAPES)
    for w in workloads.WORKLOADS:
        assert (w.n_rows, w.real_tokens, w.hidden, w.n_experts, w.top_k) == SHAPES[w.name]


@pytest.mark.parametrize("name", list(SHAPES))
def test_real_rows_take_distinct_experts(name):
    _, w, ids, wts, real = _routing(name)
    assert ids.dtype == np.int32 and ids.shape == (w.n_rows, w.top_k) and real == w.real_tokens
    r = np.sort(ids[:real], axis=1)
    assert r.min() >= 0 and r.max() < w.n_experts
    assert (np.diff(r, axis=1) > 0).all()           # k distinct experts per real token


@pytest.mark.parametrize("name", [n for n, s in SHAPES.items() if s[0] > s[1]])
def test_padding_rows_hold_garbage_ids(name):
    _, w, ids, _, real = _routing(name)
    pad = ids[real:]
    assert pad.min() >= 0 and pad.max() < w.n_experts   # valid-looking ids: only the mask removes them
    repeats = (np.diff(np.sort(pad, axis=1), axis=1) == 0).any(axis=1)
    assert repeats.any()                                 # drawn with repeats, unlike real rows


@pytest.mark.parametrize("name", list(SHAPES))
def test_router_weights_are_a_softmax(name):
    _, w, _, wts, _ = _routing(name)
    assert wts.dtype == np.float32 and (wts > 0).all()
    np.testing.assert_allclose(wts.astype(np.float64).sum(axis=1), 1.0, rtol=0, atol=1e-6)


def test_stress_hot_and_cold_experts():
    cfg, w, ids, _, real = _routing("large_prefill_stress")
    perm = workloads.rng(cfg, workloads.S_EXPERTSET).permutation(w.n_experts)
    hot, cold = perm[:w.n_hot], perm[w.n_hot:w.n_hot + w.n_cold]
    r = ids[:real]
    on_hot = np.isin(r, hot).sum(axis=1)
    assert (on_hot == w.top_k // 2).all()              # every real token: 4 hot, 4 others
    assert not np.isin(r, cold).any()                  # cold experts never chosen
    counts = np.bincount(r.ravel(), minlength=w.n_experts)
    assert (counts > 0).sum() == w.n_experts - w.n_cold == 253
    assert counts[hot].sum() * 2 == r.size              # exactly half of the routed slots are hot
    # about 9452 slots per hot expert and 1083 per other one
    assert abs(counts[hot].mean() - 9452) < 5
    others = np.setdiff1d(np.arange(w.n_experts), np.concatenate([hot, cold]))
    assert abs(counts[others].mean() - 1083) < 5


def test_deepseek_zipf_skew():
    cfg, w, ids, _, real = _routing("deepseek_v3_prefill")
    perm = workloads.rng(cfg, workloads.S_EXPERTSET).permutation(w.n_experts)
    counts = np.bincount(ids[:real].ravel(), minlength=w.n_experts)
    assert (counts > 0).all()                          # all 256 experts active
    top = counts[perm[0]]                              # rank-1 expert
    assert top == counts.max() and 3000 < top <= real  # most tokens reach the top expert
    ranks = counts[perm]
    assert ranks[:8].mean() > 4 * ranks[-64:].mean()   # popularity falls with rank


def test_deepseek_outlier_rows():
    cfg = [w.name for w in workloads.WORKLOADS].index("deepseek_v3_prefill")
    w = workloads.WORKLOADS[cfg]
    rows = workloads.outlier_rows(w, cfg)
    assert rows.size == round(0.01 * w.n_rows) == 41 and np.unique(rows).size == 41
    assert workloads.outlier_rows(workloads.BY_NAME["decode"], 3).size == 0
    small = workloads.scaled(w, hidden=64)
    x, _ = workloads.make_dense(small, cfg, "cpu", y_rows=1)
    mag = x.float().abs().mean(dim=1).numpy()
    mask = np.zeros(w.n_rows, bool)
    mask[rows] = True
    assert mag[mask].min() > 10 * mag[~mask].max()     # scaled by 50 before the bf16 rounding


def test_draws_are_reproducible():
    for name in ("decode", "mixtral_prefill"):
        a = _routing(name)
        b = _routing(name)
        assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])
    w = workloads.scaled(workloads.BY_NAME["tiny"], hidden=32)
    x1, y1 = workloads.make_dense(w, 0, "cpu")
    x2, y2 = workloads.make_dense(w, 0, "cpu")
    assert torch.equal(x1, x2) and torch.equal(y1, y2)
    assert x1.dtype == torch.bfloat16 and y1.shape == (w.n_slots, 32)
