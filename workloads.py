"""Seeded synthetic inputs for the MoE token-routing path.

This module only draws random inputs; it holds none of the routing
arithmetic (no masking, counting, sorting, quantisation or weighted sums).
Both the CPU oracle tests and the GPU path are fed from here, so the two
sides always see identical bytes.

Shapes follow the tensors of the pages:
  * ``topk_ids`` / ``routing_map``  int32 [N, top_k]  (token-major routing map,
    "core.transformer.moe.inference_routing_mask_kernel", mask_routing_padding
    parameters; "moe_create_indices", Args: topk_ids)
  * ``router_weights`` fp32 [N, top_k]   ("Struct_ep_combine_wait", Args)
  * ``input_tokens`` bf16 [N, H]         ("Struct_ep_dispatch_async_mxfp4", Args)
  * expert outputs ``y`` bf16 [N*top_k, H], rows in expert-grouped order.

Routing draws (ids, weights, padding garbage, outlier rows, expert sets) use
NumPy PCG64 seeded by ``SeedSequence(SEED, spawn_key=(config, stream))``.
Dense activations use a torch generator on the target device (Philox on the
GPU, so the 7.5 GB expert-output tensor of the largest workload is drawn in
HBM in milliseconds); tests read back whatever rows they check.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED = 20261203

# stream ids of the seed sequence
S_IDS, S_LOGITS, S_X, S_Y, S_GARBAGE, S_OUTLIER, S_EXPERTSET = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_rows: int          # N: rows of the (possibly padded) routing map
    real_tokens: int     # R: real_token_count
    hidden: int          # H
    n_experts: int       # E
    top_k: int           # k
    routing: str         # "uniform" | "zipf" | "hotcold"
    dispatch: tuple      # subset of ("bf16", "mxfp4")
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    zipf_s: float = 1.2
    n_hot: int = 26
    n_cold: int = 3

    @property
    def n_slots(self) -> int:
        return self.n_rows * self.top_k


WORKLOADS = [
    Workload("tiny", 64, 64, 256, 8, 2, "uniform", ("bf16",)),
    Workload("mixtral_prefill", 8192, 7000, 4096, 8, 2, "uniform", ("bf16",)),
    Workload("deepseek_v3_prefill", 4096, 4096, 7168, 256, 8, "zipf", ("mxfp4",),
             outlier_frac=0.01, outlier_scale=50.0),
    Workload("decode", 256, 97, 7168, 256, 8, "uniform", ("bf16", "mxfp4")),
    Workload("large_prefill_stress", 65536, 61440, 7168, 256, 8, "hotcold",
             ("bf16", "mxfp4")),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def rng(cfg: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=(cfg, stream))))


def torch_seed(cfg: int, stream: int) -> int:
    st = np.random.SeedSequence(SEED, spawn_key=(cfg, stream)).generate_state(1, dtype=np.uint64)[0]
    return int(st) & ((1 << 63) - 1)


def _distinct_uniform(g: np.random.Generator, rows: int, n_experts: int, k: int) -> np.ndarray:
    """k distinct experts per row, uniform without replacement."""
    return np.argsort(g.random((rows, n_experts)), axis=1)[:, :k]


def _distinct_zipf(g: np.random.Generator, perm: np.ndarray, rows: int, n_experts: int,
                   k: int, s: float) -> np.ndarray:
    """k distinct experts per row drawn without replacement with popularity
    p(rank r) proportional to r^-s (Gumbel top-k); rank r is expert perm[r-1]."""
    logp = -s * np.log(np.arange(1, n_experts + 1, dtype=np.float64))
    keys = logp[None, :] + g.gumbel(size=(rows, n_experts))
    top = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return perm[top]


def _hotcold(g: np.random.Generator, perm: np.ndarray, rows: int, k: int, n_hot: int,
             n_cold: int) -> np.ndarray:
    """Half of each row's k slots on distinct hot experts, half on distinct
    'other' experts, shuffled; cold experts are never chosen."""
    assert k % 2 == 0
    hot = perm[:n_hot]
    other = perm[n_hot + n_cold:]
    h = hot[np.argsort(g.random((rows, hot.size)), axis=1)[:, : k // 2]]
    o = other[np.argsort(g.random((rows, other.size)), axis=1)[:, : k // 2]]
    both = np.concatenate([h, o], axis=1)
    order = np.argsort(g.random((rows, k)), axis=1)
    return np.take_along_axis(both, order, axis=1)


def make_routing(w: Workload, cfg: int = 0):
    """Return (topk_ids int32 [N,k], router_weights fp32 [N,k], real_token_count int).

    Rows at or past real_token_count hold garbage expert ids (uniform in
    [0, E), repeats allowed), as padded rows of a captured graph do."""
    N, R, E, k = w.n_rows, w.real_tokens, w.n_experts, w.top_k
    ids = np.empty((N, k), dtype=np.int64)
    g = rng(cfg, S_IDS)
    if w.routing == "uniform":
        ids[:R] = _distinct_uniform(g, R, E, k)
    elif w.routing == "zipf":
        perm = rng(cfg, S_EXPERTSET).permutation(E)
        ids[:R] = _distinct_zipf(g, perm, R, E, k, w.zipf_s)
    elif w.routing == "hotcold":
        perm = rng(cfg, S_EXPERTSET).permutation(E)
        ids[:R] = _hotcold(g, perm, R, k, w.n_hot, w.n_cold)
    else:
        raise ValueError(w.routing)
    if N > R:
        ids[R:] = rng(cfg, S_GARBAGE).integers(0, E, size=(N - R, k))
    logits = rng(cfg, S_LOGITS).standard_normal((N, k))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    weights = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids.astype(np.int32), weights, R


def outlier_rows(w: Workload, cfg: int = 0) -> np.ndarray:
    n = int(round(w.outlier_frac * w.n_rows))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng(cfg, S_OUTLIER).choice(w.n_rows, size=n, replace=False))


def make_dense(w: Workload, cfg: int, device, y_rows: Optional[int] = None, chunk_elems: int = 1 << 26):
    """Return (x bf16 [N,H], y bf16 [y_rows,H]) as torch tensors on ``device``.

    Values are N(0,1) drawn in fp32 and rounded to bf16 by torch; the
    configured outlier rows of x are scaled in fp32 before rounding."""
    import torch

    def randn_bf16(rows, cols, stream):
        gen = torch.Generator(device=device)
        gen.manual_seed(torch_seed(cfg, stream))
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
        step = max(1, chunk_elems // max(cols, 1))
        for r0 in range(0, rows, step):
            r1 = min(rows, r0 + step)
            f = torch.randn((r1 - r0, cols), generator=gen, device=device, dtype=torch.float32)
            if stream == S_X and w.outlier_frac > 0:
                sel = outlier_rows(w, cfg)
                sel = sel[(sel >= r0) & (sel < r1)] - r0
                if sel.size:
                    f[torch.as_tensor(sel, device=device)] *= w.outlier_scale
            out[r0:r1] = f.to(torch.bfloat16)
        return out

    x = randn_bf16(w.n_rows, w.hidden, S_X)
    y = randn_bf16(w.n_slots if y_rows is None else y_rows, w.hidden, S_Y)
    return x, y


def scaled(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some sizes replaced (used for small parity cases)."""
    return dataclasses.replace(w, **kw)
