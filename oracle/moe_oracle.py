"""Plain CPU oracle of the MoE token-routing path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code with the HIP library
(``expert_grouping_dispatch_amd``) and imports nothing from it.

Each function writes out the plain definition of one step, in NumPy, with no
blocking, fusion or reordering beyond what the definition states.  Sources
(the web pages this method is described on):

  * mask       -- "core.transformer.moe.inference_routing_mask_kernel"
                  (module summary; API: mask_routing_padding and its
                  routing_map / real_token_count_tensor / tp_rank parameters)
  * indices    -- "moe_create_indices" (description; Args)
  * dispatch   -- "Struct_ep_dispatch_async_mxfp4" (execute description;
                  Parameters dispatch_dtype / dispatch_scale_dtype; Args
                  input_tokens / topk_ids)
  * combine    -- "Struct_ep_combine_wait" (execute description; Args
                  output_tokens / router_weights)

Readings taken where the pages are silent:
  * topk_ids is int32 [N, top_k], viewed flat as slots i = t*top_k + j; a
    slot is routed iff 0 <= id < n_experts (the mask's -1 and any garbage id
    are unrouted).
  * token_expert_order holds slot indices i (source row i // top_k), in a
    stable order: ascending expert id, then ascending slot index.
  * expert_ids / expert_start_indices are compacted over the experts that
    received at least one slot; unused tails hold -1 / the routed count V.
  * expert_usage_stats = [max slots on one expert, number of active experts].
  * scales_offset (optional): for active expert j, the sum over earlier
    active experts of their slot count rounded up to a multiple of
    scales_align; entries from the active count on hold the total.
  * unused entries of token_expert_order and restore_token_order hold
    0xFFFFFFFF.
  * MXFP4: blocks of 32 elements along the hidden dimension, E2M1 payload
    and one E8M0 scale byte per block.  Scale exponent = floor(log2 amax) - 2
    (2 = largest E2M1 exponent), clamped to [-127, 127]; an all-zero block
    gets exponent -127.  Element code = nearest E2M1 magnitude to
    |v| * 2**-exponent, ties to the even code, saturating at 6; the sign bit
    is kept (also on zero).  Element 2m in the low nibble of byte m.
    Non-finite inputs are outside the pinned domain (parity unpinned there).
    "Even-mode" scale: max |v| is first rounded to E2M1's one mantissa bit,
    halves up, so floor(log2) gains 1 when its mantissa fraction is >= 0.75.
    Packed rows: each slot's H/2 payload bytes followed by its H/32 scales.
  * combine epilogue: out = bf16(fl(fl(scale * acc) + residual)), residual
    optional, each operation rounded on its own.
  * combine: fp32, acc = +0, then for j = 0..top_k-1 in order and only for
    routed slots, acc = fl(acc + fl(w[t,j] * y[pos])) with every operation
    rounded on its own (no fused multiply-add); output = bf16 round to
    nearest even of acc.  Rows with no routed slot give +0.
"""
from __future__ import annotations

import numpy as np

SENT = 0xFFFFFFFF
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_EMAX = 2          # largest binary exponent of an E2M1 value (6 = 1.5 * 2**2)
MX_BLOCK = 32
E8M0_BIAS = 127


# --------------------------------------------------------------------------
# bf16 / fp32 bit helpers
# --------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# stage 1: mask padding rows
# --------------------------------------------------------------------------
def mask_routing_padding(routing_map: np.ndarray, real_token_count: int, tp_rank: int = 0) -> np.ndarray:
    """Return a copy of routing_map with -1 in every top-k slot of the padding rows.

    Local row r is global row r + tp_rank * N; it is padding when that global
    row is at or past real_token_count ("inference_routing_mask_kernel",
    mask_routing_padding: routing_map and tp_rank parameters).  Counts
    outside [0, N] simply mask nothing or everything."""
    ids = np.array(routing_map, copy=True)
    n = ids.shape[0]
    first = int(real_token_count) - int(tp_rank) * n
    first = min(max(first, 0), n)
    ids[first:, :] = -1
    return ids


# --------------------------------------------------------------------------
# stage 2: expert-grouped indices
# --------------------------------------------------------------------------
def create_indices(topk_ids: np.ndarray, n_experts: int, scales_align: int = None) -> dict:
    """Group routed slots by expert ("moe_create_indices", description and Args).

    Histogram of expert ids -> CSR starts over the active experts -> stable
    scatter of slot indices, with its inverse.  With scales_align, also the
    aligned scale offsets (Args: scales_offset_p)."""
    f = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    n_slots = f.size
    routed = (f >= 0) & (f < n_experts)

    counts = np.bincount(f[routed], minlength=n_experts).astype(np.int64)
    n_routed = int(counts.sum())
    active = np.flatnonzero(counts > 0)
    n_active = int(active.size)

    expert_ids = np.full(n_experts, -1, dtype=np.int32)
    expert_ids[:n_active] = active
    expert_start_indices = np.full(n_experts + 1, n_routed, dtype=np.uint32)
    expert_start_indices[0] = 0
    expert_start_indices[1:n_active + 1] = np.cumsum(counts[active])
    max_count = int(counts.max()) if n_routed > 0 else 0
    expert_usage_stats = np.array([max_count, n_active], dtype=np.uint32)

    # stable counting sort: key = expert id, unrouted slots after every expert
    key = np.where(routed, f, n_experts)
    order = np.argsort(key, kind="stable")
    token_expert_order = np.full(n_slots, SENT, dtype=np.uint32)
    token_expert_order[:n_routed] = order[:n_routed]
    restore_token_order = np.full(n_slots, SENT, dtype=np.uint32)
    restore_token_order[order[:n_routed]] = np.arange(n_routed, dtype=np.uint32)

    out = dict(token_expert_order=token_expert_order,
               expert_start_indices=expert_start_indices,
               restore_token_order=restore_token_order,
               expert_ids=expert_ids,
               expert_usage_stats=expert_usage_stats,
               n_routed=n_routed)
    if scales_align is not None:
        padded = -(-counts[active] // scales_align) * scales_align
        total = int(padded.sum())
        scales_offset = np.full(n_experts + 1, total, dtype=np.uint32)
        scales_offset[:n_active] = np.concatenate([[0], np.cumsum(padded)[:-1]]) if n_active else []
        out["scales_offset"] = scales_offset
    return out


# --------------------------------------------------------------------------
# stage 3a: dispatch, bf16
# --------------------------------------------------------------------------
def dispatch(input_tokens: np.ndarray, token_expert_order: np.ndarray, top_k: int, n_routed: int) -> np.ndarray:
    """Expert-contiguous copy of token rows: row p <- input_tokens[teo[p] // top_k].

    Rows [0, n_routed) only; rows past it are not part of the result."""
    src = token_expert_order[:n_routed].astype(np.int64) // top_k
    return np.asarray(input_tokens)[src]


# --------------------------------------------------------------------------
# stage 3b: dispatch, MXFP4
# --------------------------------------------------------------------------
def mxfp4_quantize(x_bits: np.ndarray, even: bool = False):
    """MXFP4 encoding of bf16 rows [T, H] -> (payload uint8 [T, H/2], scales uint8 [T, H/32]).

    ("Struct_ep_dispatch_async_mxfp4": FP4 quants with scales; block of 32,
    E8M0 scale and the rounding rule as stated in the module docstring.)
    Every value involved is exact in float64: bf16 inputs, scaling by a power
    of two, and distances to the E2M1 grid near any tie."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    t, h = x_bits.shape
    assert h % MX_BLOCK == 0
    nb = h // MX_BLOCK
    v = bf16_bits_to_f32(x_bits).astype(np.float64).reshape(t, nb, MX_BLOCK)

    amax = np.abs(v).max(axis=2)
    m, e = np.frexp(amax)                   # amax = m * 2**e with m in [0.5, 1)
    floor_log2 = e.astype(np.int64) - 1
    if even:                                # mantissa fraction 2m - 1 >= 0.75 rounds up a binade
        floor_log2 = floor_log2 + (m >= 0.875)
    se = np.where(amax > 0, np.clip(floor_log2 - E2M1_EMAX, -127, 127), -127)

    s = np.abs(v) * np.ldexp(1.0, -se)[:, :, None]
    d = np.abs(s[..., None] - E2M1_GRID)    # distance to each E2M1 magnitude
    dmin = d.min(axis=-1, keepdims=True)
    cand = d == dmin
    first = np.argmax(cand, axis=-1)        # lowest nearest code
    tie = cand.sum(axis=-1) > 1
    code = np.where(tie & (first % 2 == 1), first + 1, first)

    nib = code.astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 3)
    payload = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8).reshape(t, h // 2)
    scales = (se + E8M0_BIAS).astype(np.uint8)
    return payload, scales


def mxfp4_dequantize(payload: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode MXFP4 rows back to float64 (value = +-E2M1[code] * 2**(scale - 127))."""
    payload = np.asarray(payload, dtype=np.uint8)
    t, hb = payload.shape
    nib = np.empty((t, hb * 2), dtype=np.uint8)
    nib[:, 0::2] = payload & 0xF
    nib[:, 1::2] = payload >> 4
    mag = E2M1_GRID[nib & 7]
    sign = np.where(nib & 8, -1.0, 1.0)
    sc = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - E8M0_BIAS)
    return (sign * mag).reshape(t, -1, MX_BLOCK) * sc[:, :, None]


def dispatch_mxfp4(input_tokens: np.ndarray, token_expert_order: np.ndarray, top_k: int, n_routed: int,
                   rows_per_pass: int = 64, even: bool = False, packed: bool = False):
    """Row p of the result is the MXFP4 encoding of input_tokens[teo[p] // top_k].

    Returns (payload, scales), or with packed=True one array whose rows are
    payload followed by scales."""
    src = token_expert_order[:n_routed].astype(np.int64) // top_k
    h = input_tokens.shape[1]
    payload = np.empty((n_routed, h // 2), dtype=np.uint8)
    scales = np.empty((n_routed, h // MX_BLOCK), dtype=np.uint8)
    for p0 in range(0, n_routed, rows_per_pass):
        p1 = min(n_routed, p0 + rows_per_pass)
        payload[p0:p1], scales[p0:p1] = mxfp4_quantize(np.asarray(input_tokens)[src[p0:p1]], even)
    if packed:
        return np.concatenate([payload, scales], axis=1)
    return payload, scales


# --------------------------------------------------------------------------
# stage 4: combine
# --------------------------------------------------------------------------
def _combine_acc(y_bits, w, pos, t0, t1, top_k):
    """fp32 sum for rows [t0, t1): acc = +0, then acc = fl(acc + fl(w*y)) over routed j ascending."""
    h = y_bits.shape[1]
    acc = np.zeros((t1 - t0, h), dtype=np.float32)
    for j in range(top_k):
        p = pos[t0:t1, j]
        routed = p != SENT
        if not routed.any():
            continue
        rows = bf16_bits_to_f32(y_bits[np.where(routed, p, 0).astype(np.int64)])
        prod = w[t0:t1, j, None] * rows            # one fp32 rounding
        acc = np.where(routed[:, None], acc + prod, acc)   # one fp32 rounding
    return acc


def combine(y_bits: np.ndarray, router_weights: np.ndarray, restore_token_order: np.ndarray,
            top_k: int, rows_per_pass: int = 256) -> np.ndarray:
    """out[t] = bf16( sum over j = 0..top_k-1 of w[t,j] * y[restore[t*top_k + j]] ).

    ("Struct_ep_combine_wait": weighted sum of routed expert outputs with the
    router weights, output [num_tokens, hidden_size].)  fp32 with each product
    and each sum rounded separately, j ascending, unrouted slots skipped."""
    return combine_epilogue(y_bits, router_weights, restore_token_order, top_k, None, None, rows_per_pass)


def combine_epilogue(y_bits: np.ndarray, router_weights: np.ndarray, restore_token_order: np.ndarray,
                     top_k: int, scale=1.0, residual_bits: np.ndarray = None,
                     rows_per_pass: int = 256) -> np.ndarray:
    """combine followed by the fused elementwise epilogue ("Struct_ep_combine_wait",
    Parameters: has_epilogue_fusion): out = bf16(fl(fl(scale * acc) + residual)).
    scale=None and residual=None give the plain combine."""
    w = np.asarray(router_weights, dtype=np.float32)
    n = w.shape[0]
    pos = np.asarray(restore_token_order, dtype=np.uint32).reshape(n, top_k)
    y_bits = np.asarray(y_bits, dtype=np.uint16)
    h = y_bits.shape[1]
    out = np.empty((n, h), dtype=np.uint16)
    for t0 in range(0, n, rows_per_pass):
        t1 = min(n, t0 + rows_per_pass)
        acc = _combine_acc(y_bits, w, pos, t0, t1, top_k)
        if scale is not None:
            acc = np.float32(scale) * acc                              # one fp32 rounding
        if residual_bits is not None:
            acc = acc + bf16_bits_to_f32(np.asarray(residual_bits)[t0:t1])   # one fp32 rounding
        out[t0:t1] = f32_to_bf16_rne(acc)
    return out
