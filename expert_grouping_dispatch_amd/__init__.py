"""Python binding of the MI355X MoE token-routing library (``libmoe_route.so``).

Thin ctypes marshalling over the C ABI declared in ``include/moe_route.h``:
each function checks dtypes, shapes and devices of torch tensors, passes
their data pointers and the current HIP stream, and raises ``MoeError`` on a
nonzero status.  Every step of the path runs in the library's HIP kernels;
torch only provides device memory and streams.  There is no fallback: if
the library is missing, importing this package fails.

    mask -> moe_mask_padding(routing_map, real_token_count, tp_rank)        int32 or int64 map
    idx  -> moe_create_indices(topk_ids, n_experts, *outputs, workspace[, scales_offset, scales_align])
    both -> moe_mask_create_indices(routing_map, real_token_count, tp_rank, n_experts, *outputs, workspace, ...)
    out  -> moe_dispatch(input_tokens, top_k, restore_token_order, out)
            moe_dispatch_mxfp4(input_tokens, top_k, restore_token_order, out_q, out_scales, flags)
    out  -> moe_combine(y, router_weights, restore_token_order, top_k, output_tokens)
            moe_combine_epilogue(..., scale, residual)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SENTINEL", "MoeError", "LIB_PATH", "lib",
    "moe_mask_padding", "moe_create_indices", "moe_create_indices_workspace_bytes", "moe_mask_create_indices",
    "moe_create_indices_noalloc", "ERR_SCRATCH_LIMIT",
    "moe_dispatch", "moe_dispatch_mxfp4", "moe_combine", "moe_combine_epilogue", "moe_error_string",
    "MXFP4_EVEN_SCALE", "MXFP4_PACKED_ROWS",
    "alloc_indices", "alloc_dispatch", "alloc_dispatch_mxfp4", "index_workspace_error",
]

SENTINEL = 0xFFFFFFFF
MXFP4_BLOCK = 32
MXFP4_EVEN_SCALE = 1   # flags bit of moe_dispatch_mxfp4: "even-mode" scale exponent
MXFP4_PACKED_ROWS = 2  # flags bit of moe_dispatch_mxfp4: payload and scales in one row
ERR_SCRATCH_LIMIT = 5  # status: input too large for moe_create_indices_noalloc's static scratch
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_route.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python expert_grouping_dispatch_amd/build_lib.py`")

# torch is imported first so the library binds to the HIP runtime torch already loaded.
lib = ctypes.CDLL(LIB_PATH)

_p, _i32, _i64, _u32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
lib.moe_error_string.argtypes = [ctypes.c_int]
lib.moe_error_string.restype = ctypes.c_char_p
for _f in (lib.moe_mask_padding, lib.moe_mask_padding_i64):
    _f.argtypes = [_p, _i64, _i32, _p, _i32, _p]
    _f.restype = ctypes.c_int
lib.moe_create_indices_workspace_bytes.argtypes = [_i64, _i32]
lib.moe_create_indices_workspace_bytes.restype = _sz
for _f in (lib.moe_create_indices, lib.moe_create_indices_i64):
    _f.argtypes = [_p, _i64, _i32, _p, _p, _p, _p, _p, _p, _u32, _p, _sz, _p]
    _f.restype = ctypes.c_int
lib.moe_create_indices_noalloc.argtypes = [_p, _i64, _i32, _p, _p, _p, _p, _p, _p, _u32, _p]
lib.moe_create_indices_noalloc.restype = ctypes.c_int
for _f in (lib.moe_mask_create_indices, lib.moe_mask_create_indices_i64):
    _f.argtypes = [_p, _i64, _i32, _p, _i32, _i32, _p, _p, _p, _p, _p, _p, _u32, _p, _sz, _p]
    _f.restype = ctypes.c_int
lib.moe_dispatch.argtypes = [_p, _i64, _i32, _i32, _p, _p, _i64, _p]
lib.moe_dispatch.restype = ctypes.c_int
lib.moe_dispatch_mxfp4.argtypes = [_p, _i64, _i32, _i32, _p, _p, _p, _i64, _u32, _p]
lib.moe_dispatch_mxfp4.restype = ctypes.c_int
lib.moe_combine.argtypes = [_p, _i64, _p, _p, _i64, _i32, _i32, _p, _p]
lib.moe_combine.restype = ctypes.c_int
lib.moe_combine_epilogue.argtypes = [_p, _i64, _p, _p, _i64, _i32, _i32, ctypes.c_float, _p, _p, _p]
lib.moe_combine_epilogue.restype = ctypes.c_int


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {moe_error_string(status)} (status {status})")


def moe_error_string(status: int) -> str:
    return lib.moe_error_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MoeError(status, what)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else ctypes.c_void_p(0)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, device: torch.device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _device_of(t: torch.Tensor) -> torch.device:
    if t.device.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    return t.device


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _id_dtype(t: torch.Tensor, name: str):
    if t.dtype not in (torch.int32, torch.int64):
        raise TypeError(f"{name} must be int32 or int64, got {t.dtype}")
    return t.dtype


def moe_mask_padding(routing_map: torch.Tensor, real_token_count: torch.Tensor, tp_rank: int = 0) -> None:
    """In place: rows r with r + tp_rank*N >= *real_token_count become -1 (int32 or int64 map)."""
    dev = _device_of(routing_map)
    dt = _id_dtype(routing_map, "routing_map")
    _need(routing_map, "routing_map", dt, dev)
    _need(real_token_count, "real_token_count", torch.int32, dev)
    if routing_map.dim() != 2 or real_token_count.numel() != 1:
        raise ValueError("routing_map must be [N, top_k] and real_token_count [1]")
    n, k = routing_map.shape
    with torch.cuda.device(dev):
        fn = lib.moe_mask_padding if dt == torch.int32 else lib.moe_mask_padding_i64
        _check(fn(_ptr(routing_map), n, k, _ptr(real_token_count), int(tp_rank), _stream(dev)),
               "moe_mask_padding")


def moe_create_indices_workspace_bytes(n_slots: int, n_experts: int) -> int:
    return int(lib.moe_create_indices_workspace_bytes(int(n_slots), int(n_experts)))


def index_workspace_error(workspace: torch.Tensor) -> int:
    """The sticky error word of an index workspace (its first 32-bit word):
    bit 0 is set if a cross-workgroup wait of moe_create_indices gave up,
    bit 1 if a call found the workspace not in the state a zero-filled one is
    left in.  0 after correct use.  Copies four bytes to the host, so it
    waits for the work queued on the workspace: not for use under graph
    capture."""
    _need(workspace, "workspace", torch.uint8, workspace.device)
    if workspace.numel() < 4:
        raise ValueError("workspace is smaller than its error word")
    return int(workspace[:4].view(torch.int32).item()) & 0xFFFFFFFF


def alloc_indices(n_slots: int, n_experts: int, device, scales_offset: bool = False) -> dict:
    """Output tensors (uninitialised) and a zero-filled workspace for moe_create_indices."""
    device = torch.device(device)
    ws = moe_create_indices_workspace_bytes(n_slots, n_experts)
    if ws == 0:
        raise ValueError("n_slots / n_experts out of range")
    u32 = dict(dtype=torch.uint32, device=device)
    return dict(
        token_expert_order=torch.empty(n_slots, **u32),
        expert_start_indices=torch.empty(n_experts + 1, **u32),
        restore_token_order=torch.empty(n_slots, **u32),
        expert_ids=torch.empty(n_experts, dtype=torch.int32, device=device),
        expert_usage_stats=torch.empty(2, **u32),
        workspace=torch.zeros(ws, dtype=torch.uint8, device=device),  # zero-filled once, reusable
        scales_offset=torch.empty(n_experts + 1, **u32) if scales_offset else None,
    )


def moe_create_indices(topk_ids: torch.Tensor, n_experts: int, token_expert_order: torch.Tensor,
                       expert_start_indices: torch.Tensor, restore_token_order: torch.Tensor,
                       expert_ids: torch.Tensor, expert_usage_stats: torch.Tensor,
                       workspace: torch.Tensor, scales_offset: torch.Tensor = None,
                       scales_align: int = 128) -> None:
    dev = _device_of(topk_ids)
    dt = _id_dtype(topk_ids, "topk_ids")
    _need(topk_ids, "topk_ids", dt, dev)
    s = topk_ids.numel()
    soff = _index_outputs(dev, s, n_experts, token_expert_order, expert_start_indices, restore_token_order,
                          expert_ids, expert_usage_stats, workspace, scales_offset)
    fn = lib.moe_create_indices if dt == torch.int32 else lib.moe_create_indices_i64
    with torch.cuda.device(dev):
        _check(fn(_ptr(topk_ids), s, int(n_experts), _ptr(token_expert_order), _ptr(expert_start_indices),
                  _ptr(restore_token_order), _ptr(expert_ids), _ptr(expert_usage_stats), soff,
                  int(scales_align), _ptr(workspace), workspace.numel(), _stream(dev)), "moe_create_indices")


def moe_create_indices_noalloc(topk_ids: torch.Tensor, n_experts: int, token_expert_order: torch.Tensor,
                               expert_start_indices: torch.Tensor, restore_token_order: torch.Tensor,
                               expert_ids: torch.Tensor, expert_usage_stats: torch.Tensor,
                               scales_offset: torch.Tensor = None, scales_align: int = 128) -> None:
    """moe_create_indices with the library's static per-GPU scratch instead of a workspace (nothing is
    allocated).  Inputs past the scratch raise MoeError with status ERR_SCRATCH_LIMIT; calls on one
    GPU must not overlap."""
    dev = _device_of(topk_ids)
    _need(topk_ids, "topk_ids", torch.int32, dev)
    s = topk_ids.numel()
    soff = _index_outputs(dev, s, n_experts, token_expert_order, expert_start_indices, restore_token_order,
                          expert_ids, expert_usage_stats, None, scales_offset)
    with torch.cuda.device(dev):
        _check(lib.moe_create_indices_noalloc(_ptr(topk_ids), s, int(n_experts), _ptr(token_expert_order),
                                              _ptr(expert_start_indices), _ptr(restore_token_order),
                                              _ptr(expert_ids), _ptr(expert_usage_stats), soff, int(scales_align),
                                              _stream(dev)), "moe_create_indices_noalloc")


def _index_outputs(dev, s, n_experts, token_expert_order, expert_start_indices, restore_token_order,
                   expert_ids, expert_usage_stats, workspace, scales_offset):
    for name, t, odt, n in (("token_expert_order", token_expert_order, torch.uint32, s),
                            ("expert_start_indices", expert_start_indices, torch.uint32, n_experts + 1),
                            ("restore_token_order", restore_token_order, torch.uint32, s),
                            ("expert_ids", expert_ids, torch.int32, n_experts),
                            ("expert_usage_stats", expert_usage_stats, torch.uint32, 2)):
        _need(t, name, odt, dev)
        if t.numel() != n:
            raise ValueError(f"{name} must have {n} elements, has {t.numel()}")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
    if scales_offset is None:
        return ctypes.c_void_p(0)
    _need(scales_offset, "scales_offset", torch.uint32, dev)
    if scales_offset.numel() != n_experts + 1:
        raise ValueError(f"scales_offset must have {n_experts + 1} elements")
    return _ptr(scales_offset)


def moe_mask_create_indices(routing_map: torch.Tensor, real_token_count: torch.Tensor, tp_rank: int,
                            n_experts: int, token_expert_order: torch.Tensor,
                            expert_start_indices: torch.Tensor, restore_token_order: torch.Tensor,
                            expert_ids: torch.Tensor, expert_usage_stats: torch.Tensor,
                            workspace: torch.Tensor, scales_offset: torch.Tensor = None,
                            scales_align: int = 128) -> None:
    """moe_mask_padding then moe_create_indices on the masked map, in one call."""
    dev = _device_of(routing_map)
    dt = _id_dtype(routing_map, "routing_map")
    _need(routing_map, "routing_map", dt, dev)
    _need(real_token_count, "real_token_count", torch.int32, dev)
    if routing_map.dim() != 2 or real_token_count.numel() != 1:
        raise ValueError("routing_map must be [N, top_k] and real_token_count [1]")
    n, k = routing_map.shape
    soff = _index_outputs(dev, n * k, n_experts, token_expert_order, expert_start_indices,
                          restore_token_order, expert_ids, expert_usage_stats, workspace, scales_offset)
    fn = lib.moe_mask_create_indices if dt == torch.int32 else lib.moe_mask_create_indices_i64
    with torch.cuda.device(dev):
        _check(fn(_ptr(routing_map), n, k, _ptr(real_token_count), int(tp_rank), int(n_experts),
                  _ptr(token_expert_order), _ptr(expert_start_indices), _ptr(restore_token_order),
                  _ptr(expert_ids), _ptr(expert_usage_stats), soff, int(scales_align), _ptr(workspace),
                  workspace.numel(), _stream(dev)), "moe_mask_create_indices")


def alloc_dispatch(n_slots: int, hidden: int, device) -> torch.Tensor:
    return torch.empty((n_slots, hidden), dtype=torch.bfloat16, device=device)


def alloc_dispatch_mxfp4(n_slots: int, hidden: int, device, packed: bool = False):
    """(payload, scales) buffers; with packed=True one [n_slots, hidden/2 + hidden/32] buffer and None."""
    if packed:
        return torch.empty((n_slots, hidden // 2 + hidden // MXFP4_BLOCK), dtype=torch.uint8, device=device), None
    return (torch.empty((n_slots, hidden // 2), dtype=torch.uint8, device=device),
            torch.empty((n_slots, hidden // MXFP4_BLOCK), dtype=torch.uint8, device=device))


def _rows_and_restore(input_tokens, restore_token_order, top_k, dev):
    _need(input_tokens, "input_tokens", torch.bfloat16, dev)
    _need(restore_token_order, "restore_token_order", torch.uint32, dev)
    if input_tokens.dim() != 2:
        raise ValueError("input_tokens must be [N, hidden]")
    n, h = input_tokens.shape
    if restore_token_order.numel() != n * top_k:
        raise ValueError("restore_token_order must have N*top_k elements")
    return n, h


def moe_dispatch(input_tokens: torch.Tensor, top_k: int, restore_token_order: torch.Tensor,
                 out: torch.Tensor) -> None:
    dev = _device_of(input_tokens)
    n, h = _rows_and_restore(input_tokens, restore_token_order, top_k, dev)
    _need(out, "out", torch.bfloat16, dev)
    if out.dim() != 2 or out.shape[1] != h:
        raise ValueError("out must be [rows, hidden]")
    with torch.cuda.device(dev):
        _check(lib.moe_dispatch(_ptr(input_tokens), n, h, int(top_k), _ptr(restore_token_order),
                                _ptr(out), out.shape[0], _stream(dev)), "moe_dispatch")


def moe_dispatch_mxfp4(input_tokens: torch.Tensor, top_k: int, restore_token_order: torch.Tensor,
                       out_q: torch.Tensor, out_scales, flags: int = 0) -> None:
    dev = _device_of(input_tokens)
    n, h = _rows_and_restore(input_tokens, restore_token_order, top_k, dev)
    _need(out_q, "out_q", torch.uint8, dev)
    if flags & MXFP4_PACKED_ROWS:
        if out_scales is not None:
            raise ValueError("out_scales must be None with MXFP4_PACKED_ROWS")
        if out_q.dim() != 2 or out_q.shape[1] != h // 2 + h // MXFP4_BLOCK:
            raise ValueError("packed out_q must be [rows, hidden/2 + hidden/32]")
        sc = ctypes.c_void_p(0)
    else:
        _need(out_scales, "out_scales", torch.uint8, dev)
        if out_q.dim() != 2 or out_q.shape[1] != h // 2 or out_scales.shape != (out_q.shape[0], h // MXFP4_BLOCK):
            raise ValueError("out_q must be [rows, hidden/2] and out_scales [rows, hidden/32]")
        sc = _ptr(out_scales)
    with torch.cuda.device(dev):
        _check(lib.moe_dispatch_mxfp4(_ptr(input_tokens), n, h, int(top_k), _ptr(restore_token_order),
                                      _ptr(out_q), sc, out_q.shape[0], int(flags), _stream(dev)),
               "moe_dispatch_mxfp4")


def moe_combine(y: torch.Tensor, router_weights: torch.Tensor, restore_token_order: torch.Tensor,
                top_k: int, output_tokens: torch.Tensor) -> None:
    dev = _device_of(y)
    _need(y, "y", torch.bfloat16, dev)
    _need(router_weights, "router_weights", torch.float32, dev)
    _need(restore_token_order, "restore_token_order", torch.uint32, dev)
    _need(output_tokens, "output_tokens", torch.bfloat16, dev)
    if y.dim() != 2 or output_tokens.dim() != 2 or y.shape[1] != output_tokens.shape[1]:
        raise ValueError("y must be [rows, hidden] and output_tokens [N, hidden]")
    n, h = output_tokens.shape
    if router_weights.numel() != n * top_k or restore_token_order.numel() != n * top_k:
        raise ValueError("router_weights / restore_token_order must have N*top_k elements")
    with torch.cuda.device(dev):
        _check(lib.moe_combine(_ptr(y), y.shape[0], _ptr(router_weights), _ptr(restore_token_order), n, h,
                               int(top_k), _ptr(output_tokens), _stream(dev)), "moe_combine")


def moe_combine_epilogue(y: torch.Tensor, router_weights: torch.Tensor, restore_token_order: torch.Tensor,
                         top_k: int, output_tokens: torch.Tensor, scale: float = 1.0,
                         residual: torch.Tensor = None) -> None:
    """moe_combine followed by out = bf16(fl(scale * acc) [+ residual])."""
    dev = _device_of(y)
    _need(y, "y", torch.bfloat16, dev)
    _need(router_weights, "router_weights", torch.float32, dev)
    _need(restore_token_order, "restore_token_order", torch.uint32, dev)
    _need(output_tokens, "output_tokens", torch.bfloat16, dev)
    if y.dim() != 2 or output_tokens.dim() != 2 or y.shape[1] != output_tokens.shape[1]:
        raise ValueError("y must be [rows, hidden] and output_tokens [N, hidden]")
    n, h = output_tokens.shape
    if router_weights.numel() != n * top_k or restore_token_order.numel() != n * top_k:
        raise ValueError("router_weights / restore_token_order must have N*top_k elements")
    res = ctypes.c_void_p(0)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, dev)
        if residual.shape != output_tokens.shape:
            raise ValueError("residual must be [N, hidden]")
        res = _ptr(residual)
    with torch.cuda.device(dev):
        _check(lib.moe_combine_epilogue(_ptr(y), y.shape[0], _ptr(router_weights), _ptr(restore_token_order), n,
                                        h, int(top_k), float(scale), res, _ptr(output_tokens), _stream(dev)),
               "moe_combine_epilogue")
