"""The no-allocation index entry point, moe_create_indices_noalloc, called
through the C ABI: its outputs against those of the entry point it varies
(moe_create_indices with a caller workspace) and against the oracle,
bit-exact on every index output.  Calls on one GPU share the library's
static scratch, so the calls follow one another with smaller inputs, which
must see nothing an earlier call left there."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import INDEX_KEYS, check_indices, gpu_available, i32, u32

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

mod = pytest.importorskip("expert_grouping_dispatch_amd") if gpu_available() else None
DEV = "cuda"


def _ids(seed, n, k, e, masked):
    """k distinct experts per row for the first n - masked rows, -1 after them."""
    g = np.random.default_rng(seed)
    ids = np.argsort(g.random((n, e), dtype=np.float32), axis=1)[:, :k].astype(np.int32)
    ids[n - masked:] = -1
    return ids


def _host(t):
    return i32(t).astype(np.int64) if t.dtype == torch.int32 else u32(t).astype(np.int64)


def _noalloc(d_ids, e, out, align):
    mod.moe_create_indices_noalloc(d_ids, e, out["token_expert_order"], out["expert_start_indices"],
                                   out["restore_token_order"], out["expert_ids"], out["expert_usage_stats"],
                                   out["scales_offset"], align or 128)


def _both(ids, e, align=None):
    """Both entry points on the same map; returns the noalloc outputs."""
    s = ids.size
    print(f"[no-alloc] slots={s} E={e} align={align}", flush=True)
    d_ids = torch.from_numpy(ids.reshape(-1)).to(DEV)
    ws = mod.alloc_indices(s, e, DEV, scales_offset=align is not None)
    na = mod.alloc_indices(s, e, DEV, scales_offset=align is not None)
    for key in INDEX_KEYS + (("scales_offset",) if align else ()):
        na[key].view(torch.int32).fill_(0x5A5A5A5A)   # entries the call forgot to write would show
    mod.moe_create_indices(d_ids, e, ws["token_expert_order"], ws["expert_start_indices"],
                           ws["restore_token_order"], ws["expert_ids"], ws["expert_usage_stats"],
                           ws["workspace"], ws["scales_offset"], align or 128)
    _noalloc(d_ids, e, na, align)
    torch.cuda.synchronize()
    for key in INDEX_KEYS + (("scales_offset",) if align else ()):
        np.testing.assert_array_equal(_host(na[key]), _host(ws[key]), err_msg=key)
    ref = oracle.create_indices(ids.reshape(-1), e, scales_align=align)
    check_indices(na, ref)
    if align:
        np.testing.assert_array_equal(u32(na["scales_offset"]), ref["scales_offset"])
    assert mod.index_workspace_error(ws["workspace"]) == 0
    return na


def test_noalloc_matches_the_workspace_entry_point_on_shrinking_inputs():
    """Three calls in a row, each smaller than the one before: the stress
    workload's shape (524,288 slots, E = 256, 256 count-table chunks, padding
    rows masked), a mid-size one (16,384 slots, E = 8, 16 chunks, the one-launch
    few-expert pass, which uses no scratch) and a
    decode-sized one (2,048 slots, E = 256, the one-workgroup pass)."""
    _both(_ids(1, 65536, 8, 256, masked=4096), 256, align=128)
    _both(_ids(2, 8192, 2, 8, masked=1192), 8)
    _both(_ids(3, 256, 8, 256, masked=159), 256, align=32)


def test_noalloc_largest_input_and_the_limit():
    """The largest input the static scratch takes at E = 256 (496 chunks of
    2048 slots) matches the workspace entry point; one row more is refused
    with MOE_ERR_SCRATCH_LIMIT and nothing is enqueued; a smaller call after
    it is still right."""
    n = 496 * 2048 // 8
    _both(_ids(4, n, 8, 256, masked=1000), 256)
    big = torch.zeros((n + 1) * 8, dtype=torch.int32, device=DEV)
    out = mod.alloc_indices((n + 1) * 8, 256, DEV)
    with pytest.raises(mod.MoeError) as err:
        _noalloc(big, 256, dict(out, scales_offset=None), None)
    assert err.value.status == mod.ERR_SCRATCH_LIMIT
    _both(_ids(5, 4000, 8, 64, masked=0), 64)


@pytest.mark.parametrize("n, k, e", [(12000, 8, 256), (8192, 2, 8)])   # count table; few-expert pass
def test_noalloc_graph_replay(n, k, e):
    """Captured once into a HIP graph (after an eager call on the device),
    replayed with new ids copied in eagerly between replays: every replay
    matches the oracle."""
    d_ids = torch.zeros(n * k, dtype=torch.int32, device=DEV)
    out = mod.alloc_indices(n * k, e, DEV)
    out["scales_offset"] = None
    _noalloc(d_ids, e, out, None)   # first call on the device, outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _noalloc(d_ids, e, out, None)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _noalloc(d_ids, e, out, None)
    for seed in range(4):
        ids = _ids(10 + seed, n, k, e, masked=seed * 997)
        d_ids.copy_(torch.from_numpy(ids.reshape(-1)))
        torch.cuda.synchronize()
        _ = (d_ids.float() * 2).sum()   # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        check_indices(out, oracle.create_indices(ids.reshape(-1), e))
