"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must export every function include/moe_route.h declares, and
argument errors must be rejected on the host before any device call.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")

mod = pytest.importorskip("expert_grouping_dispatch_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_path():
    assert declared_functions() == sorted([
        "moe_error_string", "moe_mask_padding", "moe_mask_padding_i64", "moe_create_indices_workspace_bytes",
        "moe_create_indices", "moe_create_indices_i64", "moe_mask_create_indices", "moe_mask_create_indices_i64",
        "moe_create_indices_noalloc",
        "moe_dispatch", "moe_dispatch_mxfp4", "moe_combine", "moe_combine_epilogue"])


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", mod.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(mod.lib, name) is not None


def test_error_strings():
    assert mod.moe_error_string(0) == "ok"
    for s in range(1, 6):
        assert mod.moe_error_string(s) not in ("ok", "unknown status")
    assert mod.moe_error_string(99) == "unknown status"


def test_workspace_size_query():
    f = mod.moe_create_indices_workspace_bytes
    assert f(-1, 8) == 0 and f(10, 0) == 0 and f(10, 1025) == 0 and f(2 ** 32 - 1, 8) == 0
    prev = 0
    for s in (0, 1, 4096, 4097, 100000, 524288, 2 ** 32 - 2):
        b = f(s, 256)
        assert b >= prev and b % 256 == 0
        prev = b
    assert f(524288, 1024) > f(524288, 8)


P = ctypes.c_void_p


def test_invalid_arguments_rejected_on_host():
    L = mod.lib
    fake = P(256)  # never dereferenced: every call below fails its argument check first
    cnt = P(512)
    assert L.moe_mask_padding(None, 4, 2, cnt, 0, None) == 1          # null map
    assert L.moe_mask_padding(fake, 4, 0, cnt, 0, None) == 1          # top_k < 1
    assert L.moe_mask_padding(fake, 4, 2, None, 0, None) == 1         # null count
    assert L.moe_mask_padding(fake, 4, 2, cnt, -1, None) == 1         # tp_rank < 0
    assert L.moe_mask_padding(fake, -1, 2, cnt, 0, None) == 1         # n_rows < 0
    assert L.moe_mask_padding(fake, 2 ** 31, 2, cnt, 0, None) == 1    # slots reach the sentinel
    ws = mod.moe_create_indices_workspace_bytes(100, 8)
    args = [fake, 100, 8, fake, fake, fake, fake, fake, None, 0, fake, ws, None]
    for fn in (L.moe_create_indices, L.moe_create_indices_i64):
        bad = list(args); bad[2] = 0
        assert fn(*bad) == 1                                        # n_experts < 1
        bad = list(args); bad[2] = 1025
        assert fn(*bad) == 1                                        # n_experts too large
        bad = list(args); bad[10] = None
        assert fn(*bad) == 1                                        # null workspace
        bad = list(args); bad[10] = P(256 + 8)
        assert fn(*bad) == 1                                        # misaligned workspace
        bad = list(args); bad[11] = ws - 1
        assert fn(*bad) == 2                                        # workspace too small
        bad = list(args); bad[8] = fake; bad[9] = 0
        assert fn(*bad) == 1                                        # scales_offset with align 0
        bad = list(args); bad[8] = fake; bad[9] = 2 ** 31
        assert fn(*bad) == 1                                        # aligned offsets would overflow
    assert L.moe_mask_padding_i64(P(260), 4, 2, cnt, 0, None) == 1   # int64 map misaligned
    ws = mod.moe_create_indices_workspace_bytes(50 * 2, 8)
    fused = [fake, 50, 2, cnt, 0, 8, fake, fake, fake, fake, fake, None, 0, fake, ws, None]
    for fn in (L.moe_mask_create_indices, L.moe_mask_create_indices_i64):
        bad = list(fused); bad[3] = None
        assert fn(*bad) == 1                                        # null count
        bad = list(fused); bad[4] = -1
        assert fn(*bad) == 1                                        # tp_rank < 0
        bad = list(fused); bad[2] = 0
        assert fn(*bad) == 1                                        # top_k < 1
        bad = list(fused); bad[5] = 1025
        assert fn(*bad) == 1                                        # n_experts too large
        bad = list(fused); bad[1] = 2 ** 31
        assert fn(*bad) == 1                                        # slots reach the sentinel
        bad = list(fused); bad[14] = ws - 1
        assert fn(*bad) == 2                                        # workspace too small
    assert L.moe_mask_create_indices_i64(P(260), 50, 2, cnt, 0, 8, fake, fake, fake, fake, fake, None, 0,
                                         fake, ws, None) == 1       # int64 map misaligned
    noalloc = [fake, 100, 8, fake, fake, fake, fake, fake, None, 0, None]
    N = L.moe_create_indices_noalloc
    bad = list(noalloc); bad[2] = 0
    assert N(*bad) == 1                                             # n_experts < 1
    bad = list(noalloc); bad[3] = None
    assert N(*bad) == 1                                             # null token_expert_order
    bad = list(noalloc); bad[8] = fake
    assert N(*bad) == 1                                             # scales_offset with align 0
    # past the static scratch (the lookback path) -> MOE_ERR_SCRATCH_LIMIT, before any device use
    for n_slots, e in [(496 * 2048 + 1, 256), (512 * 2048 + 1, 8), (127 * 2048 + 1, 1024), (2 ** 32 - 2, 1)]:
        bad = list(noalloc); bad[1] = n_slots; bad[2] = e
        assert N(*bad) == mod.ERR_SCRATCH_LIMIT, (n_slots, e)
    assert L.moe_dispatch(fake, 10, 12, 2, fake, fake, 20, None) == 1        # hidden % 8
    assert L.moe_dispatch(P(258), 10, 16, 2, fake, fake, 20, None) == 1      # misaligned x
    assert L.moe_dispatch(fake, 10, 16, 0, fake, fake, 20, None) == 1        # top_k < 1
    assert L.moe_dispatch(fake, 10, 16, 1025, fake, fake, 20, None) == 1     # top_k too large
    assert L.moe_dispatch_mxfp4(fake, 10, 48, 2, fake, fake, fake, 20, 0, None) == 1  # hidden % 32
    assert L.moe_dispatch_mxfp4(fake, 10, 64, 2, fake, fake, fake, 20, 4, None) == 1  # unknown flag
    assert L.moe_dispatch_mxfp4(fake, 10, 256, 2, fake, fake, None, 20, 2, None) == 1  # packed: hidden % 512
    assert L.moe_dispatch_mxfp4(fake, 10, 512, 2, fake, fake, fake, 20, 2, None) == 1  # packed: scales given
    assert L.moe_dispatch_mxfp4(fake, 10, 512, 2, fake, fake, None, 20, 0, None) == 1  # unpacked: no scales
    assert L.moe_combine(fake, 20, fake, fake, 10, 12, 2, fake, None) == 1   # hidden % 8
    assert L.moe_combine(fake, 20, None, fake, 10, 16, 2, fake, None) == 1   # null weights
    assert L.moe_combine(fake, -1, fake, fake, 10, 16, 2, fake, None) == 1   # y_rows < 0
    E = L.moe_combine_epilogue
    assert E(fake, 20, fake, fake, 10, 16, 2, ctypes.c_float(1.0), P(264), fake, None) == 1  # residual misaligned
    assert E(fake, 20, fake, fake, 10, 16, 2, ctypes.c_float(1.0), P(256 + 160), P(256), None) == 1  # overlap


def _hip_device_count():
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return 0
    n = ctypes.c_int(0)
    return n.value if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 else 0


@pytest.mark.skipif(_hip_device_count() > 0, reason="a HIP device is present: valid arguments would launch")
def test_no_device_is_rejected_after_the_argument_checks():
    """Valid arguments with no HIP device: the device check returns
    MOE_ERR_UNSUPPORTED_DEVICE and nothing is launched (the pointers are
    never dereferenced)."""
    L = mod.lib
    fake, cnt = P(256), P(512)
    assert L.moe_mask_padding(fake, 4, 2, cnt, 0, None) == 3
    ws = mod.moe_create_indices_workspace_bytes(100, 8)
    assert L.moe_create_indices(fake, 100, 8, fake, fake, fake, fake, fake, None, 0, P(1024), ws, None) == 3
    assert L.moe_dispatch(fake, 10, 16, 2, fake, fake, 20, None) == 3
    assert L.moe_dispatch_mxfp4(fake, 10, 64, 2, fake, fake, fake, 20, 0, None) == 3
    assert L.moe_combine(fake, 20, fake, fake, 10, 16, 2, fake, None) == 3
    # the largest inputs the static scratch takes reach the device check
    for n_slots, e in [(100, 8), (496 * 2048, 256), (512 * 2048, 8), (127 * 2048, 1024)]:
        assert L.moe_create_indices_noalloc(fake, n_slots, e, fake, fake, fake, fake, fake, None, 0, None) == 3


def test_workspace_size_follows_the_index_paths():
    """Inputs of up to 512 chunks (2048 slots each, 1024 up to 65536 slots)
    whose count table of 16-bit counts (rows of E+1 rounded up to a multiple
    of 8) holds at most 2^17 entries need only the fixed part of the
    workspace; larger ones add 8 bytes per (chunk, bucket) lookback word."""
    f = mod.moe_create_indices_workspace_bytes
    fixed = f(1, 8)
    assert fixed == f(2048, 1024) == f(65536, 1024)            # one workgroup; 64 chunks of 1024 slots
    for s, e in [(496 * 2048, 256), (512 * 2048, 8), (127 * 2048, 1024), (24000, 1024)]:
        assert f(s, e) == fixed, (s, e)
    for s, e, chunks in [(496 * 2048 + 1, 256, 497), (512 * 2048 + 1, 8, 513), (127 * 2048 + 1, 1024, 128)]:
        want = fixed + (chunks * (e + 1) * 8 + 255) // 256 * 256
        assert f(s, e) == want, (s, e)


def test_workspace_size_is_monotone_in_slots():
    """A workspace sized for some slot count fits every smaller one (across the
    switch between chunk sizes too)."""
    f = mod.moe_create_indices_workspace_bytes
    sizes = sorted(set(list(range(0, 140000, 97)) + [2047, 2048, 2049, 65535, 65536, 65537, 131072, 131073,
                                                     524288, 2 ** 32 - 2]))
    for e in (1, 8, 256, 1024):
        prev = 0
        for s in sizes:
            b = f(s, e)
            assert b >= prev, (s, e)
            prev = b
