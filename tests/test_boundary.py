"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, and rejects bad arguments with the
documented status before enqueuing anything.  Fake (but aligned, non-null)
pointers are used only in calls that must fail validation."""
import ctypes
import os
import re

import numpy as np
import pytest

import top_routing_grouped_router_amd as M
from top_routing_grouped_router_amd import _lib as L
from oracle import moe_oracle as O
from synth import stream

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUP, WS, PLACE = 0, 1, 2, 3, 4
FAKE = 1 << 20           # aligned, non-null, never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    declared = header_functions()
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(L.EXPORTED) == declared


def test_status_strings():
    lib = L.lib()
    for code, name in L.STATUS_NAMES.items():
        assert lib.moe_status_string(code).decode() == name


def dims(T=64, d=64, E=8, f=64, k=2, act=1):
    return L.moe_dims(T, d, E, f, k, act)


@pytest.mark.parametrize("kw,expect", [
    (dict(E=257), UNSUP), (dict(k=9, E=8), UNSUP), (dict(k=17, E=32), UNSUP),
    (dict(d=96), UNSUP), (dict(f=32), UNSUP), (dict(act=7), UNSUP),
    (dict(T=-1), INVALID), (dict(d=0), INVALID), (dict(k=0), INVALID), (dict(E=0), INVALID),
    (dict(T=1 << 28, k=8), UNSUP),
])
def test_route_rejects_bad_dims(kw, expect):
    lib = L.lib()
    dm = dims(**kw)
    st = lib.moe_route(ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-3, FAKE, 1,
                       None, None, None, FAKE, 1 << 30, None)
    assert st == expect, L.last_error()
    assert L.last_error()
    assert lib.moe_workspace_bytes(ctypes.byref(dm), 1) == 0


def test_null_and_misaligned_pointers_are_rejected():
    lib = L.lib()
    dm = dims()
    st = lib.moe_route(ctypes.byref(dm), None, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-3, FAKE, 1,
                       None, None, None, FAKE, 1 << 30, None)
    assert st == INVALID and "'x'" in L.last_error()
    st = lib.moe_combine(ctypes.byref(dm), FAKE + 4, FAKE, None, FAKE, None)
    assert st == INVALID and "aligned" in L.last_error()
    st = lib.moe_permute(ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                         1 << 30, None)
    assert st == INVALID and "x_perm" in L.last_error()


def test_gathered_calls_check_their_table_and_x():
    lib = L.lib()
    dm = dims()
    st = lib.moe_expert_up_gather(ctypes.byref(dm), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, None)
    assert st == INVALID and "src_token" in L.last_error()
    st = lib.moe_grouped_swiglu_fwd_gather(ctypes.byref(dm), None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == INVALID and "'x'" in L.last_error()
    st = lib.moe_expert_wgrad_gather(ctypes.byref(dm), FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, FAKE, FAKE, L.MOE_BF16, FAKE, 1 << 30, None)
    assert st == INVALID and "aligned" in L.last_error()
    # bf16 offsets into X are 32-bit: X of 2 GiB or more is refused
    big = dims(T=1 << 20, d=1024)
    st = lib.moe_expert_up_gather(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, None)
    assert st == UNSUP and "2 GiB" in L.last_error()


def test_groups_must_divide_tokens():
    lib = L.lib()
    dm = dims(T=60)
    st = lib.moe_route(ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-3, FAKE, 8,
                       None, None, None, FAKE, 1 << 30, None)
    assert st == INVALID and "divide" in L.last_error()
    st = lib.moe_route(ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-3, FAKE, 0,
                       None, None, None, FAKE, 1 << 30, None)
    assert st == INVALID


def test_small_workspace_is_rejected():
    lib = L.lib()
    dm = dims(T=4096, d=256, E=16, f=256, k=4)
    need = lib.moe_workspace_bytes(ctypes.byref(dm), 8)
    assert need > 0
    st = lib.moe_grouped_swiglu_bwd(ctypes.byref(dm), *([FAKE] * 13), L.MOE_BF16, FAKE, 1024,
                                    None)
    assert st == WS and "needed" in L.last_error()
    st = lib.moe_grouped_swiglu_bwd(ctypes.byref(dm), *([FAKE] * 13), L.MOE_BF16, None, need,
                                    None)
    assert st == WS
    st = lib.moe_route(ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-3, FAKE, 8,
                       None, None, None, FAKE, 64, None)
    assert st == WS


def _bwd(lib, dm, saved, wgrad_dtype, ws_bytes):
    """moe_grouped_swiglu_bwd with fake pointers; saved = (a, b, h) pointers."""
    return lib.moe_grouped_swiglu_bwd(ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, *saved,
                                      FAKE, FAKE, FAKE, FAKE, FAKE, wgrad_dtype, FAKE, ws_bytes,
                                      None)


def test_bwd_saved_activations_are_all_given_or_all_null():
    lib = L.lib()
    dm = dims(T=4096, d=256, E=16, f=256, k=4)
    need = lib.moe_grouped_swiglu_bwd_workspace_bytes(ctypes.byref(dm), 1)
    for saved in ((None, FAKE, FAKE), (FAKE, None, FAKE), (FAKE, FAKE, None), (None, None, FAKE)):
        assert _bwd(lib, dm, saved, L.MOE_BF16, need) == INVALID
        assert "all NULL" in L.last_error()


def test_bwd_recompute_needs_three_more_activation_buffers():
    lib = L.lib()
    dm = dims(T=4096, d=256, E=16, f=256, k=4)
    saved_ws = lib.moe_grouped_swiglu_bwd_workspace_bytes(ctypes.byref(dm), 0)
    recompute_ws = lib.moe_grouped_swiglu_bwd_workspace_bytes(ctypes.byref(dm), 1)
    assert 0 < saved_ws <= lib.moe_workspace_bytes(ctypes.byref(dm), 1)
    assert recompute_ws >= saved_ws + 3 * 4096 * 4 * 256 * 2
    # the saved-activation size is too small once the call must recompute
    assert _bwd(lib, dm, (None, None, None), L.MOE_BF16, saved_ws) == WS


def test_bwd_wgrad_dtype_is_checked():
    lib = L.lib()
    dm = dims(T=4096, d=256, E=16, f=256, k=4)
    need = lib.moe_grouped_swiglu_bwd_workspace_bytes(ctypes.byref(dm), 0)
    assert _bwd(lib, dm, (FAKE, FAKE, FAKE), 7, need) == INVALID
    assert "wgrad_dtype" in L.last_error()
    dm32 = dims(T=4096, d=256, E=16, f=256, k=4, act=L.MOE_F32)
    need32 = lib.moe_grouped_swiglu_bwd_workspace_bytes(ctypes.byref(dm32), 0)
    assert _bwd(lib, dm32, (FAKE, FAKE, FAKE), L.MOE_BF16, need32) == UNSUP
    st = lib.moe_expert_wgrad(ctypes.byref(dm32), *([FAKE] * 9), L.MOE_BF16, FAKE, need32, None)
    assert st == UNSUP


def test_workspace_covers_the_bwd_scratch():
    dm = dims(T=16384, d=2048, E=64, f=1024, k=6)
    n = L.workspace_bytes(dm, 16)
    assert n >= 2 * 16384 * 6 * 1024 * 2


def _pl(arr):
    return (ctypes.c_int32 * len(arr))(*arr)


def test_dispatch_plan_rejects_bad_placements():
    lib = L.lib()
    args = [FAKE] * 6 + [FAKE, 1 << 30, None]
    bad = [0] * 16                                  # all experts in group 0
    st = lib.moe_dispatch_plan(64, 2, 16, 4, FAKE, _pl(bad), *args)
    assert st == PLACE and "group" in L.last_error()
    st = lib.moe_dispatch_plan(64, 2, 16, 4, FAKE, _pl([5] * 16), *args)
    assert st == PLACE
    st = lib.moe_dispatch_plan(64, 2, 16, 3, FAKE, _pl([0] * 16), *args)   # G does not divide E
    assert st in (PLACE, INVALID)
    st = lib.moe_dispatch_plan(60, 2, 16, 8, FAKE, _pl(list(np.arange(16) // 2)), *args)
    assert st == INVALID                            # G does not divide T
    st = lib.moe_dispatch_plan(64, 2, 128, 128, FAKE, _pl(list(range(128))), *args)
    assert st == UNSUP                              # G > 64
    assert lib.moe_check_placement(16, 4, _pl(list(np.arange(16) // 4))) == OK
    with pytest.raises(M.MoEError) as ei:
        M.moe_check_placement(16, 4, [0, 1, 2, 3] * 3 + [0, 0, 0, 0])
    assert ei.value.status == PLACE


@pytest.mark.parametrize("E,G,seed", [(8, 2, 0), (16, 4, 1), (64, 8, 2), (64, 16, 3), (32, 32, 4),
                                      (12, 3, 5), (64, 1, 6)])
def test_greedy_placement_matches_oracle(E, G, seed):
    g = stream(seed, 77)
    W = g.integers(0, 50, size=(E, E)).astype(np.int64)
    W = W + W.T
    np.fill_diagonal(W, 0)
    W[g.integers(E), :] = 0          # an expert nobody co-selects
    W[:, g.integers(E)] = W[:, g.integers(E)]
    W = np.maximum(W, W.T)
    np.fill_diagonal(W, 0)
    ours = M.moe_placement_greedy(E, G, W)
    ref = O.placement_greedy(W, G)
    assert ours == [int(v) for v in ref]


def test_greedy_placement_ties_and_zero_matrix():
    E, G = 16, 4
    W = np.zeros((E, E), dtype=np.int64)
    assert M.moe_placement_greedy(E, G, W) == [int(v) for v in O.placement_greedy(W, G)]
    assert M.moe_placement_greedy(E, G, W) == [e // 4 for e in range(E)]


def test_gate_folded_support_query():
    """The folded path is offered on the LDS-DMA kernels (both tiles) where the
    weight gradients take a one-pass kernel, bf16 only; one dgate part per
    column tile of the output-gradient GEMM (128 wide, 256 on the big tile)."""
    lib = L.lib()
    for kw, ok, parts in [(dict(T=16384, d=256, E=16, f=256, k=4), 1, 2),      # C2
                          (dict(T=16384, d=256, E=64, f=64, k=4), 1, 1),       # C3
                          (dict(T=1000, d=256, E=16, f=192, k=3), 1, 2),
                          (dict(T=16384, d=2048, E=64, f=1024, k=6), 1, 4),    # C5: big tiles
                          (dict(T=1000, d=256, E=8, f=192, k=3), 0, 2)]:       # split-K wgrad
        dm = dims(**kw)
        assert lib.moe_gate_folded_supported(ctypes.byref(dm)) == ok, kw
        assert lib.moe_dgate_parts(ctypes.byref(dm)) == parts, kw
    dm = dims(T=2048, d=256, E=16, f=256, k=4, act=0)   # fp32
    assert lib.moe_gate_folded_supported(ctypes.byref(dm)) == 0
    split = dims(T=1000, d=256, E=8, f=192, k=3)   # split-K weight gradients
    st = lib.moe_expert_up_folded(ctypes.byref(split), *([FAKE] * 9), None)
    assert st == UNSUP and "moe_gate_folded_supported" in L.last_error()


def test_route_noalloc_rejects_dims_beyond_its_static_scratch():
    """The allocation-free router refuses, on the host and before any device
    call, dims whose scratch exceeds the static array (4 MiB)."""
    lib = L.lib()
    assert L.moe_route_noalloc_max_bytes() == 4 << 20
    dm = dims(T=1 << 20, d=64, E=256, f=64, k=1)
    st = lib.moe_route_noalloc(ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-3, FAKE,
                               1, None, None, None, None)
    assert st == UNSUP, L.last_error()
    assert "static scratch" in L.last_error()
