"""The C-ABI library loads, exports every declared entry point and rejects bad
arguments on the host (no GPU needed: a call that fails a host check launches
nothing)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "epx.h")
LIB = os.path.join(ROOT, "combine_epx_get_amd", "libepx.so")


@pytest.fixture(scope="module")
def epx():
    if not os.path.exists(LIB):
        from combine_epx_get_amd import build
        build.build()
    from combine_epx_get_amd import epx as mod
    return mod


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"EPX_API\s+[\w\s\*]+?\b(epx_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for need in ("epx_get_layout", "epx_dispatch", "epx_combine", "epx_layout_sizes",
                 "epx_read_error", "epx_status_string", "epx_abi_version", "epx_f32_to_e4m3"):
        assert need in names


def test_library_exports_every_declared_symbol(epx):
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and nothing else with external linkage besides the ABI
    out = os.popen(f"nm -D --defined-only {LIB}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_abi_version_and_status_strings(epx):
    assert epx.abi_version() == 4
    for code in range(6):
        assert epx._lib.epx_status_string(code)


def test_layout_sizes(epx):
    p = epx.make_problem(4096, 8, 256, 16, 2, 3, epx.MODE_HOST_RELAY)
    s = dict(zip(epx.LAYOUT_FIELDS, epx.epx_layout_sizes(p)))
    assert s["expert_count"] == 256 and s["expert_offset"] == 257
    assert s["rank_rows"] == 16 and s["rank_offset"] == 17
    assert s["host_tokens"] == 2 and s["host_offset"] == 3
    assert s["slot"] == s["row_token"] == 4096 * 8
    assert s["relay_slot"] == 4096 * 2
    assert s["relay_token"] == s["fanout_rank_mask"] == 4096 * 2
    assert s["fanout_expert"] == 4096 * 2 * 8
    assert s["totals"] == 4
    assert s["group_offset"] == 16 + 1
    assert s["workspace"] == (128 + 1) * (256 + 16 + 2 + 1)    # 128 chunks of 32 tokens, + totals
    pg = epx.make_problem(4096, 8, 256, 16, 2, 3, epx.MODE_PER_EXPERT, 4)
    sg = dict(zip(epx.LAYOUT_FIELDS, epx.epx_layout_sizes(pg)))
    assert sg["group_offset"] == 4 * 16 + 1 and sg["slot"] == 4096 * 8
    p0 = epx.make_problem(0, 2, 16, 4, 2)
    s0 = dict(zip(epx.LAYOUT_FIELDS, epx.epx_layout_sizes(p0)))
    assert s0["slot"] == 0 and s0["workspace"] == (4 + 1) * (16 + 4 + 2 + 1)   # columns padded to 4


@pytest.mark.parametrize("geom", [
    (10, 0, 16, 4, 2, 0, 0),      # k = 0
    (10, 65, 128, 4, 2, 0, 0),    # k above the limit
    (10, 17, 16, 4, 2, 0, 0),     # k > E
    (10, 2, 16, 3, 1, 0, 0),      # E % R
    (10, 2, 16, 4, 3, 0, 0),      # R % H
    (10, 2, 16, 4, 2, 4, 0),      # my_rank out of range
    (10, 2, 16, 4, 2, -1, 0),
    (10, 2, 4096, 4, 2, 0, 0),    # E above the limit
    (10, 2, 128, 128, 128, 0, 0), # H above the limit
    (10, 2, 128, 64, 1, 0, 0),    # ranks per host above 32
    (10, 2, 16, 4, 2, 0, 7),      # bad mode
    (-1, 2, 16, 4, 2, 0, 0),      # negative T
    ((1 << 24) + 1, 2, 16, 4, 2, 0, 0),
    (10, 2, 24, 4, 2, 0, 0, 4),   # 6 experts per rank, 4 groups
    (10, 2, 16, 4, 2, 0, 1, 2),   # groups in relay mode
    (10, 2, 16, 4, 2, 0, 0, -1),  # negative group count
    (10, 2, 16, 4, 2, 0, 0, 8),   # more groups than experts per rank
])
def test_bad_geometry_is_rejected_on_the_host(epx, geom):
    p = epx.make_problem(*geom)
    with pytest.raises(epx.EpxError) as ei:
        epx.epx_layout_sizes(p)
    assert ei.value.code == 1
    lay = epx.epx_layout()
    assert epx._lib.epx_get_layout(ctypes.byref(p), None, ctypes.byref(lay), None) == 1


def _fake_layout(epx, relay):
    # distinct, 256-byte aligned fake addresses: never dereferenced because
    # every call below fails a host check first
    ptrs = [0x100000 + 0x1000 * i for i in range(len(epx.LAYOUT_FIELDS))]
    if not relay:
        for i, n in enumerate(epx.LAYOUT_FIELDS):
            if n in epx.RELAY_FIELDS:
                ptrs[i] = None
    return epx.epx_layout(*ptrs)


def test_host_checks_of_the_calls(epx):
    lib = epx._lib
    p = epx.make_problem(64, 2, 16, 4, 2, 0, epx.MODE_PER_EXPERT)
    pr = epx.make_problem(64, 2, 16, 4, 2, 0, epx.MODE_HOST_RELAY)
    L = _fake_layout(epx, relay=False)
    A = 0x200000
    by = ctypes.byref
    # layout: missing topk_idx, misaligned topk_idx, relay arrays missing in relay mode
    assert lib.epx_get_layout(by(p), None, by(L), None) == 1
    assert lib.epx_get_layout(by(p), A + 2, by(L), None) == 1
    assert lib.epx_get_layout(by(pr), A, by(L), None) == 1
    assert lib.epx_get_layout(by(p), A, None, None) == 1
    # dispatch: dtype, hidden, alignment, scales, capacity
    assert lib.epx_dispatch(by(p), by(L), A, 256, 5, A, None, 128, None) == 1
    assert lib.epx_dispatch(by(p), by(L), A, 252, 0, A, None, 128, None) == 1
    assert lib.epx_dispatch(by(p), by(L), A, 264, 1, A, A, 128, None) == 1     # fp8 needs h % 128
    assert lib.epx_dispatch(by(p), by(L), A + 8, 256, 0, A, None, 128, None) == 1
    assert lib.epx_dispatch(by(p), by(L), A, 256, 0, A + 4, None, 128, None) == 1
    assert lib.epx_dispatch(by(p), by(L), A, 256, 1, A, None, 128, None) == 1  # fp8 without scales
    assert lib.epx_dispatch(by(p), by(L), A, 256, 0, A, None, 127, None) == 3  # T*k = 128 rows
    LR = _fake_layout(epx, relay=True)
    assert lib.epx_dispatch(by(pr), by(LR), A, 256, 0, A, None, 127, None) == 3  # T*min(k,H) = 128
    assert lib.epx_dispatch(by(p), by(L), None, 256, 0, A, None, 128, None) == 1
    # combine: y rows, alignment, weights
    assert lib.epx_combine(by(p), by(L), A, 127, A, 256, A, None) == 3
    assert lib.epx_combine(by(p), by(L), A, 128, None, 256, A, None) == 1
    assert lib.epx_combine(by(p), by(L), A, 128, A + 2, 256, A, None) == 1
    assert lib.epx_combine(by(p), by(L), A, 128, A, 250, A, None) == 1
    assert lib.epx_combine(by(p), by(L), A + 8, 128, A, 256, A, None) == 1
    # conversion entry point
    assert lib.epx_f32_to_e4m3(None, None, -1, None) == 1
    assert lib.epx_f32_to_e4m3(None, None, 0, None) == 0
    assert lib.epx_read_error(None, None, None) == 1


@pytest.mark.parametrize("args", [
    # E, R, H, tau, and which pointer (by position) is bad
    (16, 3, 1, 0, None),        # E % R
    (16, 4, 3, 0, None),        # R % H
    (4096, 4, 1, 0, None),      # E above the limit
    (128, 64, 1, 0, None),      # 64 ranks on one host
    (128, 128, 128, 0, None),   # H above the limit
    (16, 4, 2, -1, None),       # negative tau
    (16, 4, 2, 0, 0),           # no expert_count
    (16, 4, 2, 0, 1),           # no slot_expert_in
    (16, 4, 2, 0, 6),           # no swaps with two ranks per host
    (16, 4, 2, 0, "alias"),     # output aliases input
    (16, 4, 2, 0, "misaligned"),
])
def test_plan_swaps_host_checks(epx, args):
    E, R, H, tau, bad = args
    ptrs = [0x300000 + 0x1000 * i for i in range(7)]   # count, in, out, before, after, swaps, bad
    if isinstance(bad, int):
        ptrs[bad if bad < 5 else 5] = None
    elif bad == "alias":
        ptrs[2] = ptrs[1]
    elif bad == "misaligned":
        ptrs[3] += 2
    c, i, o, lb, la, sw, hb = ptrs
    assert epx._lib.epx_plan_swaps(E, R, H, c, i, tau, o, lb, la, sw, hb, None) == 1


def test_group_entry_host_checks(epx):
    lib = epx._lib
    by = ctypes.byref
    A = 0x200000
    p = epx.make_problem(64, 2, 16, 4, 2, 0, epx.MODE_PER_EXPERT, 2)
    p1 = epx.make_problem(64, 2, 16, 4, 2, 0, epx.MODE_PER_EXPERT, 1)
    L = _fake_layout(epx, relay=False)
    assert lib.epx_dispatch_group(by(p), by(L), -1, A, 256, 0, A, None, 128, None) == 1
    assert lib.epx_dispatch_group(by(p), by(L), 2, A, 256, 0, A, None, 128, None) == 1
    assert lib.epx_dispatch_group(by(p), by(L), 0, A, 256, 0, A, None, 127, None) == 3
    assert lib.epx_dispatch_group(by(p1), by(L), 1, A, 256, 0, A, None, 128, None) == 1
    assert lib.epx_combine_group(by(p), by(L), 2, A, 128, A, 256, A, A, None) == 1
    assert lib.epx_combine_group(by(p), by(L), -1, A, 128, A, 256, A, A, None) == 1
    assert lib.epx_combine_group(by(p), by(L), 0, A, 128, A, 256, None, A, None) == 1      # no carry
    assert lib.epx_combine_group(by(p), by(L), 0, A, 128, A, 256, A + 8, A, None) == 1     # misaligned
    assert lib.epx_combine_group(by(p), by(L), 0, A, 127, A, 256, A, A, None) == 3
    # the layout needs group_offset
    ptrs = [0x100000 + 0x1000 * i for i in range(len(epx.LAYOUT_FIELDS))]
    ptrs[epx.LAYOUT_FIELDS.index("group_offset")] = None
    for n in epx.RELAY_FIELDS:
        ptrs[epx.LAYOUT_FIELDS.index(n)] = None
    assert lib.epx_get_layout(by(p), A, by(epx.epx_layout(*ptrs)), None) == 1


def test_fused_entry_host_checks(epx):
    """epx_layout_dispatch fails the checks of either call before launching."""
    lib = epx._lib
    by = ctypes.byref
    A = 0x200000
    p = epx.make_problem(64, 2, 16, 4, 2, 0, epx.MODE_PER_EXPERT)
    pr = epx.make_problem(64, 2, 16, 4, 2, 0, epx.MODE_HOST_RELAY)
    L = _fake_layout(epx, relay=False)
    # layout side: routing ids missing or misaligned, relay arrays missing, no layout
    assert lib.epx_layout_dispatch(by(p), None, by(L), A, 256, 0, A, None, 128, None) == 1
    assert lib.epx_layout_dispatch(by(p), A + 2, by(L), A, 256, 0, A, None, 128, None) == 1
    assert lib.epx_layout_dispatch(by(pr), A, by(L), A, 256, 0, A, None, 128, None) == 1
    assert lib.epx_layout_dispatch(by(p), A, None, A, 256, 0, A, None, 128, None) == 1
    # dispatch side: dtype, hidden, alignment, fp8 scales, capacity
    assert lib.epx_layout_dispatch(by(p), A, by(L), A, 256, 5, A, None, 128, None) == 1
    assert lib.epx_layout_dispatch(by(p), A, by(L), A, 252, 0, A, None, 128, None) == 1
    assert lib.epx_layout_dispatch(by(p), A, by(L), A, 264, 1, A, A, 128, None) == 1
    assert lib.epx_layout_dispatch(by(p), A, by(L), A + 8, 256, 0, A, None, 128, None) == 1
    assert lib.epx_layout_dispatch(by(p), A, by(L), A, 256, 0, A + 4, None, 128, None) == 1
    assert lib.epx_layout_dispatch(by(p), A, by(L), A, 256, 1, A, None, 128, None) == 1
    assert lib.epx_layout_dispatch(by(p), A, by(L), A, 256, 0, A, None, 127, None) == 3
    LR = _fake_layout(epx, relay=True)
    assert lib.epx_layout_dispatch(by(pr), A, by(LR), A, 256, 0, A, None, 127, None) == 3
    # geometry
    bad = epx.make_problem(64, 2, 16, 3, 1, 0, epx.MODE_PER_EXPERT)   # E % R != 0
    assert lib.epx_layout_dispatch(by(bad), A, by(L), A, 256, 0, A, None, 128, None) == 1


def test_noalloc_entry_host_checks(epx):
    """epx_layout_dispatch_noalloc refuses a problem whose workspace would not
    fit its static scratch before any HIP call (so on any host), and bad
    problems or a missing layout as epx_layout_dispatch does."""
    lib = epx._lib
    by = ctypes.byref
    A = 0x200000
    L = _fake_layout(epx, relay=False)
    big = epx.make_problem(1 << 20, 8, 2048, 64, 2, 0, epx.MODE_PER_EXPERT)
    ws = epx.epx_layout_sizes(big)[epx.LAYOUT_FIELDS.index("workspace")]
    assert ws * 4 > (16 << 20)
    assert lib.epx_layout_dispatch_noalloc(by(big), A, by(L), A, 256, 0, A, None, (1 << 20) * 8, None) == 5
    p = epx.make_problem(64, 2, 16, 4, 2, 0, epx.MODE_PER_EXPERT)
    assert lib.epx_layout_dispatch_noalloc(by(p), A, None, A, 256, 0, A, None, 128, None) == 1
    bad = epx.make_problem(64, 2, 16, 3, 1, 0, epx.MODE_PER_EXPERT)   # E % R != 0
    assert lib.epx_layout_dispatch_noalloc(by(bad), A, by(L), A, 256, 0, A, None, 128, None) == 1
    # the large-batch workload fits with room to spare
    lb = epx.make_problem(4096, 8, 256, 16, 2, 0, epx.MODE_PER_EXPERT)
    assert epx.epx_layout_sizes(lb)[epx.LAYOUT_FIELDS.index("workspace")] * 4 < (1 << 20)


def test_release_build_checks_nothing(epx):
    """epx_checked_violations is for the bounds-checked build; the release
    library refuses it on the host (count -1), before any HIP call."""
    n = ctypes.c_int64(7)
    assert epx._lib.epx_checked_violations(ctypes.byref(n), None) == 1 and n.value == -1
    assert epx._lib.epx_checked_violations(None, None) == 1


def test_checked_library_exports_the_same_symbols(epx):
    lib = os.path.join(ROOT, "combine_epx_get_amd", "libepx_checked.so")
    out = os.popen(f"nm -D --defined-only {lib}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_binding_rejects_wrong_tensors(epx):
    import torch
    p = epx.make_problem(4, 2, 16, 4, 2)
    with pytest.raises(ValueError):
        epx.epx_get_layout(p, torch.zeros(4, 2, dtype=torch.int64), None)
