"""The bounds-checked build (libepx_checked.so) on the GPU.

In that build every row index a kernel computes, or reads from a layout, is
checked against the buffer it addresses before the access; an index out of
bounds skips the access and is counted (epx_checked_violations).

* The parity cases (layout, dispatch in both modes and payloads, the fused
  call at decode and large sizes, combine, the relay receive side, expert
  groups, a third of the seeded random geometries) run through the checked
  library: results bit-exact against the oracle and not one violation.
* A layout made for a larger problem, used with a smaller one, yields rows
  past the declared capacities. The buffers are allocated at the larger
  problem's size, so each skipped access would still have landed inside an
  allocation, and so are the token-indexed inputs (x, the weights), which
  the kernels only read for tokens below the declared count. The test checks
  that the rows past the declared capacity are untouched, the rows inside it
  are right, and that the skipped accesses were counted (once per lane that
  skipped).
"""
import importlib.util
import os

import numpy as np
import pytest
import torch

import oracle
from combine_epx_get_amd import workloads as W
from tests import test_parity_fused_gpu as TF
from tests import test_parity_gpu as TP
from tests import test_parity_random_gpu as TRG
from tests import test_parity_relay_gpu as TR

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECKED = os.path.join(ROOT, "combine_epx_get_amd", "libepx_checked.so")


@pytest.fixture(scope="module")
def epxc():
    """A second instance of the binding, bound to the checked library."""
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    if not os.path.exists(CHECKED):
        raise RuntimeError(f"{CHECKED} is not built")
    old = os.environ.get("EPX_LIBRARY")
    os.environ["EPX_LIBRARY"] = CHECKED
    try:
        spec = importlib.util.spec_from_file_location(
            "epx_checked_binding", os.path.join(ROOT, "combine_epx_get_amd", "epx.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
    finally:
        if old is None:
            del os.environ["EPX_LIBRARY"]
        else:
            os.environ["EPX_LIBRARY"] = old
    assert mod._LIB_PATH == CHECKED
    mod.epx_checked_violations()   # starts from zero
    return mod


CASES = [("tiny", "per_expert", "bf16"), ("tiny", "relay", "fp8"), ("decode_skewed", "relay", "bf16"),
         ("large_batch", "per_expert", "bf16"), ("fp8_dispatch", "relay", "fp8"),
         ("rank_heavy", "per_expert", "fp8")]


@pytest.mark.parametrize("name,mode,dtype", CASES)
def test_checked_parity_without_violations(epxc, name, mode, dtype):
    w = W.WORKLOADS[name]
    d = W.make_inputs(w)
    print(f"[checked] {name} {mode} {dtype}", flush=True)
    TP.run_case(epxc, d["x"], d["topk_idx"], d["topk_weights"], w.num_experts, w.num_ranks,
                w.num_hosts, w.my_rank, mode == "relay", dtype, f"checked/{name}/{mode}/{dtype}")
    TF.run_fused(epxc, d["x"], d["topk_idx"], w.num_experts, w.num_ranks, w.num_hosts, w.my_rank,
                 mode == "relay", dtype, what=f"checked fused/{name}/{mode}/{dtype}")
    if mode == "relay":
        TR.run_relay_case(epxc, d["x"], d["topk_idx"], d["topk_weights"], w.num_experts, w.num_ranks,
                          w.num_hosts, w.my_rank, f"checked relay/{name}")
    assert epxc.epx_checked_violations() == 0


def test_checked_groups_without_violations(epxc):
    rng = np.random.Generator(np.random.PCG64(21))
    T, k, E, R, H, h, m = 600, 8, 64, 8, 2, 256, 4
    x = W.f32_to_bf16_bits(rng.standard_normal((T, h), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, "uniform")
    TF.run_fused(epxc, x, idx, E, R, H, 0, False, "bf16", m=m, what="checked groups")
    p = epxc.make_problem(T, k, E, R, H, 0, epxc.MODE_PER_EXPERT, m)
    L = epxc.Layout(p)
    epxc.epx_get_layout(p, torch.from_numpy(idx).cuda(), L)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    recv = torch.zeros((T * k, h), dtype=torch.bfloat16, device="cuda")
    y = torch.from_numpy(W.random_bf16((T * k, h), seed=3).view(np.int16)).view(torch.bfloat16).cuda()
    wts = torch.from_numpy(W.draw_gate_weights(rng, T, k)).cuda()
    carry = torch.empty((T, h), dtype=torch.float32, device="cuda")
    out = torch.empty((T, h), dtype=torch.bfloat16, device="cuda")
    for g in range(m):
        epxc.epx_dispatch_group(p, L, g, xt, epxc.BF16, recv)
    for g in range(m):
        epxc.epx_combine_group(p, L, g, y, wts, carry, out)
    ora = oracle.layout_grouped(idx, E, R, m)
    assert np.array_equal(TP._bits(recv), x[ora["row_token"]])
    assert epxc.epx_checked_violations() == 0


RANDOM = TRG.CASES[::3]


@pytest.mark.parametrize("case", RANDOM, ids=[f"c{c['seed']}-T{c['T']}k{c['k']}E{c['E']}R{c['R']}H{c['H']}h{c['hidden']}"
                                              for c in RANDOM])
def test_checked_random_geometries_without_violations(epxc, case):
    """A third of the seeded random geometries (empty batches, k up to 64,
    up to 64 hosts, duplicate ids) through the checked library: every call,
    the relay receive side included, bit-exact and in bounds."""
    c = case
    print(f"[checked random] {c}", flush=True)
    rng = np.random.Generator(np.random.PCG64(5000 + c["seed"]))
    T, k, E, R, H, s, h = c["T"], c["k"], c["E"], c["R"], c["H"], c["s"], c["hidden"]
    x = W.f32_to_bf16_bits(rng.standard_normal((T, h), dtype=np.float32))
    if c["dup"]:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    else:
        idx = W.draw_routing(rng, T, E, k, c["routing"], 1.1)
    w = W.draw_gate_weights(rng, T, k)
    dtypes = ("bf16", "fp8") if h % 128 == 0 else ("bf16",)
    for relay in (False, True):
        for dt in dtypes:
            TP.run_case(epxc, x, idx, w, E, R, H, s, relay, dt, f"checked {c}/relay={relay}/{dt}")
            TF.run_fused(epxc, x, idx, E, R, H, s, relay, dt, what=f"checked {c}/relay={relay}/fused {dt}")
    if T > 0:
        TR.run_relay_case(epxc, x, idx, w, E, R, H, s, f"checked relay {c}")
    assert epxc.epx_checked_violations() == 0


def _sentinel_rows(n, h):
    return torch.full((n, h), TP.SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def test_checked_build_skips_and_counts_rows_past_the_declared_capacity(epxc):
    """A layout made for 200 tokens used for the first 100 of them: about
    half of their rows lie past the 100-token capacity."""
    rng = np.random.Generator(np.random.PCG64(22))
    Tb, Ts, k, E, R, H, h = 200, 100, 4, 16, 4, 2, 256
    idx = W.draw_routing(rng, Tb, E, k, "uniform")
    x = W.f32_to_bf16_bits(rng.standard_normal((Tb, h), dtype=np.float32))
    pb = epxc.make_problem(Tb, k, E, R, H, 0, epxc.MODE_PER_EXPERT)
    ps = epxc.make_problem(Ts, k, E, R, H, 0, epxc.MODE_PER_EXPERT)
    Lb = epxc.Layout(pb)
    epxc.epx_get_layout(pb, torch.from_numpy(idx).cuda(), Lb)
    assert epxc.epx_checked_violations() == 0
    slot = Lb["slot"].cpu().numpy()[:Ts * k]
    over = int(np.count_nonzero(slot >= Ts * k))
    assert over > 0

    # dispatch: recv allocated for the large problem, declared with the small capacity
    recv = _sentinel_rows(Tb * k, h)
    xb = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()   # Tb rows
    ctypes = epxc.ctypes
    st = epxc._lib.epx_dispatch(ctypes.byref(ps), ctypes.byref(Lb.struct), xb.data_ptr(), h, epxc.BF16,
                                recv.data_ptr(), None, Ts * k, epxc._stream(None))
    assert st == 0
    assert epxc.epx_checked_violations() >= over
    got = TP._bits(recv)
    assert np.all(got[Ts * k:] == TP.SENTINEL_BF16 & 0xFFFF)           # nothing past the capacity
    inside = slot < Ts * k
    rows = slot[inside]
    toks = np.repeat(np.arange(Ts), k)[inside]
    assert np.array_equal(got[rows], x[toks])                          # the rows inside it are right

    # combine: y allocated for the large problem, declared with the small row count
    y = torch.from_numpy(W.random_bf16((Tb * k, h), seed=5).view(np.int16)).view(torch.bfloat16).cuda()
    wts = torch.ones((Tb, k), dtype=torch.float32, device="cuda")
    out = _sentinel_rows(Tb, h)
    st = epxc._lib.epx_combine(ctypes.byref(ps), ctypes.byref(Lb.struct), y.data_ptr(), Ts * k, wts.data_ptr(),
                               h, out.data_ptr(), epxc._stream(None))
    assert st == 0
    assert epxc.epx_checked_violations() >= over
    assert np.all(TP._bits(out)[Ts:] == TP.SENTINEL_BF16 & 0xFFFF)

    # relay fan-out: relay rows and recv declared at the small problem's capacities
    pbr = epxc.make_problem(Tb, k, E, R, H, 0, epxc.MODE_HOST_RELAY)
    psr = epxc.make_problem(Ts, k, E, R, H, 0, epxc.MODE_HOST_RELAY)
    Lr = epxc.Layout(pbr)
    epxc.epx_get_layout(pbr, torch.from_numpy(idx).cuda(), Lr)
    relay_rows = torch.from_numpy(W.random_bf16((Tb * 2, h), seed=6).view(np.int16)).view(torch.bfloat16).cuda()
    fan = _sentinel_rows(Tb * k, h)
    st = epxc._lib.epx_relay_fanout(ctypes.byref(psr), ctypes.byref(Lr.struct), relay_rows.data_ptr(), None,
                                    Ts * 2, h, epxc.BF16, fan.data_ptr(), None, Ts * k, epxc._stream(None))
    assert st == 0
    assert epxc.epx_checked_violations() > 0
    assert np.all(TP._bits(fan)[Ts * k:] == TP.SENTINEL_BF16 & 0xFFFF)
