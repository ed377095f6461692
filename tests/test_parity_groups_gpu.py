"""GPU parity of expert groups for per-expert overlap (digest "Balancing and
Beyond", section 3.3, Figure 4) against the oracle: the grouped layout, each
group's dispatch (bf16 and fp8 rows, other groups' rows untouched) and the
group combines carried in float32 across groups, all bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from combine_epx_get_amd import workloads as W
from tests.test_parity_gpu import (SENTINEL_BF16, SENTINEL_U8, _bf16_dev, _bits, _dev,
                                   expert_outputs, layout_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def epx():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


def _group_of(e, epr, m):
    return (e % epr) // (epr // m)


def run_group_case(epx, x_bits, idx, w, E, R, H, s, m, what=""):
    T, k = idx.shape
    hidden = x_bits.shape[1]
    epr = E // R
    ora = oracle.layout_grouped(idx, E, R, m)
    plain = oracle.layout(idx, E, R, H, s)
    p = epx.make_problem(T, k, E, R, H, s, epx.MODE_PER_EXPERT, m)
    L = epx.Layout(p)
    epx.epx_get_layout(p, _dev(idx), L)
    got = layout_np(epx, L, False)
    for n in ("expert_count", "expert_offset", "group_offset", "slot", "row_token"):
        assert np.array_equal(got[n], ora[n]), (what, n)
    assert np.array_equal(got["totals"][[0, 2, 3]], ora["totals"][[0, 2, 3]]), (what, "totals")
    for n in ("rank_rows", "rank_tokens", "host_tokens", "host_offset", "relay_dst_rank"):
        assert np.array_equal(got[n], plain[n]), (what, n)
    assert np.all(got["rank_offset"] == (plain["rank_offset"] if m == 1 else -1)), (what, "rank_offset")
    rows = T * k
    go = ora["group_offset"]
    x_t = _bf16_dev(x_bits)

    # one group at a time: group g's rows appear, later groups' rows untouched
    recv = torch.full((rows, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    for g in range(m):
        epx.epx_dispatch_group(p, L, g, x_t, epx.BF16, recv)
        r = _bits(recv)
        want = oracle.dispatch_group(x_bits, ora, idx, E, R, m, g)
        lo, hi = go[g * R], go[(g + 1) * R]
        assert np.array_equal(r[lo:hi], want[lo:hi]), (what, "bf16 group", g)
        assert np.all(r[hi:] == np.uint16(SENTINEL_BF16 & 0xFFFF)), (what, "later groups touched", g)
    assert np.array_equal(_bits(recv), x_bits[ora["row_token"]]), (what, "all groups")
    # the plain dispatch over a grouped layout writes the same rows
    whole = torch.empty_like(recv)
    epx.epx_dispatch(p, L, x_t, epx.BF16, whole)
    assert np.array_equal(_bits(whole), _bits(recv)), (what, "plain dispatch")

    if hidden % 128 == 0:
        q = torch.full((rows, hidden), SENTINEL_U8, dtype=torch.uint8, device="cuda")
        sc = torch.full((rows, hidden // 128), -1.0, dtype=torch.float32, device="cuda")
        for g in range(m):
            epx.epx_dispatch_group(p, L, g, x_t, epx.FP8_E4M3, q, sc)
            wq, wsc = oracle.dispatch_group(x_bits, ora, idx, E, R, m, g, fp8=True)
            lo, hi = go[g * R], go[(g + 1) * R]
            qn, sn = q.cpu().numpy(), sc.cpu().numpy()
            assert np.array_equal(qn[lo:hi], wq[lo:hi]), (what, "fp8 codes", g)
            assert np.array_equal(sn[lo:hi].view(np.uint32), wsc[lo:hi].view(np.uint32)), (what, "scales", g)
            assert np.all(qn[hi:] == SENTINEL_U8) and np.all(sn[hi:] == -1.0), (what, "fp8 later groups", g)

    # group combines on one carry that starts as NaN: only carried values are read
    y = expert_outputs(W.bf16_bits_to_f32(x_bits), idx, ora["slot"])
    y_t, w_t = _bf16_dev(y), _dev(w)
    carry = torch.full((T, hidden), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((T, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    last = _group_of(idx, epr, m).max(axis=1) if T else np.zeros(0, int)
    for g in range(m):
        epx.epx_combine_group(p, L, g, y_t, w_t, carry, out)
        o = _bits(out)
        pending = last > g
        assert np.all(o[pending] == np.uint16(SENTINEL_BF16 & 0xFFFF)), (what, "out before last group", g)
    want_o = oracle.combine_grouped(y, ora, idx, w, E, R, m)
    assert np.array_equal(_bits(out), want_o), (what, "grouped combine")
    if m == 1:
        flat = torch.empty_like(out)
        epx.epx_combine(p, L, y_t, w_t, flat)
        assert np.array_equal(_bits(flat), want_o), (what, "one group = plain combine")


@pytest.mark.parametrize("name", ["tiny", "decode_skewed", "large_batch", "fp8_dispatch"])
@pytest.mark.parametrize("m", [2, 4])
def test_group_workload_parity(epx, name, m):
    w = W.WORKLOADS[name]
    d = W.make_inputs(w)
    print(f"[group parity] {name} m={m} T={d['T']}", flush=True)
    run_group_case(epx, d["x"], d["topk_idx"], d["topk_weights"], w.num_experts, w.num_ranks,
                   w.num_hosts, w.my_rank, m, f"{name} m={m}")


SHAPES = [
    # T, k, E, R, H, s, m, hidden
    (1, 1, 4, 2, 1, 0, 2, 8),
    (63, 3, 12, 2, 2, 1, 3, 136),       # 6 experts per rank, 3 groups
    (200, 4, 32, 8, 4, 6, 4, 1024),
    (257, 2, 16, 4, 2, 3, 2, 256),
    (130, 6, 6, 3, 1, 1, 2, 264),       # one expert per group per rank
    (3000, 16, 2048, 64, 2, 33, 2, 256),
    (50, 64, 64, 8, 4, 1, 4, 128),
    (5000, 8, 256, 16, 2, 5, 4, 128),
    (300, 8, 64, 8, 1, 0, 1, 512),      # one group
    (1500, 24, 96, 12, 3, 7, 4, 128),   # k = 24 in the multi-workgroup layout
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{s[0]}k{s[1]}E{s[2]}R{s[3]}m{s[6]}h{s[7]}" for s in SHAPES])
def test_group_shape_parity(epx, shape):
    T, k, E, R, H, s, m, hidden = shape
    rng = np.random.Generator(np.random.PCG64(T * 5 + k + m + hidden))
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, "zipf", 0.9)
    w = W.draw_gate_weights(rng, T, k)
    print(f"[group parity] shape {shape}", flush=True)
    run_group_case(epx, x, idx, w, E, R, H, s, m, str(shape))


def test_group_duplicate_ids_and_empty_batch(epx):
    rng = np.random.Generator(np.random.PCG64(77))
    T, k, E, R, m, hidden = 90, 6, 16, 4, 2, 128
    idx = rng.integers(0, E, (T, k)).astype(np.int32)          # duplicates in a row
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    w = W.draw_gate_weights(rng, T, k)
    run_group_case(epx, x, idx, w, E, R, 2, 0, m, "duplicates")
    p = epx.make_problem(0, 2, 16, 4, 2, 0, epx.MODE_PER_EXPERT, 2)
    L = epx.Layout(p)
    epx.epx_get_layout(p, torch.zeros((0, 2), dtype=torch.int32, device="cuda"), L)
    e = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    epx.epx_dispatch_group(p, L, 1, e, epx.BF16, e)
    epx.epx_combine_group(p, L, 1, e, torch.zeros((0, 2), dtype=torch.float32, device="cuda"),
                          torch.zeros((0, 64), dtype=torch.float32, device="cuda"), e)
    torch.cuda.synchronize()
    assert list(L["group_offset"].cpu().numpy()) == [0] * 9


def test_group_bad_ids_write_nothing(epx):
    T, k, E, R, m, hidden = 40, 4, 16, 4, 2, 64
    idx = np.zeros((T, k), np.int32)
    idx[:, 1] = np.arange(1, T + 1) % E
    idx[7, 2] = E + 3
    p = epx.make_problem(T, k, E, R, 2, 0, epx.MODE_PER_EXPERT, m)
    L = epx.Layout(p)
    epx.epx_get_layout(p, _dev(idx), L)
    assert epx.epx_read_error(L) == 1
    x = torch.ones((T, hidden), dtype=torch.bfloat16, device="cuda")
    recv = torch.full((T * k, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out = torch.full((T, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    carry = torch.zeros((T, hidden), dtype=torch.float32, device="cuda")
    for g in range(m):
        epx.epx_dispatch_group(p, L, g, x, epx.BF16, recv)
        epx.epx_combine_group(p, L, g, recv, torch.ones((T, k), dtype=torch.float32, device="cuda"), carry, out)
    torch.cuda.synchronize()
    assert np.all(_bits(recv) == np.uint16(SENTINEL_BF16 & 0xFFFF))
    assert np.all(_bits(out) == np.uint16(SENTINEL_BF16 & 0xFFFF))
