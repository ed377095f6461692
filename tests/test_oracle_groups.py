"""Pins of the oracle's expert groups for per-expert overlap (digest "Balancing
and Beyond", section 3.3 and Figure 4: the experts are split into 2 or 4
groups, each dispatched, computed and combined in turn, the whole batch in
every group).

* one group is the plain layout and the plain combine, bit for bit;
* rows are the brute-force sort of the pairs by (group, expert, token, j);
  block offsets count the pairs before each (group, rank) block;
* every rank has the same number of experts in every group, and the groups of
  a rank are contiguous ranges of its local experts (the reading that lets
  every GPU overlap);
* the group dispatches together write every row exactly once;
* the combine order (groups ascending, j ascending inside a group, float32
  carried) is fixed by two cases whose float32 results differ by order,
  with hand-computed expected values; float64 bound on random data.
"""
import numpy as np
import pytest

import oracle
from combine_epx_get_amd import workloads as W

SHAPES = [
    # T, k, E, R, m
    (1, 1, 4, 2, 2),
    (7, 3, 16, 4, 2),
    (33, 4, 32, 4, 4),
    (50, 8, 64, 8, 2),
    (20, 6, 24, 3, 4),
    (64, 8, 256, 16, 4),
    (9, 2, 8, 8, 1),
]


def _routing(shape, seed=0, dups=False):
    T, k, E, R, m = shape
    rng = np.random.Generator(np.random.PCG64(seed + T * 31 + E))
    if dups:
        return rng.integers(0, E, (T, k)).astype(np.int32)
    return W.draw_routing(rng, T, E, k, "zipf", 0.8)


def _group(e, epr, m):
    return (e % epr) // (epr // m)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dups", [False, True])
def test_grouped_layout_brute_force(shape, dups):
    T, k, E, R, m = shape
    idx = _routing(shape, dups=dups)
    lay = oracle.layout_grouped(idx, E, R, m)
    epr = E // R
    pairs = sorted(((_group(int(idx[t, j]), epr, m), int(idx[t, j]), t, j)
                    for t in range(T) for j in range(k)))
    want = np.zeros(T * k, np.int32)
    for row, (_, _, t, j) in enumerate(pairs):
        want[t * k + j] = row
    assert np.array_equal(lay["slot"], want)
    assert np.array_equal(lay["row_token"], np.array([p[2] for p in pairs], np.int32))
    assert np.array_equal(lay["expert_count"], np.bincount(idx.ravel(), minlength=E))
    # each (group, rank) block starts after the pairs of every earlier block
    for g in range(m):
        for r in range(R):
            before = sum(1 for p in pairs if (p[0], p[1] // epr) < (g, r))
            assert lay["group_offset"][g * R + r] == before
    assert lay["group_offset"][m * R] == T * k == lay["expert_offset"][E]
    # every expert's rows sit inside its (group, rank) block, in token order
    for e in range(E):
        g, r = _group(e, epr, m), e // epr
        lo, hi = lay["group_offset"][g * R + r], lay["group_offset"][g * R + r + 1]
        rows = np.arange(lay["expert_offset"][e], lay["expert_offset"][e] + lay["expert_count"][e])
        assert np.all((rows >= lo) & (rows < hi))
        assert np.all(np.diff(lay["row_token"][rows]) >= 0)


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_every_rank_has_every_group(m):
    E, R = 64, 8
    epr = E // R
    for r in range(R):
        local = [_group(e, epr, m) for e in range(r * epr, (r + 1) * epr)]
        assert [local.count(g) for g in range(m)] == [epr // m] * m
        assert local == sorted(local)             # contiguous ranges of local experts
    # and the oracle's blocks say the same: with one pair per expert every
    # (group, rank) block holds epr / m rows
    idx = np.arange(E, dtype=np.int32).reshape(E, 1)
    lay = oracle.layout_grouped(idx, E, R, m)
    assert np.all(np.diff(lay["group_offset"]) == epr // m)


@pytest.mark.parametrize("shape", [(40, 8, 64, 8, 1), (30, 4, 16, 4, 1), (5, 3, 9, 3, 1)])
def test_one_group_is_the_plain_layout_and_combine(shape):
    T, k, E, R, m = shape
    idx = _routing(shape, seed=3)
    plain = oracle.layout(idx, E, R, 1)
    lay = oracle.layout_grouped(idx, E, R, 1)
    for n in ("expert_count", "expert_offset", "slot", "row_token"):
        assert np.array_equal(lay[n], plain[n]), n
    assert np.array_equal(lay["group_offset"], plain["rank_offset"])
    assert np.array_equal(lay["totals"][[0, 2, 3]], plain["totals"][[0, 2, 3]])
    rng = np.random.Generator(np.random.PCG64(4))
    y = W.f32_to_bf16_bits(rng.standard_normal((T * k, 72), dtype=np.float32))
    w = W.draw_gate_weights(rng, T, k)
    assert np.array_equal(oracle.combine_grouped(y, lay, idx, w, E, R, 1), oracle.combine(y, plain, w))


@pytest.mark.parametrize("shape", SHAPES)
def test_group_dispatches_cover_every_row_once(shape):
    T, k, E, R, m = shape
    idx = _routing(shape, seed=5)
    lay = oracle.layout_grouped(idx, E, R, m)
    seen = np.zeros(T * k, np.int32)
    for g in range(m):
        sg = oracle.group_slots(idx, lay, E, R, m, g)
        hit = sg >= 0
        seen[sg[hit]] += 1
        lo, hi = lay["group_offset"][g * R], lay["group_offset"][(g + 1) * R]
        assert np.all((sg[hit] >= lo) & (sg[hit] < hi))    # a group's rows are one range
        assert np.array_equal(sg[hit], lay["slot"][hit])
    assert np.all(seen == 1)
    # the rows each group's dispatch writes are the token's row
    rng = np.random.Generator(np.random.PCG64(6))
    x = W.f32_to_bf16_bits(rng.standard_normal((T, 128), dtype=np.float32))
    full = np.zeros((T * k, 128), np.uint16)
    for g in range(m):
        rows = oracle.dispatch_group(x, lay, idx, E, R, m, g)
        sg = oracle.group_slots(idx, lay, E, R, m, g)
        written = np.zeros(T * k, bool)
        written[sg[sg >= 0]] = True
        assert not rows[~written].any()
        full[written] = rows[written]
    assert np.array_equal(full, x[lay["row_token"]])


def _bf16(v):
    return int(W.f32_to_bf16_bits(np.array([v], np.float32))[0])


def test_combine_order_cases():
    """E = 4 experts on one rank, m = 2: group 0 = experts {0, 1}, group 1 =
    {2, 3}. Unit weights; each pair's expert output is a constant row."""
    E, R, m = 4, 1, 2
    big = 2.0 ** 24
    # (a) j0 in group 1 (+1), j1 and j2 in group 0 (+2^24, -2^24).
    #     Group order: (2^24 - 2^24) + 1 = 1. Plain j order: 1 + 2^24 rounds
    #     to 2^24 (the tie goes to even), minus 2^24 = 0.
    # (b) j0 = +2^24 (g0), j1 = +1 (g1), j2 = +1 (g0), j3 = -2^24 (g1).
    #     Groups ascending: 2^24 + 1 -> 2^24, then + 1 -> 2^24, - 2^24 = 0.
    #     Groups descending would give (1 - 2^24) + 2^24 + 1 = 2.
    cases = [([2, 0, 1], [1.0, big, -big], 1.0, 0.0),
             ([0, 2, 1, 3], [big, 1.0, 1.0, -big], 0.0, 0.0)]
    for ids, vals, want_grouped, want_plain in cases:
        idx = np.array([ids], np.int32)
        k = len(ids)
        lay = oracle.layout_grouped(idx, E, R, m)
        y = np.zeros((k, 8), np.uint16)
        for j, v in enumerate(vals):
            y[lay["slot"][j]] = _bf16(v)
        w = np.ones((1, k), np.float32)
        got = oracle.combine_grouped(y, lay, idx, w, E, R, m)
        assert np.all(got == _bf16(want_grouped)), (ids, got[0, 0])
        assert np.all(oracle.combine(y, lay, w) == _bf16(want_plain))
    # (b) with the groups swapped (experts 2, 3 <-> 0, 1) is the descending
    #     order: 2
    idx = np.array([[2, 0, 3, 1]], np.int32)
    lay = oracle.layout_grouped(idx, E, R, m)
    y = np.zeros((4, 8), np.uint16)
    for j, v in enumerate([big, 1.0, 1.0, -big]):
        y[lay["slot"][j]] = _bf16(v)
    got = oracle.combine_grouped(y, lay, idx, np.ones((1, 4), np.float32), E, R, m)
    assert np.all(got == _bf16(2.0))


@pytest.mark.parametrize("shape", SHAPES[1:6])
def test_grouped_combine_within_float64_bound(shape):
    T, k, E, R, m = shape
    idx = _routing(shape, seed=8)
    lay = oracle.layout_grouped(idx, E, R, m)
    rng = np.random.Generator(np.random.PCG64(9))
    h = 64
    y = W.f32_to_bf16_bits(rng.standard_normal((T * k, h), dtype=np.float32))
    w = W.draw_gate_weights(rng, T, k)
    got = W.bf16_bits_to_f32(oracle.combine_grouped(y, lay, idx, w, E, R, m)).astype(np.float64)
    yf = W.bf16_bits_to_f32(y).astype(np.float64)
    exact = np.einsum("tk,tkh->th", w.astype(np.float64), yf[lay["slot"].reshape(T, k)])
    absum = np.einsum("tk,tkh->th", np.abs(w.astype(np.float64)), np.abs(yf[lay["slot"].reshape(T, k)]))
    # k float32 fmas (each within 2^-24 of the running sum, so the chain is
    # within about k * 2^-24 * sum |w y|), then one bf16 rounding (half an ulp,
    # at most 2^-8 of the value it rounds)
    chain = 1.01 * k * 2.0 ** -24 * absum
    bound = chain + 2.0 ** -8 * (np.abs(exact) + chain)
    assert np.all(np.abs(got - exact) <= bound)


def test_grouped_bad_geometry():
    idx = np.zeros((2, 2), np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.layout_grouped(idx, 12, 2, 4)      # 6 experts per rank, 4 groups
    with pytest.raises(oracle.OracleError):
        oracle.layout_grouped(np.full((2, 2), 99, np.int32), 16, 2, 2)
