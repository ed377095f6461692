"""Pins of the oracle's per-step intra-host swap planner (digest "Balancing
and Beyond", section 3.1 and Figure 2(b)).

* the worked example of Figure 2(b): loads 160 / 100 become 130 / 130 by
  swapping e0 (60 tokens) with e1 (30), accepted for tau <= 30 only;
* every recorded swap is optimal among all single swaps of its pair
  (enumerated here independently), with the stated tie rule;
* pairs are i-th heaviest with i-th lightest in each host;
* loads and experts are conserved within each host; tau is honoured.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_figure_example():
    g = json.load(open(os.path.join(GOLDEN, "swap_example.json")))
    counts, se = np.array(g["counts"]), np.array(g["slot_expert"])
    r = oracle.plan_swaps(counts, g["ranks"], g["hosts"], 30, se)
    assert list(r["load_before"]) == [g["before"]["G0"], g["before"]["G1"]]
    assert list(r["load_after"]) == [g["after"]["G0"], g["after"]["G1"]]
    heavy, ea, light, eb, old, new, applied = r["swaps"][0]
    assert (heavy, light) == (0, 1)
    assert counts[ea] == g["before"]["e0"] and counts[eb] == g["before"]["e1"]
    assert (old, new, applied) == (160, 130, 1)
    # the maximum falls by 30: a threshold of 31 rejects the swap
    r2 = oracle.plan_swaps(counts, g["ranks"], g["hosts"], 31, se)
    assert r2["swaps"][0][6] == 0
    assert np.array_equal(r2["slot_expert"], se)
    assert np.array_equal(r2["load_after"], r2["load_before"])


def _random_case(seed, E, R, H, skew=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    counts = (rng.pareto(1.2, E) * 20).astype(np.int32) if skew else rng.integers(0, 50, E).astype(np.int32)
    se = np.arange(E, dtype=np.int32)
    for h in range(H):      # shuffle experts among the host's slots
        lo, hi = h * (E // H), (h + 1) * (E // H)
        se[lo:hi] = rng.permutation(se[lo:hi])
    return counts, se


CASES = [(1, 16, 4, 1), (2, 64, 8, 2), (3, 256, 32, 4), (4, 48, 12, 2), (5, 40, 8, 8), (6, 30, 6, 2)]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("tau", [0, 5, 40])
def test_swaps_optimal_and_consistent(case, tau):
    seed, E, R, H = case
    counts, se = _random_case(seed, E, R, H)
    r = oracle.plan_swaps(counts, R, H, tau, se)
    epr, rph = E // R, R // H
    load = np.array([counts[se[i * epr:(i + 1) * epr]].sum() for i in range(R)])
    assert np.array_equal(r["load_before"], load)
    for h in range(H):
        ranks = list(range(h * rph, (h + 1) * rph))
        order = sorted(ranks, key=lambda q: (-load[q], q))
        for p in range(rph // 2):
            rec = r["swaps"][h * (rph // 2) + p]
            A, B = order[p], order[rph - 1 - p]
            assert (rec[0], rec[2]) == (A, B)
            # every single swap of the pair, enumerated
            best = None
            for a, b in itertools.product(range(epr), range(epr)):
                ca, cb = counts[se[A * epr + a]], counts[se[B * epr + b]]
                m = max(load[A] - ca + cb, load[B] - cb + ca)
                if best is None or m < best[0]:
                    best = (m, a, b)
            m, a, b = best
            assert rec[5] == m and rec[1] == se[A * epr + a] and rec[3] == se[B * epr + b]
            old = max(load[A], load[B])
            assert rec[4] == old
            assert rec[6] == int(old - m > 0 and old - m >= tau)
        # conservation inside the host
        sl = slice(h * rph * epr, (h + 1) * rph * epr)
        assert sorted(r["slot_expert"][sl]) == sorted(se[sl])
        assert r["load_after"][ranks].sum() == load[ranks].sum()
    after = np.array([counts[r["slot_expert"][i * epr:(i + 1) * epr]].sum() for i in range(R)])
    assert np.array_equal(r["load_after"], after)


def test_degenerate_cases():
    # one rank per host: no pairs, nothing moves
    counts = np.arange(16, dtype=np.int32)
    r = oracle.plan_swaps(counts, 4, 4, 0)
    assert r["swaps"].size == 0 and np.array_equal(r["slot_expert"], np.arange(16))
    # equal loads: no swap lowers the maximum
    r = oracle.plan_swaps(np.full(32, 7, np.int32), 8, 2, 0)
    assert np.all(r["swaps"][:, 6] == 0)
    # odd ranks per host: the middle rank stays unpaired
    counts, se = _random_case(9, 30, 6, 2)
    r = oracle.plan_swaps(counts, 6, 2, 0, se)
    assert r["swaps"].shape == (2, 7)


def test_bad_slot_ids_leave_only_their_host_unplanned():
    """A host whose slots hold an id outside [0, E) is not planned (slots
    copied, loads and records -1, applied 0, host_bad = the count); every
    other host's plan equals its plan on a valid placement, since hosts are
    planned independently (each pair stays inside one host)."""
    rng = np.random.Generator(np.random.PCG64(17))
    E, R, H = 64, 8, 4
    counts = rng.integers(0, 200, size=E).astype(np.int32)
    se = np.arange(E, dtype=np.int32)
    bad = se.copy()
    bad[E // H + 2] = E
    bad[E // H + 9] = -5
    got = oracle.plan_swaps(counts, R, H, 0, bad)
    want = oracle.plan_swaps(counts, R, H, 0, se)
    assert list(got["host_bad"]) == [0, 2, 0, 0] and not want["host_bad"].any()
    rph, npair, nslot = R // H, (R // H) // 2, E // H
    for h in range(H):
        s_, r_, q_ = (slice(h * nslot, (h + 1) * nslot), slice(h * rph, (h + 1) * rph),
                      slice(h * npair, (h + 1) * npair))
        if h == 1:
            assert np.array_equal(got["slot_expert"][s_], bad[s_])
            assert np.all(got["load_before"][r_] == -1) and np.all(got["load_after"][r_] == -1)
            assert np.all(got["swaps"][q_][:, :6] == -1) and np.all(got["swaps"][q_][:, 6] == 0)
        else:
            for n, sl in (("slot_expert", s_), ("load_before", r_), ("load_after", r_), ("swaps", q_)):
                assert np.array_equal(got[n][sl], want[n][sl]), (h, n)
