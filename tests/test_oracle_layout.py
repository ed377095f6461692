"""Pins of the oracle's layout against what the pages and the definitions fix.

Independent checks (none re-runs the oracle's own algorithm):
  * brute force: every position is recounted from its definition by
    enumerating all pairs (O((T*k)^2), pure Python) on small inputs;
  * invariants that any correct layout satisfies, at full sizes;
  * the copy-count closed forms of the digest "Balancing and Beyond", section
    3.2, by Monte Carlo, and the values the digest prints for EP32;
  * the worked example of the DeepEP issue "[GH-ISSUE #250] Profiling when
    rank unbalance" (receive counts 192 / 28 / 220 and 210 / 112).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from combine_epx_get_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- brute force
def brute_layout(idx, E, R, H, s):
    """Every output recounted from its definition, pair by pair."""
    idx = [list(map(int, row)) for row in idx]
    T = len(idx)
    k = len(idx[0]) if T else 0
    epr, rph = E // R, R // H
    pairs = [(t, j, idx[t][j]) for t in range(T) for j in range(k)]
    rank = lambda e: e // epr
    host = lambda e: e // epr // rph
    out = {}
    out["expert_count"] = [sum(1 for (_, _, e) in pairs if e == x) for x in range(E)]
    out["expert_offset"] = [sum(1 for (_, _, e) in pairs if e < x) for x in range(E + 1)]
    out["rank_rows"] = [sum(1 for (_, _, e) in pairs if rank(e) == r) for r in range(R)]
    out["rank_offset"] = [sum(1 for (_, _, e) in pairs if rank(e) < r) for r in range(R + 1)]
    out["rank_tokens"] = [len({t for (t, _, e) in pairs if rank(e) == r}) for r in range(R)]
    out["host_tokens"] = [len({t for (t, _, e) in pairs if host(e) == h}) for h in range(H)]
    hosts_of = [sorted({host(e) for e in idx[t]}) for t in range(T)]
    out["host_offset"] = [sum(1 for t in range(T) for g in hosts_of[t] if g < h) for h in range(H + 1)]
    # row of (t, j): pairs of smaller expert id, plus earlier pairs of the same
    # expert in (token, position) order
    slot = []
    for (t, j, e) in pairs:
        before = sum(1 for (t2, j2, e2) in pairs if e2 < e)
        same = sum(1 for (t2, j2, e2) in pairs if e2 == e and (t2, j2) < (t, j))
        slot.append(before + same)
    out["slot"] = slot
    row_token = [None] * len(pairs)
    for p, (t, j, e) in enumerate(pairs):
        row_token[slot[p]] = t
    out["row_token"] = row_token
    # relay rows: all (host, token) with the token touching the host, sorted
    rows = sorted((h, t) for t in range(T) for h in hosts_of[t])
    relay_slot = [rows.index((h, t)) if (h, t) in set(rows) else -1
                  for t in range(T) for h in range(H)]
    out["relay_slot"] = relay_slot
    cap = T * min(k, H)
    out["relay_token"] = [t for (h, t) in rows] + [-1] * (cap - len(rows))
    fan = []
    masks = []
    for (h, t) in rows:
        fan += [e if host(e) == h else -1 for e in idx[t]]
        masks.append(sum(set(1 << (rank(e) % rph) for e in idx[t] if host(e) == h)))
    out["fanout_expert"] = fan + [-1] * ((cap - len(rows)) * k)
    out["fanout_rank_mask"] = masks + [0] * (cap - len(rows))
    out["relay_dst_rank"] = [h * rph + s % rph for h in range(H)]
    out["totals"] = [T * k, len(rows), max(out["expert_count"]) if E else 0, 0]
    return out


def assert_layout_equal(got, want, keys=None):
    for name in keys or want:
        g = np.asarray(got[name]).astype(np.int64).ravel()
        w = np.asarray(want[name], dtype=np.int64).ravel()
        assert g.shape == w.shape, (name, g.shape, w.shape)
        assert np.array_equal(g, w), (name, g[:16], w[:16])


SMALL_SHAPES = [
    # T, k, E, R, H, s, routing
    (64, 2, 16, 4, 2, 0, "uniform"),      # the tiny workload's geometry
    (0, 2, 16, 4, 2, 0, "uniform"),       # empty batch
    (1, 3, 12, 4, 2, 3, "uniform"),
    (17, 1, 8, 8, 8, 5, "uniform"),       # k = 1, one expert per rank, one rank per host
    (9, 6, 6, 3, 1, 1, "uniform"),        # k = E, single host
    (33, 4, 32, 8, 4, 6, "zipf"),
    (40, 3, 24, 6, 3, 4, "zipf"),
    (5, 2, 4, 4, 2, 1, "uniform"),
]


@pytest.mark.parametrize("shape", SMALL_SHAPES)
@pytest.mark.parametrize("relay", [False, True])
def test_layout_matches_brute_force(shape, relay):
    T, k, E, R, H, s, routing = shape
    rng = np.random.Generator(np.random.PCG64(T * 131 + k))
    idx = W.draw_routing(rng, T, E, k, routing, 1.1) if T else np.zeros((0, k), np.int32)
    got = oracle.layout(idx, E, R, H, s, relay=relay)
    want = brute_layout(idx, E, R, H, s)
    keys = ["expert_count", "expert_offset", "rank_rows", "rank_offset", "rank_tokens",
            "host_tokens", "host_offset", "slot", "row_token", "relay_dst_rank", "totals"]
    if relay:
        keys += ["relay_slot", "relay_token", "fanout_expert", "fanout_rank_mask"]
    else:
        want["totals"][1] = sum(want["host_tokens"])
    assert_layout_equal(got, want, keys)


@pytest.mark.parametrize("case", ["one_expert", "duplicates", "random_with_dups"])
def test_layout_degenerate_routing(case):
    """All tokens on one expert; the same expert twice in one token's row
    (allowed: one row per pair, its host counted once)."""
    T, k, E, R, H, s = 23, 4, 16, 4, 2, 2
    rng = np.random.Generator(np.random.PCG64(7))
    if case == "one_expert":
        idx = np.full((T, k), 9, np.int32)
    elif case == "duplicates":
        idx = np.tile(np.array([[3, 3, 12, 3]], np.int32), (T, 1))
    else:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    got = oracle.layout(idx, E, R, H, s, relay=True)
    want = brute_layout(idx, E, R, H, s)
    assert_layout_equal(got, want)


def test_layout_rejects_out_of_range_ids():
    idx = np.array([[0, 5], [16, 2], [-1, 3]], np.int32)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.layout(idx, 16, 4, 2, 0)
    assert ei.value.code == 2


@pytest.mark.parametrize("geom", [(10, 2, 16, 3, 1, 0), (10, 2, 16, 4, 3, 0), (10, 17, 16, 4, 2, 0),
                                  (10, 2, 16, 4, 2, 4), (10, 0, 16, 4, 2, 0)])
def test_layout_rejects_bad_geometry(geom):
    T, k, E, R, H, s = geom
    idx = np.zeros((T, max(k, 1)), np.int32)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.layout(idx[:, :k] if k else idx[:, :0], E, R, H, s)
    assert ei.value.code == 1


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("name", ["decode_uniform", "decode_skewed", "large_batch", "fp8_dispatch"])
def test_layout_invariants_full_size(name):
    w = W.WORKLOADS[name]
    d = W.make_inputs(w)
    idx = d["topk_idx"]
    T, k = idx.shape
    lay = oracle.layout(idx, w.num_experts, w.num_ranks, w.num_hosts, w.my_rank, relay=True)
    # counts sum to T*k; bytes per direction are T*k*h*2 (digest section 1)
    assert lay["expert_count"].sum() == T * k == lay["totals"][0]
    assert lay["totals"][0] * w.hidden * 2 == T * k * w.hidden * 2
    # slots: a permutation of [0, T*k), increasing with token inside each expert
    slot = lay["slot"].reshape(T, k)
    assert np.array_equal(np.sort(slot.ravel()), np.arange(T * k))
    e_of = oracle.expert_of_rows(lay)
    assert np.array_equal(e_of[slot], idx)
    assert np.array_equal(lay["row_token"][slot], np.repeat(np.arange(T), k).reshape(T, k))
    rt = lay["row_token"]
    same = e_of[1:] == e_of[:-1]
    assert np.all(rt[1:][same] >= rt[:-1][same])
    # relay rows per token = its number of distinct hosts (glossary, "De-redundancy")
    epr, rph = w.experts_per_rank, w.ranks_per_host
    hosts = idx // epr // rph
    distinct = np.array([len(set(r)) for r in hosts])
    assert lay["host_tokens"].sum() == distinct.sum() == lay["totals"][1]
    rs = lay["relay_slot"].reshape(T, w.num_hosts)
    assert np.array_equal((rs >= 0).sum(1), distinct)
    used = rs[rs >= 0]
    assert np.array_equal(np.sort(used), np.arange(distinct.sum()))
    # imbalance ratio = max expert count / mean expert count (digest section 2)
    ratio = lay["totals"][2] / (T * k / w.num_experts)
    assert ratio >= 1.0
    assert lay["totals"][2] == lay["expert_count"].max()


# ---------------------------------------------------------------- closed forms
def _c2(E, k, H):
    return (H - 1) * (1 - math.comb(E - E // H, k) / math.comb(E, k))


def test_copy_count_formula_matches_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "copy_counts.json")))["deepseek_r1_ep32"]
    E, k, H = g["E"], g["k"], g["H"]
    c1 = k * (H - 1) / H
    c2 = _c2(E, k, H)
    assert c1 == g["c1_printed"]
    assert abs(c2 - g["c2_printed_approx"]) < 0.05
    assert round(100 * (1 - c2 / c1)) == g["fewer_network_bytes_printed_pct"]


@pytest.mark.parametrize("E,k,R,H", [(256, 8, 32, 4), (256, 8, 16, 2), (160, 8, 32, 4), (64, 4, 8, 8)])
def test_copy_counts_monte_carlo(E, k, R, H):
    """Oracle counts agree with c0, c1, c2 (digest section 3.2) for uniform routing."""
    T = 20000
    rng = np.random.Generator(np.random.PCG64(E + k + R + H))
    idx = W.draw_routing(rng, T, E, k, "uniform")
    s = 1
    lay = oracle.layout(idx, E, R, H, s)
    rph = R // H
    my_host = s // rph
    c0 = (T * k - lay["rank_rows"][s]) / T
    c1 = (T * k - lay["rank_rows"][my_host * rph:(my_host + 1) * rph].sum()) / T
    c2 = (lay["host_tokens"].sum() - lay["host_tokens"][my_host]) / T
    all_hosts = lay["host_tokens"].sum() / T
    # per-token values lie in [0, k]; standard error <= k / (2 sqrt(T))
    tol = 4 * k / (2 * math.sqrt(T))
    assert abs(c0 - k * (1 - 1 / R)) < tol
    assert abs(c1 - k * (H - 1) / H) < tol
    tol_h = 4 * (H - 1) / (2 * math.sqrt(T)) + 1e-12
    assert abs(c2 - _c2(E, k, H)) < tol_h
    assert abs(all_hosts - H * (1 - math.comb(E - E // H, k) / math.comb(E, k))) < 4 * H / (2 * math.sqrt(T))


def test_rank_imbalance_worked_example():
    """Receive/send token counts of the worked example, built as the sum of
    16 single-source layouts (k = 1, every source spreads its tokens evenly)."""
    g = json.load(open(os.path.join(GOLDEN, "p1_worked_example.json")))
    R, H, E = 16, 2, 16
    rph = R // H

    def recv_matrix(n_tokens):
        m = np.zeros((R, R), np.int64)      # m[src, dst] tokens
        for src in range(R):
            n = n_tokens[src]
            idx = (np.arange(n) % R).astype(np.int32).reshape(n, 1)
            lay = oracle.layout(idx, E, R, H, src)
            m[src] = lay["rank_tokens"]
        return m

    ub = g["unbalanced"]
    n = [ub["tokens_per_rank_machine1"]] * rph + [ub["tokens_per_rank_machine2"]] * rph
    m = recv_matrix(n)
    dst = rph + 3                           # some rank of machine 2
    from_m1 = m[:rph, dst].sum()
    from_m2 = sum(m[src, dst] for src in range(rph, R) if src != dst)
    assert from_m1 == ub["recv_from_machine1"]
    assert from_m2 == ub["recv_from_machine2_peers"]
    assert from_m1 + from_m2 == ub["recv_total"]
    assert m[2, rph:].sum() == ub["send_over_rdma_per_machine1_rank"]

    bal = g["balanced"]
    m = recv_matrix([bal["tokens_per_rank"]] * R)
    assert sum(m[src, dst] for src in range(R) if src != dst) == bal["recv_total_from_others"]
    assert m[:rph, dst].sum() == bal["recv_over_rdma"]
    assert m[2, rph:].sum() == bal["send_over_rdma_per_rank"]


def test_imbalance_ratio_constructed():
    """All k*T copies on k experts out of E gives the ratio E/k; uniform
    round-robin gives exactly 1."""
    T, k, E, R, H = 32, 4, 64, 8, 2
    idx = np.tile(np.array([[5, 17, 40, 63]], np.int32), (T, 1))
    lay = oracle.layout(idx, E, R, H, 0)
    assert lay["totals"][2] / (T * k / E) == E / k
    idx = (np.arange(T * k) % E).astype(np.int32).reshape(T, k)
    lay = oracle.layout(idx, E, R, H, 0)
    assert lay["totals"][2] / (T * k / E) == 1.0    # 128 copies over 64 experts: 2 each


def test_relay_rows_reproduce_the_hybridep_rdma_counter():
    """The HybridEP log prints 117.11 MB of RDMA sends per rank for its BF16
    dispatch (4096 tokens, hidden 7168, top-8, 128 experts on 16 ranks over 2
    nodes). One bf16 row per (token, destination host), the token's own host
    included, reproduces it; remote hosts alone would give half."""
    g = json.load(open(os.path.join(GOLDEN, "hybridep_bf16_counters.json")))
    T, k, E, R, H, h = g["tokens"], g["topk"], g["num_experts"], g["num_ranks"], g["num_hosts"], g["hidden"]
    rng = np.random.Generator(np.random.PCG64(590))
    idx = W.draw_routing(rng, T, E, k, "uniform")
    lay = oracle.layout(idx, E, R, H, 0, relay=True)
    rows = int(lay["totals"][1])
    assert rows == int(lay["host_tokens"].sum())
    mb = rows * h * 2 / 1e6
    assert abs(mb - g["rdma_send_MB"]) / g["rdma_send_MB"] < 0.005, mb
    remote_only = rows - T + int(np.sum(~np.any(idx // (E // R) // (R // H) == 0, axis=1)))
    assert abs(remote_only * h * 2 / 1e6 - g["rdma_send_MB"] / 2) / (g["rdma_send_MB"] / 2) < 0.01


# ---------------------------------------------------------------- property sweep
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402


@st.composite
def _geometry_and_routing(draw):
    """Small geometries across the edge cases: T = 0 or 1, k = 1 or k = E,
    E = R, H = 1, H = R, one expert for every pair, repeated ids in a row."""
    H = draw(st.integers(1, 4))
    rph = draw(st.integers(1, 3))
    R = H * rph
    epr = draw(st.integers(1, 3))
    E = R * epr
    k = draw(st.integers(1, min(E, 5)))
    T = draw(st.integers(0, 12))
    s = draw(st.integers(0, R - 1))
    kind = draw(st.sampled_from(["any", "one_expert", "distinct"]))
    if kind == "one_expert":
        e = draw(st.integers(0, E - 1))
        idx = [[e] * k for _ in range(T)]
    elif kind == "distinct":
        idx = [draw(st.permutations(list(range(E))))[:k] for _ in range(T)]
    else:
        idx = [[draw(st.integers(0, E - 1)) for _ in range(k)] for _ in range(T)]
    return np.array(idx, np.int32).reshape(T, k), E, R, H, s


@settings(max_examples=150, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(_geometry_and_routing())
def test_layout_property_sweep(case):
    idx, E, R, H, s = case
    got = oracle.layout(idx, E, R, H, s, relay=True)
    want = brute_layout(idx, E, R, H, s)
    assert_layout_equal(got, want, ["expert_count", "expert_offset", "rank_rows", "rank_offset",
                                    "rank_tokens", "host_tokens", "host_offset", "slot", "row_token",
                                    "relay_dst_rank", "totals", "relay_slot", "relay_token",
                                    "fanout_expert", "fanout_rank_mask"])
