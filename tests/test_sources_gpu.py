"""Sixteen source ranks of the DeepEP rank-imbalance issue (2 machines x 8
ranks; 384 tokens per rank on machine 1 and 64 on machine 2, or 224
everywhere): each source's layout computed on the GPU with its own rank id
and token count, equal to the oracle's, and the receive counts an exchange
would deliver summed per destination rank: copies (rank_rows) and tokens
(rank_tokens, the one-copy-per-rank view), and relay rows per destination
host."""
import numpy as np
import pytest
import torch

import oracle
from combine_epx_get_amd import workloads as W
from tests.test_parity_gpu import _dev, assert_layout_parity, layout_np

pytestmark = pytest.mark.gpu

R, H, E, K = 16, 2, 256, 8


@pytest.fixture(scope="module")
def epx():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


@pytest.mark.parametrize("scenario", ["unbalanced", "balanced"])
def test_sixteen_sources(epx, scenario):
    tokens = [384] * 8 + [64] * 8 if scenario == "unbalanced" else [224] * 16
    rng = np.random.Generator(np.random.PCG64(250))
    recv_rows = np.zeros((R, R), np.int64)      # [src, dst] copies
    recv_tok = np.zeros((R, R), np.int64)       # [src, dst] tokens (one copy per rank)
    relay = np.zeros((R, H), np.int64)          # [src, dst host] relay rows
    print(f"[sources] {scenario}", flush=True)
    for src, T in enumerate(tokens):
        idx = W.draw_routing(rng, T, E, K, "uniform")
        p = epx.make_problem(T, K, E, R, H, src, epx.MODE_HOST_RELAY)
        L = epx.Layout(p)
        epx.epx_get_layout(p, _dev(idx), L)
        got = layout_np(epx, L, True)
        ora = oracle.layout(idx, E, R, H, src, relay=True)
        assert_layout_parity(got, ora, True, f"{scenario} src {src}")
        recv_rows[src] = got["rank_rows"]
        recv_tok[src] = got["rank_tokens"]
        relay[src] = got["host_tokens"]
        assert got["relay_dst_rank"].tolist() == [h * 8 + src % 8 for h in range(H)]
    # every copy and every token lands somewhere
    assert np.array_equal(recv_rows.sum(axis=1), np.array(tokens) * K)
    assert np.all(recv_tok <= recv_rows) and np.all(recv_tok.sum(axis=1) >= np.array(tokens))
    # a machine-2 rank: copies from machine 1 scatter around tokens * k / R each
    dst = 11
    from_m1 = recv_rows[:8, dst].sum()
    mean = sum(tokens[:8]) * K / R
    assert abs(from_m1 - mean) < 6 * np.sqrt(mean), (from_m1, mean)
    # relay rows to a host = tokens touching it; the own host included
    for src, T in enumerate(tokens):
        assert relay[src].sum() >= T and np.all(relay[src] <= T)
