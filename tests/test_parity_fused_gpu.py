"""GPU parity of the fused layout-and-dispatch call (epx_layout_dispatch).

Bar: bit-exact against the oracle (layout arrays, bf16 rows, fp8 codes and
scales) and, array by array, identical to epx_get_layout followed by
epx_dispatch on arrays pre-filled with the same sentinel, so that an entry
one path writes and the other leaves alone also fails. Decode batches of
the digest "Balancing and Beyond" (section 1: at most 128 tokens on a GPU;
section 5: 256 experts, top-8, hidden 7168) take the fused kernel; the
sizes past its limits (T > 1024, T*k > 4096, E > 512, LDS) take the two
launches inside the same call and must give the same results too.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_epx_get_amd import workloads as W
from tests.test_parity_gpu import (SENTINEL_BF16, SENTINEL_U8, _bf16_dev, _bits, _dev,
                                   assert_layout_parity, layout_np)

pytestmark = pytest.mark.gpu

FILL = -7   # layout sentinel: no layout entry holds it


@pytest.fixture(scope="module")
def epx():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


def _fresh_layout(epx, p):
    L = epx.Layout(p)
    for t in L.tensors.values():
        t.fill_(FILL)
    return L


def _recv(cap, hidden, dtype):
    if dtype == "bf16":
        return (torch.full((cap, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda")
                .view(torch.bfloat16), None)
    return (torch.full((cap, hidden), SENTINEL_U8, dtype=torch.uint8, device="cuda"),
            torch.full((cap, hidden // 128), -1.0, dtype=torch.float32, device="cuda"))


def run_fused(epx, x_bits, idx, E, R, H, s, relay, dtype, m=1, what=""):
    T, k = idx.shape
    hidden = x_bits.shape[1]
    mode = epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT
    p = epx.make_problem(T, k, E, R, H, s, mode, m)
    cap = epx.relay_capacity(p) if relay else T * k
    odt = epx.BF16 if dtype == "bf16" else epx.FP8_E4M3
    x_t, idx_t = _bf16_dev(x_bits), _dev(idx)

    # the two calls
    L1 = _fresh_layout(epx, p)
    r1, s1 = _recv(cap, hidden, dtype)
    epx.epx_get_layout(p, idx_t, L1)
    epx.epx_dispatch(p, L1, x_t, odt, r1, s1)
    # the fused call
    L2 = _fresh_layout(epx, p)
    r2, s2 = _recv(cap, hidden, dtype)
    epx.epx_layout_dispatch(p, idx_t, L2, x_t, odt, r2, s2)
    torch.cuda.synchronize()

    for name in L1.tensors:
        if name == "workspace":
            continue
        a, b = L1[name].cpu().numpy(), L2[name].cpu().numpy()
        bad = np.nonzero(a != b)[0]
        assert bad.size == 0, (what, name, int(bad[0]), int(a[bad[0]]), int(b[bad[0]]))
    if dtype == "bf16":
        assert np.array_equal(_bits(r1), _bits(r2)), (what, "bf16 rows")
    else:
        assert np.array_equal(r1.cpu().numpy(), r2.cpu().numpy()), (what, "fp8 codes")
        assert np.array_equal(s1.cpu().numpy().view(np.uint32), s2.cpu().numpy().view(np.uint32)), \
            (what, "fp8 scales")

    # and against the oracle
    if m == 1:
        ora = oracle.layout(idx, E, R, H, s, relay=relay)
        assert_layout_parity(layout_np(epx, L2, relay), ora, relay, what)
        rows = int(ora["totals"][1] if relay else ora["totals"][0])
        if dtype == "bf16":
            want = oracle.dispatch_bf16(x_bits, ora, k, H, relay)
            got = _bits(r2)
            assert np.array_equal(got[:rows], want), (what, "oracle bf16 rows")
            assert np.all(got[rows:] == np.uint16(SENTINEL_BF16 & 0xFFFF)), (what, "rows past the end")
        else:
            wq, ws = oracle.dispatch_fp8(x_bits, ora, k, H, relay)
            assert np.array_equal(r2.cpu().numpy()[:rows], wq), (what, "oracle fp8 codes")
            assert np.array_equal(s2.cpu().numpy()[:rows].view(np.uint32), ws.view(np.uint32)), \
                (what, "oracle fp8 scales")
    else:
        ora = oracle.layout_grouped(idx, E, R, m)
        got = layout_np(epx, L2, False)
        for n in ("expert_count", "expert_offset", "group_offset", "slot", "row_token"):
            assert np.array_equal(got[n], ora[n]), (what, n)
        if dtype == "bf16":
            assert np.array_equal(_bits(r2), x_bits[ora["row_token"]]), (what, "grouped rows")


DECODE = [("decode_uniform", "per_expert"), ("decode_skewed", "per_expert"),
          ("decode_skewed", "relay"), ("decode_skewed_s06", "relay"), ("tiny", "per_expert"),
          ("tiny", "relay"), ("rank_light", "per_expert"), ("rank_light", "relay"),
          ("rank_heavy", "per_expert"), ("rank_balanced", "relay"),
          # past the decode limits: count, scan and the assign-and-copy launch
          ("large_batch", "per_expert"), ("large_batch", "relay"), ("fp8_dispatch", "relay"),
          ("hybridep_bf16", "relay")]


@pytest.mark.parametrize("name,mode", DECODE)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_fused_workloads(epx, name, mode, dtype):
    w = W.WORKLOADS[name]
    d = W.make_inputs(w)
    print(f"[fused] {name} {mode} {dtype} T={d['T']}", flush=True)
    run_fused(epx, d["x"], d["topk_idx"], w.num_experts, w.num_ranks, w.num_hosts, w.my_rank,
              mode == "relay", dtype, what=f"{name}/{mode}/{dtype}")


SHAPES = [
    # T, k, E, R, H, s, hidden, routing
    (1, 1, 8, 8, 8, 5, 128, "uniform"),
    (2, 8, 256, 32, 4, 3, 7168, "zipf"),
    (63, 3, 12, 4, 2, 3, 136, "uniform"),
    (65, 8, 256, 32, 4, 7, 128, "zipf"),
    (130, 6, 6, 3, 1, 1, 264, "uniform"),        # k = E, one host
    (257, 2, 16, 16, 16, 15, 2048, "uniform"),   # one rank per host
    (50, 64, 64, 8, 4, 1, 128, "uniform"),       # largest k
    (512, 8, 512, 64, 8, 9, 256, "zipf"),        # T*k = 4096, E = 512: the fused limits
    (1024, 4, 64, 64, 64, 63, 128, "uniform"),   # T = 1024, 64 hosts
    (513, 8, 256, 32, 4, 2, 256, "uniform"),     # T*k > 4096: two launches
    (100, 4, 1024, 32, 4, 2, 128, "uniform"),    # E > 512: two launches
    (1025, 2, 16, 4, 2, 1, 128, "uniform"),      # T > 1024: two launches
    # past the decode limits (k <= 16) the call takes count, scan and one
    # assign-and-copy launch
    (4096, 8, 256, 16, 2, 3, 7168, "uniform"),   # the 4096-token batch
    (700, 8, 256, 32, 4, 1, 1024, "zipf"),       # column slices (T < 2048)
    (2000, 16, 2048, 64, 8, 5, 256, "zipf"),     # k = 16, E = 2048
    (4097, 1, 8, 2, 1, 0, 128, "uniform"),       # k = 1, ragged last chunk
    (3000, 5, 40, 8, 2, 3, 136, "uniform"),      # k = 5, hidden 136
    (600, 17, 64, 8, 2, 1, 128, "uniform"),      # k = 17: layout and dispatch launches
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{s[0]}k{s[1]}E{s[2]}R{s[3]}H{s[4]}h{s[6]}" for s in SHAPES])
@pytest.mark.parametrize("relay", [False, True])
def test_fused_shapes(epx, shape, relay):
    T, k, E, R, H, s, hidden, routing = shape
    rng = np.random.Generator(np.random.PCG64(T * 11 + k * 5 + hidden))
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, routing, 1.2)
    print(f"[fused] shape {shape} relay={relay}", flush=True)
    run_fused(epx, x, idx, E, R, H, s, relay, "bf16", what=f"{shape}/bf16")
    if hidden % 128 == 0:
        run_fused(epx, x, idx, E, R, H, s, relay, "fp8", what=f"{shape}/fp8")


@pytest.mark.parametrize("m", [2, 4, 8])
def test_fused_expert_groups(epx, m):
    rng = np.random.Generator(np.random.PCG64(40 + m))
    T, k, E, R, H, hidden = 128, 8, 256, 32, 4, 1024
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, "zipf", 1.2)
    print(f"[fused] groups m={m}", flush=True)
    run_fused(epx, x, idx, E, R, H, 5, False, "bf16", m=m, what=f"groups {m}")
    run_fused(epx, x, idx, E, R, H, 5, False, "fp8", m=m, what=f"groups {m}/fp8")


def test_fused_expert_groups_large(epx):
    """Past the decode limits, expert groups take the layout and dispatch
    launches inside the call."""
    rng = np.random.Generator(np.random.PCG64(44))
    T, k, E, R, H, hidden = 1500, 8, 256, 16, 2, 256
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, "uniform", 1.0)
    print("[fused] groups m=2, 1500 tokens", flush=True)
    run_fused(epx, x, idx, E, R, H, 3, False, "bf16", m=2, what="groups 2 large")
    run_fused(epx, x, idx, E, R, H, 3, False, "fp8", m=2, what="groups 2 large/fp8")


@pytest.mark.parametrize("relay", [False, True])
def test_fused_duplicate_ids(epx, relay):
    rng = np.random.Generator(np.random.PCG64(9))
    T, k, E, R, H, hidden = 300, 4, 16, 4, 2, 256
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    run_fused(epx, x, idx, E, R, H, 2, relay, "bf16", what="duplicates")
    run_fused(epx, x, idx, E, R, H, 2, relay, "fp8", what="duplicates/fp8")
    run_fused(epx, x, np.full((T, k), 11, np.int32), E, R, H, 1, relay, "bf16", what="one expert")


@pytest.mark.parametrize("relay", [False, True])
def test_fused_duplicate_ids_large(epx, relay):
    """Past the decode limits: many pairs of a token on one expert."""
    rng = np.random.Generator(np.random.PCG64(19))
    T, k, E, R, H, hidden = 2000, 8, 16, 4, 2, 256
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    run_fused(epx, x, idx, E, R, H, 3, relay, "bf16", what="duplicates large")
    run_fused(epx, x, idx, E, R, H, 3, relay, "fp8", what="duplicates large/fp8")
    run_fused(epx, x, np.full((T, k), 5, np.int32), E, R, H, 0, relay, "bf16", what="one expert large")


@pytest.mark.parametrize("relay", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_fused_out_of_range_ids_large(epx, relay, dtype):
    """Past the decode limits: bad ids are counted and nothing is copied."""
    T, k, E, R, H, hidden = 1000, 8, 64, 8, 2, 128
    rng = np.random.Generator(np.random.PCG64(23))
    idx = W.draw_routing(rng, T, E, k, "uniform", 1.0)
    idx[5, 3] = E
    idx[999, 7] = -2
    p = epx.make_problem(T, k, E, R, H, 0, epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT)
    cap = epx.relay_capacity(p) if relay else T * k
    L = _fresh_layout(epx, p)
    recv, sc = _recv(cap, hidden, dtype)
    epx.epx_layout_dispatch(p, _dev(idx), L, torch.ones((T, hidden), dtype=torch.bfloat16, device="cuda"),
                            epx.BF16 if dtype == "bf16" else epx.FP8_E4M3, recv, sc)
    assert epx.epx_read_error(L) == 2
    if dtype == "bf16":
        assert np.all(_bits(recv) == np.uint16(SENTINEL_BF16 & 0xFFFF))
    else:
        assert np.all(recv.cpu().numpy() == SENTINEL_U8) and np.all(sc.cpu().numpy() == -1.0)


@pytest.mark.parametrize("relay", [False, True])
def test_fused_out_of_range_ids(epx, relay):
    """Bad ids: totals[3] counts them, recv is not touched."""
    T, k, E, R, H, hidden = 100, 2, 16, 4, 2, 128
    idx = np.tile(np.array([[1, 2]], np.int32), (T, 1))
    idx[17, 1] = 16
    idx[90, 0] = -1
    idx[0, 0] = 1 << 30
    p = epx.make_problem(T, k, E, R, H, 0, epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT)
    cap = epx.relay_capacity(p) if relay else T * k
    for dtype in ("bf16", "fp8"):
        L = _fresh_layout(epx, p)
        recv, sc = _recv(cap, hidden, dtype)
        epx.epx_layout_dispatch(p, _dev(idx), L, torch.ones((T, hidden), dtype=torch.bfloat16, device="cuda"),
                                epx.BF16 if dtype == "bf16" else epx.FP8_E4M3, recv, sc)
        assert epx.epx_read_error(L) == 3   # the number of bad ids
        if dtype == "bf16":
            assert np.all(_bits(recv) == np.uint16(SENTINEL_BF16 & 0xFFFF))
        else:
            assert np.all(recv.cpu().numpy() == SENTINEL_U8) and np.all(sc.cpu().numpy() == -1.0)


def test_fused_empty_batch(epx):
    for relay in (False, True):
        p = epx.make_problem(0, 2, 16, 4, 2, 1, epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT)
        L = _fresh_layout(epx, p)
        x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
        recv = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
        epx.epx_layout_dispatch(p, torch.zeros((0, 2), dtype=torch.int32, device="cuda"), L, x, epx.BF16, recv)
        ora = oracle.layout(np.zeros((0, 2), np.int32), 16, 4, 2, 1, relay=relay)
        assert_layout_parity(layout_np(epx, L, relay), ora, relay, "empty")
