"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact for the layout, relay indices, bf16 rows, fp8 codes and
scales; combine bit-exact as designed (same fma order as the oracle) and, as
the stated gate, |gpu - oracle| <= 1e-2 + 4e-3 |oracle| elementwise.

Expert outputs feeding combine follow the stand-in expert rule
y = bf16(dispatched row * (1 + e/16)), built on the CPU from the oracle's
dispatch so both combines read the same bytes.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_epx_get_amd import workloads as W

pytestmark = pytest.mark.gpu

SENTINEL_BF16 = 0x7FBF   # a NaN pattern no valid output row can hold
SENTINEL_U8 = 0xA5


@pytest.fixture(scope="module")
def epx():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


def _dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def _bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return _dev(bits.view(np.int16), torch.bfloat16)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def layout_np(epx, L, relay):
    out = {}
    for name in epx.LAYOUT_FIELDS:
        if name == "workspace" or (name in epx.RELAY_FIELDS and not relay):
            continue
        a = L[name].cpu().numpy()
        out[name] = a.view(np.uint32) if name == "fanout_rank_mask" else a
    return out


def assert_layout_parity(got, want, relay, what=""):
    names = ["expert_count", "expert_offset", "rank_rows", "rank_tokens", "rank_offset",
             "host_tokens", "host_offset", "slot", "row_token", "relay_dst_rank", "totals"]
    if relay:
        names += ["relay_slot", "relay_token", "fanout_expert", "fanout_rank_mask"]
    for n in names:
        g, w = got[n], want[n]
        assert g.shape == w.shape, (what, n, g.shape, w.shape)
        bad = np.nonzero(g.astype(np.int64) != w.astype(np.int64))[0]
        assert bad.size == 0, (what, n, int(bad[0]), g[bad[0]], w[bad[0]], bad.size)
    if "group_offset" in got and "group_offset" not in want:   # one group: the rank offsets
        assert np.array_equal(got["group_offset"], want["rank_offset"]), (what, "group_offset")


def expert_outputs(tok_rows_f32: np.ndarray, idx: np.ndarray, slot: np.ndarray) -> np.ndarray:
    """y[slot[t, j]] = bf16(row_t * (1 + idx[t, j]/16)) (float32 product, then bf16)."""
    T, k = idx.shape
    y = np.empty((T * k, tok_rows_f32.shape[1]), np.uint16)
    s = slot.reshape(T, k)
    for j in range(k):
        fac = (1.0 + idx[:, j].astype(np.float32) / np.float32(16.0)).astype(np.float32)
        y[s[:, j]] = W.f32_to_bf16_bits(tok_rows_f32 * fac[:, None])
    return y


def check_combine(got_bits, want_bits, what=""):
    g = W.bf16_bits_to_f32(got_bits).astype(np.float64)
    r = W.bf16_bits_to_f32(want_bits).astype(np.float64)
    err = np.abs(g - r)
    assert np.all(err <= 1e-2 + 4e-3 * np.abs(r)), (what, float(err.max()))
    mism = int(np.count_nonzero(got_bits != want_bits))
    assert mism == 0, (what, "non-identical bf16 elements", mism)


def run_case(epx, x_bits, idx, w, E, R, H, s, relay, dtype, what=""):
    """Layout + dispatch + combine on the GPU, each compared with the oracle."""
    T, k = idx.shape
    hidden = x_bits.shape[1]
    ora = oracle.layout(idx, E, R, H, s, relay=relay)
    p = epx.make_problem(T, k, E, R, H, s, epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT)
    L = epx.Layout(p)
    epx.epx_get_layout(p, _dev(idx), L)
    assert epx.epx_read_error(L) == 0
    got = layout_np(epx, L, relay)
    assert_layout_parity(got, ora, relay, what)

    rows = int(ora["totals"][1] if relay else ora["totals"][0])
    cap = epx.relay_capacity(p) if relay else T * k
    x_t = _bf16_dev(x_bits)
    if dtype == "bf16":
        recv = torch.full((cap, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        epx.epx_dispatch(p, L, x_t, epx.BF16, recv)
        want = oracle.dispatch_bf16(x_bits, ora, k, H, relay)
        gb = _bits(recv)
        assert np.array_equal(gb[:rows], want), (what, "bf16 rows")
        assert np.all(gb[rows:] == SENTINEL_BF16), (what, "rows past the end were written")
        tok_rows = W.bf16_bits_to_f32(x_bits)
    else:
        recv = torch.full((cap, hidden), SENTINEL_U8, dtype=torch.uint8, device="cuda")
        scales = torch.full((cap, hidden // 128), -1.0, dtype=torch.float32, device="cuda")
        epx.epx_dispatch(p, L, x_t, epx.FP8_E4M3, recv, scales)
        wq, ws = oracle.dispatch_fp8(x_bits, ora, k, H, relay)
        gq = recv.cpu().numpy()
        gs = scales.cpu().numpy()
        bad = np.nonzero(gq[:rows] != wq)
        assert bad[0].size == 0, (what, "fp8 codes", bad[0][:4], bad[1][:4])
        assert np.array_equal(gs[:rows].view(np.uint32), ws.view(np.uint32)), (what, "fp8 scales")
        assert np.all(gq[rows:] == SENTINEL_U8) and np.all(gs[rows:] == -1.0)
        # the stand-in experts see the dequantised rows fl32(code * scale)
        first = (ora["relay_slot"].reshape(T, H).max(1) if relay else ora["slot"].reshape(T, k)[:, 0])
        deq = oracle.e4m3_to_f32(wq[first]).reshape(T, hidden // 128, 128)
        tok_rows = (deq * ws[first][:, :, None]).astype(np.float32).reshape(T, hidden)

    y = expert_outputs(tok_rows, idx, ora["slot"])
    out = torch.full((T, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    epx.epx_combine(p, L, _bf16_dev(y), _dev(w), out)
    want_out = oracle.combine(y, ora, w)
    check_combine(_bits(out), want_out, what)
    return ora


# ---------------------------------------------------------------- the workloads
CASES = []
for _name, _w in W.WORKLOADS.items():
    for _mode in _w.modes:
        for _dt in _w.dtypes:
            CASES.append((_name, _mode, _dt))
CASES.append(("tiny", "per_expert", "fp8"))
CASES.append(("decode_skewed", "relay", "fp8"))
CASES.append(("large_batch", "relay", "bf16"))


@pytest.mark.parametrize("name,mode,dtype", CASES)
def test_workload_parity(epx, name, mode, dtype):
    w = W.WORKLOADS[name]
    d = W.make_inputs(w)
    print(f"[parity] {name} {mode} {dtype} T={d['T']} h={w.hidden}", flush=True)
    run_case(epx, d["x"], d["topk_idx"], d["topk_weights"], w.num_experts, w.num_ranks,
             w.num_hosts, w.my_rank, mode == "relay", dtype, f"{name}/{mode}/{dtype}")


# ---------------------------------------------------------------- ragged and edge shapes
SHAPES = [
    # T, k, E, R, H, s, hidden, routing
    (1, 1, 8, 8, 8, 5, 8, "uniform"),
    (63, 3, 12, 4, 2, 3, 136, "uniform"),
    (65, 8, 256, 32, 4, 7, 128, "zipf"),
    (130, 6, 6, 3, 1, 1, 264, "uniform"),       # k = E, one host
    (200, 4, 32, 8, 4, 6, 1000, "zipf"),
    (257, 2, 16, 16, 16, 15, 2048, "uniform"),  # one rank per host
    (1000, 8, 256, 32, 4, 0, 7168, "zipf"),
    (4097, 8, 160, 32, 4, 9, 512, "uniform"),   # 160 experts, one token past 64 chunks
    (3000, 16, 2048, 64, 2, 33, 256, "uniform"),  # largest E, 32 ranks per host
    (50, 64, 64, 8, 4, 1, 128, "uniform"),      # largest k
    (5000, 8, 256, 256, 64, 200, 128, "uniform"),  # 64 hosts, 1 expert per rank
    (200, 32, 64, 8, 4, 2, 136, "zipf"),        # k > 16 in the multi-workgroup layout (32-token chunks)
    (100, 64, 128, 16, 8, 3, 128, "uniform"),   # k = 64 there: 16-token chunks, assign sums columns
    (1500, 24, 96, 12, 3, 7, 128, "zipf"),      # k = 24: 42-token chunks, 36 workgroups
    (8200, 8, 256, 32, 4, 5, 128, "zipf"),      # 65 600 pairs: 257 chunk workgroups, a ragged last chunk
    (8192, 8, 256, 16, 2, 3, 128, "uniform"),   # 65 536 pairs: 256 full chunks
    (2051, 6, 48, 6, 3, 4, 1000, "zipf"),       # relay to 3 hosts, a wave per token, 3 tokens in the last workgroup
    (2049, 2, 8, 4, 1, 1, 7168, "uniform"),     # relay to 1 host, a wave per token, 1 token in the last workgroup
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{s[0]}k{s[1]}E{s[2]}R{s[3]}H{s[4]}h{s[6]}" for s in SHAPES])
@pytest.mark.parametrize("relay", [False, True])
def test_shape_parity(epx, shape, relay):
    T, k, E, R, H, s, hidden, routing = shape
    rng = np.random.Generator(np.random.PCG64(T * 7 + k * 3 + hidden))
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, routing, 1.2)
    w = W.draw_gate_weights(rng, T, k)
    print(f"[parity] shape {shape} relay={relay}", flush=True)
    run_case(epx, x, idx, w, E, R, H, s, relay, "bf16", f"{shape}/bf16")
    if hidden % 128 == 0:
        run_case(epx, x, idx, w, E, R, H, s, relay, "fp8", f"{shape}/fp8")


@pytest.mark.parametrize("relay", [False, True])
def test_duplicate_ids_and_one_hot_expert(epx, relay):
    """Repeated expert ids in a row (one row per pair, host counted once) and
    every token on one expert."""
    rng = np.random.Generator(np.random.PCG64(3))
    T, k, E, R, H, hidden = 300, 4, 16, 4, 2, 256
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    w = W.draw_gate_weights(rng, T, k)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    run_case(epx, x, idx, w, E, R, H, 2, relay, "bf16", "duplicates")
    run_case(epx, x, idx, w, E, R, H, 2, relay, "fp8", "duplicates/fp8")
    idx1 = np.full((T, k), 11, np.int32)
    run_case(epx, x, idx1, w, E, R, H, 1, relay, "bf16", "one expert")


def test_fp8_special_blocks(epx):
    """Zero, negative-zero, tiny (subnormal scale), saturating and mixed blocks."""
    rng = np.random.Generator(np.random.PCG64(4))
    T, hidden = 40, 1024
    x = rng.standard_normal((T, hidden), dtype=np.float32)
    x[0, :128] = 0.0
    x[1, :128] = -0.0
    x[2, 128:256] *= 1e-38
    x[3, 256:384] = 3e38
    x[4, 384:512] = np.where(rng.random(128) < 0.5, 1e-30, -2e30)
    x[5, 512:640] = 448.0
    x[6, :] *= 1e4
    xb = W.f32_to_bf16_bits(x)
    idx = W.draw_routing(rng, T, 16, 2, "uniform")
    w = W.draw_gate_weights(rng, T, 2)
    run_case(epx, xb, idx, w, 16, 4, 2, 0, False, "fp8", "fp8 specials")
    run_case(epx, xb, idx, w, 16, 4, 2, 0, True, "fp8", "fp8 specials relay")


def test_empty_batch(epx):
    for relay in (False, True):
        p = epx.make_problem(0, 2, 16, 4, 2, 1, epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT)
        L = epx.Layout(p)
        epx.epx_get_layout(p, torch.zeros((0, 2), dtype=torch.int32, device="cuda"), L)
        got = layout_np(epx, L, relay)
        ora = oracle.layout(np.zeros((0, 2), np.int32), 16, 4, 2, 1, relay=relay)
        assert_layout_parity(got, ora, relay, "empty")
        x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
        recv = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
        epx.epx_dispatch(p, L, x, epx.BF16, recv)
        out = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
        epx.epx_combine(p, L, recv, torch.zeros((0, 2), dtype=torch.float32, device="cuda"), out)
        torch.cuda.synchronize()


def test_out_of_range_ids_are_reported_and_nothing_is_written(epx):
    T, k, E, R, H, hidden = 100, 2, 16, 4, 2, 64
    idx = np.tile(np.array([[1, 2]], np.int32), (T, 1))
    idx[17, 1] = 16
    idx[90, 0] = -1
    for relay in (False, True):
        p = epx.make_problem(T, k, E, R, H, 0, epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT)
        L = epx.Layout(p)
        epx.epx_get_layout(p, _dev(idx), L)
        assert epx.epx_read_error(L) == 2
        cap = epx.relay_capacity(p) if relay else T * k
        recv = torch.full((cap, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        epx.epx_dispatch(p, L, torch.ones((T, hidden), dtype=torch.bfloat16, device="cuda"), epx.BF16, recv)
        out = torch.full((T, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        y = torch.ones((T * k, hidden), dtype=torch.bfloat16, device="cuda")
        epx.epx_combine(p, L, y, torch.ones((T, k), dtype=torch.float32, device="cuda"), out)
        assert np.all(_bits(recv) == SENTINEL_BF16)
        assert np.all(_bits(out) == SENTINEL_BF16)
        # a valid layout on the same arrays clears the error
        epx.epx_get_layout(p, _dev(np.ones((T, k), np.int32)), L)
        assert epx.epx_read_error(L) == 0


def test_repeat_runs_are_bitwise_identical(epx):
    w = W.WORKLOADS["large_batch"]
    d = W.make_inputs(w, num_tokens=2048)
    p = epx.make_problem(2048, 8, 256, 16, 2, 0, epx.MODE_HOST_RELAY)
    idx = _dev(d["topk_idx"])
    outs = []
    for _ in range(3):
        L = epx.Layout(p)
        epx.epx_get_layout(p, idx, L)
        outs.append(layout_np(epx, L, True))
    for n in outs[0]:
        assert np.array_equal(outs[0][n], outs[1][n]) and np.array_equal(outs[0][n], outs[2][n]), n


@pytest.mark.parametrize("relay", [False, True])
def test_repeat_layer_runs_are_bitwise_identical(epx, relay):
    """Three runs of the whole layer through the fused call (4096 tokens: the
    count, scan and assign-and-copy launches) and the combine give the same
    bytes, layout arrays included."""
    w = W.WORKLOADS["large_batch"]
    d = W.make_inputs(w)
    T, k, h = d["T"], w.topk, w.hidden
    p = epx.make_problem(T, k, w.num_experts, w.num_ranks, w.num_hosts, 0,
                         epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT)
    cap = epx.relay_capacity(p) if relay else T * k
    idx, x = _dev(d["topk_idx"]), _bf16_dev(d["x"])
    wts = _dev(d["topk_weights"])
    y = _bf16_dev(W.random_bf16((T * k, h), seed=11))
    runs = []
    for _ in range(3):
        L = epx.Layout(p)
        recv = torch.zeros((cap, h), dtype=torch.bfloat16, device="cuda")
        out = torch.zeros((T, h), dtype=torch.bfloat16, device="cuda")
        epx.epx_layout_dispatch(p, idx, L, x, epx.BF16, recv)
        epx.epx_combine(p, L, y, wts, out)
        torch.cuda.synchronize()
        runs.append((layout_np(epx, L, relay), _bits(recv), _bits(out)))
    for lay, rows, o in runs[1:]:
        for n in lay:
            assert np.array_equal(lay[n], runs[0][0][n]), n
        assert np.array_equal(rows, runs[0][1]) and np.array_equal(o, runs[0][2])


def test_e4m3_conversion_exhaustive_vs_oracle(epx):
    """The kernel's float32 -> E4M3FN conversion on every non-negative finite
    float32 pattern, and a sample of negatives (the oracle's converter is
    itself pinned exhaustively against torch)."""
    chunk = 1 << 27
    end = 0x7F800000
    for start in range(0, end, chunk):
        bits = np.arange(start, min(start + chunk, end), dtype=np.uint32)
        v = bits.view(np.float32)
        dv = _dev(v)
        dq = torch.empty(v.size, dtype=torch.uint8, device="cuda")
        epx.epx_f32_to_e4m3(dv, dq)
        got = dq.cpu().numpy()
        want = oracle.f32_to_e4m3(v)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (hex(int(bits[bad[0]])), got[bad[0]], want[bad[0]])
    rng = np.random.Generator(np.random.PCG64(5))
    v = -(rng.integers(0, end, size=1 << 24, dtype=np.uint32).view(np.float32))
    dq = torch.empty(v.size, dtype=torch.uint8, device="cuda")
    epx.epx_f32_to_e4m3(_dev(v), dq)
    assert np.array_equal(dq.cpu().numpy(), oracle.f32_to_e4m3(v))


# ---------------------------------------------------------------- equivalences
@pytest.mark.parametrize("name,relay", [("tiny", True), ("decode_skewed", False), ("fp8_dispatch", True)])
def test_fused_fp8_equals_quantising_the_bf16_rows(epx, name, relay):
    """The fp8 dispatch (quantised once per token, stored to every row) equals
    the bf16 dispatch followed by quantising each dispatched row on its own."""
    w = W.WORKLOADS[name]
    d = W.make_inputs(w)
    T, k, h = d["T"], w.topk, w.hidden
    p = epx.make_problem(T, k, w.num_experts, w.num_ranks, w.num_hosts, w.my_rank,
                         epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT)
    L = epx.Layout(p)
    epx.epx_get_layout(p, _dev(d["topk_idx"]), L)
    cap = epx.relay_capacity(p) if relay else T * k
    rows = int(L["totals"].cpu().numpy()[1 if relay else 0])
    x = _bf16_dev(d["x"])
    rb = torch.empty((cap, h), dtype=torch.bfloat16, device="cuda")
    epx.epx_dispatch(p, L, x, epx.BF16, rb)
    q = torch.empty((cap, h), dtype=torch.uint8, device="cuda")
    sc = torch.empty((cap, h // 128), dtype=torch.float32, device="cuda")
    epx.epx_dispatch(p, L, x, epx.FP8_E4M3, q, sc)
    bf_rows = _bits(rb)[:rows]
    ident = {"slot": np.arange(rows, dtype=np.int32), "totals": np.array([rows, 0, 0, 0], np.int32)}
    wq, wsc = oracle.dispatch_fp8(bf_rows, ident, 1, 1, False)
    assert np.array_equal(q.cpu().numpy()[:rows], wq), name
    assert np.array_equal(sc.cpu().numpy()[:rows].view(np.uint32), wsc.view(np.uint32)), name
