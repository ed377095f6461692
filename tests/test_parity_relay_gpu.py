"""GPU parity of the relay receive side and the two-level combine against the
oracle: fan-out rows (bf16, fp8 codes + scales), level-1 partials (fp32 and
bf16 wire form) and the level-2 output, all bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from combine_epx_get_amd import workloads as W
from tests.test_parity_gpu import (SENTINEL_BF16, SENTINEL_U8, _bf16_dev, _bits, _dev,
                                   assert_layout_parity, expert_outputs, layout_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def epx():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


def run_relay_case(epx, x_bits, idx, w, E, R, H, s, what=""):
    T, k = idx.shape
    hidden = x_bits.shape[1]
    ora = oracle.layout(idx, E, R, H, s, relay=True)
    p = epx.make_problem(T, k, E, R, H, s, epx.MODE_HOST_RELAY)
    L = epx.Layout(p)
    epx.epx_get_layout(p, _dev(idx), L)
    assert_layout_parity(layout_np(epx, L, True), ora, True, what)
    cap = epx.relay_capacity(p)
    rows = int(ora["totals"][1])
    x_t = _bf16_dev(x_bits)

    # bf16: relay dispatch, then fan-out == per-expert rows
    relay = torch.empty((cap, hidden), dtype=torch.bfloat16, device="cuda")
    epx.epx_dispatch(p, L, x_t, epx.BF16, relay)
    recv = torch.full((T * k, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    epx.epx_relay_fanout(p, L, relay, recv)
    want = oracle.relay_fanout(_bits(relay)[:rows], ora, idx, E, R, H)
    assert np.array_equal(_bits(recv), want), (what, "fan-out bf16")
    assert np.array_equal(want, oracle.dispatch_bf16(x_bits, ora, k, H, False))

    # fp8: relay dispatch, fan-out of codes and scales
    if hidden % 128 == 0:
        q = torch.empty((cap, hidden), dtype=torch.uint8, device="cuda")
        sc = torch.empty((cap, hidden // 128), dtype=torch.float32, device="cuda")
        epx.epx_dispatch(p, L, x_t, epx.FP8_E4M3, q, sc)
        rq = torch.full((T * k, hidden), SENTINEL_U8, dtype=torch.uint8, device="cuda")
        rsc = torch.full((T * k, hidden // 128), -1.0, dtype=torch.float32, device="cuda")
        epx.epx_relay_fanout(p, L, q, rq, relay_scales=sc, recv_scales=rsc)
        wq, wsc = oracle.relay_fanout(q.cpu().numpy()[:rows], ora, idx, E, R, H,
                                      relay_scales=sc.cpu().numpy()[:rows])
        assert np.array_equal(rq.cpu().numpy(), wq), (what, "fan-out fp8 codes")
        assert np.array_equal(rsc.cpu().numpy().view(np.uint32), wsc.view(np.uint32)), (what, "scales")

    # two-level combine, fp32 and bf16 partials
    y = expert_outputs(W.bf16_bits_to_f32(x_bits), idx, ora["slot"])
    y_t = _bf16_dev(y)
    w_t = _dev(w)
    for dt, np_dt in ((torch.float32, np.float32), (torch.bfloat16, np.uint16)):
        bf16 = dt == torch.bfloat16
        part = torch.full((cap, hidden), -7.0, dtype=torch.float32, device="cuda").to(dt)
        epx.epx_combine_relay_partials(p, L, y_t, w_t, part)
        want_p = oracle.relay_partials(y, ora, idx, w, E, R, H, bf16=bf16)
        got_p = _bits(part) if bf16 else part.cpu().numpy()
        assert np.array_equal(got_p[:rows].view(np.uint16 if bf16 else np.uint32),
                              want_p.view(np.uint16 if bf16 else np.uint32)), (what, "partials", dt)
        sentinel = _bits(torch.full((1,), -7.0, dtype=dt, device="cuda")) if bf16 else None
        if rows < cap:
            tail = got_p[rows:]
            assert np.all(tail == (sentinel[0] if bf16 else np.float32(-7.0))), (what, "partial rows past the end")
        out = torch.full((T, hidden), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        epx.epx_combine_relay_finish(p, L, part, out)
        want_o = oracle.relay_finish(want_p, ora, T, H)
        assert np.array_equal(_bits(out), want_o), (what, "finish", dt)
    return ora


RELAY_WORKLOADS = ["tiny", "decode_skewed", "decode_skewed_s06", "fp8_dispatch", "large_batch",
                   "hybridep_bf16"]


@pytest.mark.parametrize("name", RELAY_WORKLOADS)
def test_relay_workload_parity(epx, name):
    w = W.WORKLOADS[name]
    d = W.make_inputs(w)
    print(f"[relay parity] {name} T={d['T']}", flush=True)
    run_relay_case(epx, d["x"], d["topk_idx"], d["topk_weights"], w.num_experts, w.num_ranks,
                   w.num_hosts, w.my_rank, name)


SHAPES = [
    # T, k, E, R, H, s, hidden
    (1, 1, 8, 8, 8, 5, 8),
    (63, 3, 12, 4, 2, 3, 136),
    (130, 6, 6, 3, 1, 1, 264),        # one host: two-level = flat
    (200, 4, 32, 8, 4, 6, 1024),
    (257, 2, 16, 16, 16, 15, 256),    # k < H
    (3000, 16, 2048, 64, 2, 33, 256),
    (50, 64, 64, 8, 4, 1, 128),
    (5000, 8, 256, 256, 64, 200, 128),
    (200, 32, 64, 8, 4, 2, 136),      # k > 16 in the multi-workgroup layout
    (100, 64, 128, 16, 8, 3, 128),
    (1500, 24, 96, 12, 3, 7, 128),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{s[0]}k{s[1]}E{s[2]}R{s[3]}H{s[4]}h{s[6]}" for s in SHAPES])
def test_relay_shape_parity(epx, shape):
    T, k, E, R, H, s, hidden = shape
    rng = np.random.Generator(np.random.PCG64(T * 3 + k + hidden))
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, "zipf", 0.9)
    w = W.draw_gate_weights(rng, T, k)
    print(f"[relay parity] shape {shape}", flush=True)
    run_relay_case(epx, x, idx, w, E, R, H, s, str(shape))


def test_one_host_two_level_equals_flat_on_gpu(epx):
    T, k, E, R, H, hidden = 300, 8, 64, 8, 1, 512
    rng = np.random.Generator(np.random.PCG64(11))
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, "uniform")
    w = W.draw_gate_weights(rng, T, k)
    p = epx.make_problem(T, k, E, R, H, 0, epx.MODE_HOST_RELAY)
    L = epx.Layout(p)
    epx.epx_get_layout(p, _dev(idx), L)
    ora = oracle.layout(idx, E, R, H, 0, relay=True)
    y = _bf16_dev(expert_outputs(W.bf16_bits_to_f32(x), idx, ora["slot"]))
    wt = _dev(w)
    flat = torch.empty((T, hidden), dtype=torch.bfloat16, device="cuda")
    epx.epx_combine(p, L, y, wt, flat)
    part = torch.empty((epx.relay_capacity(p), hidden), dtype=torch.float32, device="cuda")
    epx.epx_combine_relay_partials(p, L, y, wt, part)
    out = torch.empty_like(flat)
    epx.epx_combine_relay_finish(p, L, part, out)
    assert np.array_equal(_bits(out), _bits(flat))


def test_relay_calls_need_relay_mode(epx):
    p = epx.make_problem(4, 2, 16, 4, 2, 0, epx.MODE_PER_EXPERT)
    L = epx.Layout(p)
    rows = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(epx.EpxError) as ei:
        epx.epx_relay_fanout(p, L, rows, rows)
    assert ei.value.code == 1


def test_fanout_binding_checks_scale_shapes(epx):
    """Undersized fp8 scale tensors are refused by the binding before the
    call (the kernel would read and write one scale per 128 channels of every
    relay and per-expert row)."""
    T, k, E, R, H, h = 64, 2, 16, 4, 2, 256
    p = epx.make_problem(T, k, E, R, H, 0, epx.MODE_HOST_RELAY)
    L = epx.Layout(p)
    epx.epx_get_layout(p, _dev(np.tile(np.array([[1, 9]], np.int32), (T, 1))), L)
    cap = epx.relay_capacity(p)
    rows = torch.zeros((cap, h), dtype=torch.uint8, device="cuda")
    recv = torch.zeros((T * k, h), dtype=torch.uint8, device="cuda")
    good_rs = torch.zeros((cap, h // 128), dtype=torch.float32, device="cuda")
    good_sc = torch.zeros((T * k, h // 128), dtype=torch.float32, device="cuda")
    short_rs = torch.zeros((cap - 1, h // 128), dtype=torch.float32, device="cuda")
    short_sc = torch.zeros((T * k, h // 128 - 1), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        epx.epx_relay_fanout(p, L, rows, recv, short_rs, good_sc)
    with pytest.raises(ValueError):
        epx.epx_relay_fanout(p, L, rows, recv, good_rs, short_sc)
    epx.epx_relay_fanout(p, L, rows, recv, good_rs, good_sc)
    torch.cuda.synchronize()
