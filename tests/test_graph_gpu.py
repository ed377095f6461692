"""A HIP graph capturing layout, dispatch and combine (or the relay receive
side: fan-out, partials and finish) replays to the eager results: several
replays, with eager work and a synchronisation between them, each checked
bit for bit (layout slots, dispatched rows, fanned-out rows and partials,
combined output). The library records no memset; every array it writes is
written by its kernels."""
import numpy as np
import pytest
import torch

from combine_epx_get_amd import workloads as W
from tests.test_parity_gpu import SENTINEL_BF16, SENTINEL_U8, _bits, _dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def epx():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


CASES = [
    # workload, relay, groups, fp8, fused layout and dispatch, relay receive side
    ("decode_skewed", False, 1, False, False, False),
    ("decode_skewed", True, 1, False, False, False),
    ("tiny", True, 1, True, False, False),
    ("tiny", False, 2, False, False, False),
    ("decode_uniform", False, 4, True, False, False),
    ("decode_skewed", True, 1, True, True, False),
    ("rank_heavy", False, 1, False, True, False),
    ("large_batch", False, 1, False, True, False),   # count, scan, assign-and-copy
    ("fp8_dispatch", True, 1, True, True, False),    # the same in relay mode, fp8
    ("decode_skewed", True, 1, True, False, True),
    ("rank_light", True, 1, False, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{'relay' if c[1] else 'expert'}-m{c[2]}-{'fp8' if c[3] else 'bf16'}"
                                             f"{'-fused' if c[4] else ''}{'-receive' if c[5] else ''}"
                                             for c in CASES])
def test_graph_replays_match_eager(epx, case):
    name, relay, m, fp8, fused, receive = case
    w = W.WORKLOADS[name]
    d = W.make_inputs(w)
    T, k, h = d["T"], w.topk, w.hidden
    print(f"[graph] {case}", flush=True)
    p = epx.make_problem(T, k, w.num_experts, w.num_ranks, w.num_hosts, w.my_rank,
                         epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT, m)
    L = epx.Layout(p)
    idx = _dev(d["topk_idx"])
    x = _dev(d["x"].view(np.int16)).view(torch.bfloat16)
    wts = _dev(d["topk_weights"])
    cap = epx.relay_capacity(p) if relay else T * k
    if fp8:
        recv = torch.empty((cap, h), dtype=torch.uint8, device="cuda")
        scales = torch.empty((cap, h // 128), dtype=torch.float32, device="cuda")
    else:
        recv = torch.empty((cap, h), dtype=torch.bfloat16, device="cuda")
        scales = None
    y = _dev(W.random_bf16((T * k, h), seed=7).view(np.int16)).view(torch.bfloat16)
    out = torch.empty((T, h), dtype=torch.bfloat16, device="cuda")
    carry = torch.empty((T, h), dtype=torch.float32, device="cuda") if m > 1 else None
    dt = epx.FP8_E4M3 if fp8 else epx.BF16
    if receive:   # the relay GPU's per-expert rows and the float32 partials
        fan = torch.empty((T * k, h), dtype=recv.dtype, device="cuda")
        fan_sc = torch.empty((T * k, h // 128), dtype=torch.float32, device="cuda") if fp8 else None
        part = torch.empty((cap, h), dtype=torch.float32, device="cuda")

    def receive_side():
        epx.epx_relay_fanout(p, L, recv, fan, scales, fan_sc)
        epx.epx_combine_relay_partials(p, L, y, wts, part)
        epx.epx_combine_relay_finish(p, L, part, out)

    def step():
        if fused:
            epx.epx_layout_dispatch(p, idx, L, x, dt, recv, scales)
            if receive:
                receive_side()
            else:
                epx.epx_combine(p, L, y, wts, out)
            return
        if receive:
            epx.epx_get_layout(p, idx, L)
            epx.epx_dispatch(p, L, x, dt, recv, scales)
            receive_side()
            return
        epx.epx_get_layout(p, idx, L)
        if m > 1:
            for g in range(m):
                epx.epx_dispatch_group(p, L, g, x, dt, recv, scales)
            for g in range(m):
                epx.epx_combine_group(p, L, g, y, wts, carry, out)
        else:
            epx.epx_dispatch(p, L, x, dt, recv, scales)
            epx.epx_combine(p, L, y, wts, out)

    def clear():
        L["slot"].fill_(-5)
        L["expert_offset"].fill_(-5)
        recv.view(torch.uint8).fill_(SENTINEL_U8)
        if scales is not None:
            scales.fill_(-1.0)
        out.view(torch.int16).fill_(SENTINEL_BF16)
        if receive:
            fan.view(torch.uint8).fill_(SENTINEL_U8)
            if fan_sc is not None:
                fan_sc.fill_(-1.0)
            part.fill_(float("nan"))

    def snapshot():
        torch.cuda.synchronize()
        rows = int(L["totals"].cpu().numpy()[1 if relay else 0])
        snap = {"slot": L["slot"].cpu().numpy().copy(), "expert_offset": L["expert_offset"].cpu().numpy().copy(),
                "recv": recv.view(torch.uint8)[:rows].cpu().numpy().copy(), "out": _bits(out).copy()}
        if scales is not None:
            snap["scales"] = scales[:rows].cpu().numpy().copy()
        if receive:
            snap["fan"] = fan.view(torch.uint8).cpu().numpy().copy()
            snap["part"] = part[:rows].cpu().numpy().copy()
            if fan_sc is not None:
                snap["fan_sc"] = fan_sc.cpu().numpy().copy()
        return snap

    clear()
    step()
    want = snapshot()
    assert not np.any(want["out"] == np.uint16(SENTINEL_BF16 & 0xFFFF))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    # eager work between replays: another layout on other routing, and fills
    other = epx.Layout(p)
    other_idx = _dev(np.ascontiguousarray(d["topk_idx"][::-1]))
    for rep in range(3):
        clear()
        epx.epx_get_layout(p, other_idx, other)
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for n in want:
            a, b = got[n], want[n]
            if a.dtype == np.float32:
                a, b = a.view(np.uint32), b.view(np.uint32)
            assert np.array_equal(a, b), (case, rep, n)


def test_current_stream_handle(epx):
    """The binding launches on torch's current stream: the raw handle it reads
    is that stream's, on the default stream and inside a side-stream context."""
    assert epx._stream(None) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert epx._stream(None) == side.cuda_stream == torch.cuda.current_stream().cuda_stream
    assert epx._stream(side) == side.cuda_stream
