"""GPU parity for rows wider than one burst (hidden > 8192 channels).

Up to 8192 channels a wave moves a whole row in one burst of 16-byte
vectors; wider rows take the kernels' loops over bursts (dispatch, the
assign-and-copy launch, the relay fan-out, partials and finish, combine) and
split the fp8 quantisation over several passes. These shapes reach those
loops with at least 2048 tokens (one column slice per token), a ragged last
burst (10 248 channels), both modes and expert groups; every result is
compared with the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

from combine_epx_get_amd import workloads as W
from tests.test_parity_fused_gpu import run_fused
from tests.test_parity_groups_gpu import run_group_case
from tests.test_parity_gpu import run_case
from tests.test_parity_relay_gpu import run_relay_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def epx():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


SHAPES = [
    # T, k, E, R, H, s, hidden, routing
    (2048, 2, 16, 4, 2, 1, 16384, "uniform"),   # two full bursts per row; fp8 in two slices
    (2050, 3, 24, 6, 3, 2, 10248, "zipf"),      # 1281 vectors: a ragged second burst (bf16 only)
    (2048, 2, 16, 4, 2, 3, 16512, "uniform"),   # 2064 vectors: a third burst, a second combine pass
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{s[0]}k{s[1]}h{s[6]}" for s in SHAPES])
@pytest.mark.parametrize("relay", [False, True])
def test_wide_row_parity(epx, shape, relay):
    T, k, E, R, H, s, hidden, routing = shape
    rng = np.random.Generator(np.random.PCG64(T + k + hidden))
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, routing, 1.1)
    w = W.draw_gate_weights(rng, T, k)
    print(f"[wide rows] {shape} relay={relay}", flush=True)
    dtypes = ("bf16", "fp8") if hidden % 128 == 0 else ("bf16",)
    for dt in dtypes:
        run_case(epx, x, idx, w, E, R, H, s, relay, dt, f"{shape}/{dt}")
        run_fused(epx, x, idx, E, R, H, s, relay, dt, what=f"{shape}/fused {dt}")
    if relay:
        run_relay_case(epx, x, idx, w, E, R, H, s, f"{shape}/relay receive")


def test_wide_row_groups(epx):
    """Two expert groups at 16 512 channels: the group dispatch and the group
    combine (with its float32 carry) over more than one burst."""
    T, k, E, R, H, s, m, hidden = 2048, 4, 32, 4, 2, 1, 2, 16512
    rng = np.random.Generator(np.random.PCG64(77))
    x = W.f32_to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, "uniform")
    w = W.draw_gate_weights(rng, T, k)
    print("[wide rows] groups", flush=True)
    run_group_case(epx, x, idx, w, E, R, H, s, m, "wide groups")
