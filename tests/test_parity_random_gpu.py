"""GPU parity on seeded random geometries.

Each case draws a valid problem (expert, rank and host counts with E % R ==
0, R % H == 0, up to 32 ranks per host and 64 hosts; k from 1 to 64; T from
0 to a few thousand; hidden a multiple of 8, or of 128 for fp8), uniform or
Zipf routing (duplicate ids allowed in some cases) and runs layout,
dispatch (both modes; bf16, and fp8 when hidden allows) and combine against
the oracle, bit for bit, through the same checks as the fixed shapes. Cases
inside the fused call's bounds also run epx_layout_dispatch against the
oracle and the two-call path. The shapes come from one seeded generator, so
a failure names a reproducible case.
"""
import numpy as np
import pytest

from combine_epx_get_amd import workloads as W
from tests.test_parity_fused_gpu import run_fused
from tests.test_parity_gpu import run_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def epx():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


def draw_case(i: int):
    rng = np.random.Generator(np.random.PCG64(1000 + i))
    H = int(rng.choice([1, 2, 3, 4, 8, 16, 64]))
    rph = int(rng.choice([r for r in (1, 2, 3, 4, 8, 32) if H * r <= 256]))
    R = H * rph
    epr = int(rng.choice([e for e in (1, 2, 3, 4, 8, 16) if R * e <= 2048]))
    E = R * epr
    k = int(min(E, rng.choice([1, 2, 3, 6, 8, 16, 24, 64])))
    T = int(rng.choice([0, 1, 2, 31, 64, 65, 127, 128, 300, 1000, 2500]))
    if T * k > 40000:
        T = 40000 // k
    hidden = int(rng.choice([8, 136, 128, 256, 896, 2048]))
    s = int(rng.integers(0, R))
    routing = "zipf" if rng.random() < 0.4 else "uniform"
    dup = rng.random() < 0.15
    return dict(T=T, k=k, E=E, R=R, H=H, s=s, hidden=hidden, routing=routing, dup=dup, seed=i)


CASES = [draw_case(i) for i in range(96)]


@pytest.mark.parametrize("case", CASES, ids=[f"c{c['seed']}-T{c['T']}k{c['k']}E{c['E']}R{c['R']}H{c['H']}h{c['hidden']}"
                                             for c in CASES])
def test_random_geometry_parity(epx, case):
    c = case
    print(f"[random] {c}", flush=True)
    rng = np.random.Generator(np.random.PCG64(5000 + c["seed"]))
    T, k, E, R, H, s, h = c["T"], c["k"], c["E"], c["R"], c["H"], c["s"], c["hidden"]
    x = W.f32_to_bf16_bits(rng.standard_normal((T, h), dtype=np.float32))
    if c["dup"]:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    else:
        idx = W.draw_routing(rng, T, E, k, c["routing"], 1.1)
    w = W.draw_gate_weights(rng, T, k)
    for relay in (False, True):
        run_case(epx, x, idx, w, E, R, H, s, relay, "bf16", f"{c}/relay={relay}/bf16")
        if h % 128 == 0:
            run_case(epx, x, idx, w, E, R, H, s, relay, "fp8", f"{c}/relay={relay}/fp8")
        run_fused(epx, x, idx, E, R, H, s, relay, "bf16", what=f"{c}/relay={relay}/fused")
        if h % 128 == 0:
            run_fused(epx, x, idx, E, R, H, s, relay, "fp8", what=f"{c}/relay={relay}/fused fp8")
