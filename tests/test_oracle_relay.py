"""Pins of the oracle's relay receive side and two-level combine (digest
"Balancing and Beyond", section 3.2 Mode 2 and Figure 3: fan-out at the
same-index GPU, per-host sums there, the source sums the hosts).

* fan-out of tagged relay rows (row r filled with r): every per-expert row
  holds the tag of the relay row of its (token, host of the expert) —
  recounted by brute force;
* fan-out of the relay dispatch equals the per-expert dispatch, bf16 and fp8;
* partial membership: weights 2^j and expert outputs 1.0 make every partial
  the exact integer sum of 2^j over the token's experts on that host;
* one host: the two-level combine is the flat combine, bit for bit;
* float64 reference within the float32 bound (fp32 partials) and within the
  bound of one extra bf16 rounding per partial (bf16 partials).
"""
import numpy as np
import pytest

import oracle
from combine_epx_get_amd import workloads as W

SHAPES = [
    # T, k, E, R, H, s
    (64, 2, 16, 4, 2, 0),
    (37, 8, 256, 32, 4, 5),
    (50, 6, 48, 12, 3, 7),
    (20, 4, 64, 64, 64, 9),
    (9, 3, 6, 3, 1, 1),
]


def _case(shape, seed=0, routing="uniform"):
    T, k, E, R, H, s = shape
    rng = np.random.Generator(np.random.PCG64(seed + T * 13 + k))
    idx = W.draw_routing(rng, T, E, k, routing, 1.1)
    lay = oracle.layout(idx, E, R, H, s, relay=True)
    return rng, idx, lay


@pytest.mark.parametrize("shape", SHAPES)
def test_fanout_of_tagged_rows_brute_force(shape):
    T, k, E, R, H, s = shape
    rng, idx, lay = _case(shape)
    rows = int(lay["totals"][1])
    tagged = np.repeat(np.arange(rows, dtype=np.int32)[:, None], 4, axis=1)   # row r holds r
    got = oracle.relay_fanout(tagged, lay, idx, E, R, H)
    epr, rph = E // R, R // H
    for t in range(T):
        for j in range(k):
            h = idx[t, j] // epr // rph
            want = lay["relay_slot"][t * H + h]
            assert want >= 0
            assert np.all(got[lay["slot"][t * k + j]] == want), (t, j)


@pytest.mark.parametrize("shape", SHAPES)
def test_fanout_of_relay_dispatch_is_per_expert_dispatch(shape):
    T, k, E, R, H, s = shape
    rng, idx, lay = _case(shape, routing="zipf")
    x = W.f32_to_bf16_bits(rng.standard_normal((T, 256), dtype=np.float32))
    relay = oracle.dispatch_bf16(x, lay, k, H, True)
    per_expert = oracle.dispatch_bf16(x, lay, k, H, False)
    assert np.array_equal(oracle.relay_fanout(relay, lay, idx, E, R, H), per_expert)
    q, sc = oracle.dispatch_fp8(x, lay, k, H, True)
    qe, sce = oracle.dispatch_fp8(x, lay, k, H, False)
    fq, fsc = oracle.relay_fanout(q, lay, idx, E, R, H, relay_scales=sc)
    assert np.array_equal(fq, qe) and np.array_equal(fsc.view(np.uint32), sce.view(np.uint32))


@pytest.mark.parametrize("shape", SHAPES)
def test_partial_membership_exact(shape):
    T, k, E, R, H, s = shape
    rng, idx, lay = _case(shape)
    w = np.tile((2.0 ** np.arange(k)).astype(np.float32), (T, 1))
    y = W.f32_to_bf16_bits(np.ones((T * k, 8), np.float32))
    part = oracle.relay_partials(y, lay, idx, w, E, R, H)
    epr, rph = E // R, R // H
    for t in range(T):
        for h in range(H):
            r = lay["relay_slot"][t * H + h]
            want = sum(2.0 ** j for j in range(k) if idx[t, j] // epr // rph == h)
            if r < 0:
                assert want == 0
            else:
                assert np.all(part[r] == want), (t, h)
    out = W.bf16_bits_to_f32(oracle.relay_finish(part, lay, T, H))
    assert np.all(out == 2.0 ** k - 1)           # every j lands in exactly one partial


@pytest.mark.parametrize("k,E,R", [(2, 16, 4), (8, 256, 32), (5, 40, 8)])
def test_one_host_two_level_is_flat(k, E, R):
    T = 57
    rng = np.random.Generator(np.random.PCG64(k + E))
    idx = W.draw_routing(rng, T, E, k, "uniform")
    w = W.draw_gate_weights(rng, T, k)
    lay = oracle.layout(idx, E, R, 1, 0, relay=True)
    y = W.f32_to_bf16_bits(rng.standard_normal((T * k, 64), dtype=np.float32) * 3)
    flat = oracle.combine(y, lay, w)
    part = oracle.relay_partials(y, lay, idx, w, E, R, 1)
    assert np.array_equal(oracle.relay_finish(part, lay, T, 1), flat)


@pytest.mark.parametrize("shape", SHAPES[:4])
def test_two_level_within_bounds_of_float64(shape):
    T, k, E, R, H, s = shape
    rng, idx, lay = _case(shape, seed=3)
    w = W.draw_gate_weights(rng, T, k)
    y = W.f32_to_bf16_bits(rng.standard_normal((T * k, 96), dtype=np.float32) * 2)
    yf = W.bf16_bits_to_f32(y).astype(np.float64)
    terms = w.astype(np.float64)[:, :, None] * yf[lay["slot"].reshape(T, k)]
    exact = terms.sum(1)
    mag = np.abs(terms).sum(1)
    g = (k + H) * 2.0 ** -24 * 1.01
    for bf16 in (False, True):
        part = oracle.relay_partials(y, lay, idx, w, E, R, H, bf16=bf16)
        out = W.bf16_bits_to_f32(oracle.relay_finish(part, lay, T, H)).astype(np.float64)
        extra = 2.0 ** -8 * mag if bf16 else 0.0          # one bf16 rounding per partial
        bound = g * mag + extra + 2.0 ** -8 * np.abs(exact) + 1e-30
        assert np.all(np.abs(out - exact) <= bound), bf16
