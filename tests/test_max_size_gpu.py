"""The largest batch the library accepts (T = 2^24 tokens): the layout's
properties on every pair, and dispatch and combine on sampled tokens
against the oracle (one by one: the oracle's combine run on just those
tokens' rows gives the same float32 chain).

Rows are 16 bytes (hidden = 8) so that the buffers stay a few hundred MB;
the routing draws k = 2 ids per token with repeats allowed."""
import numpy as np
import pytest
import torch

import oracle
from combine_epx_get_amd import workloads as W
from tests.test_parity_gpu import _bits, _dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def epx():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


@pytest.mark.parametrize("relay", [False, True])
def test_max_tokens(epx, relay):
    T, k, E, R, H, s, h = 1 << 24, 2, 256, 16, 2, 5, 8
    rng = np.random.Generator(np.random.PCG64(24))
    idx = rng.integers(0, E, (T, k), dtype=np.int32)
    print(f"[max size] T={T} relay={relay}", flush=True)
    p = epx.make_problem(T, k, E, R, H, s, epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT)
    L = epx.Layout(p)
    epx.epx_get_layout(p, _dev(idx), L)
    assert epx.epx_read_error(L) == 0

    # layout properties on every pair
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    assert np.array_equal(L["expert_count"].cpu().numpy(), counts)
    off = L["expert_offset"].cpu().numpy()
    assert off[0] == 0 and np.array_equal(np.diff(off), counts)
    slot = L["slot"].cpu().numpy()
    row_token = L["row_token"].cpu().numpy()
    pair_token = np.repeat(np.arange(T, dtype=np.int32), k)
    assert np.array_equal(row_token[slot], pair_token)            # rows point back at their tokens
    seen = np.zeros(T * k, np.uint8)
    seen[slot] = 1
    assert seen.all()                                             # slot is a permutation
    e_of_row = np.repeat(np.arange(E, dtype=np.int32), counts)
    assert np.array_equal(e_of_row[slot], idx.ravel())            # each row in its expert's range
    same = e_of_row[1:] == e_of_row[:-1]
    assert np.all(row_token[1:][same] >= row_token[:-1][same])    # token order inside an expert
    del seen, e_of_row, same
    if relay:
        host_of_pair = idx // (E // R) // (R // H)
        touches = np.zeros((T, H), bool)
        touches[np.repeat(np.arange(T), k), host_of_pair.ravel()] = True
        want_ht = touches.sum(axis=0).astype(np.int32)
        assert np.array_equal(L["host_tokens"].cpu().numpy(), want_ht)
        rs = L["relay_slot"].cpu().numpy().reshape(T, H)
        assert np.array_equal(rs >= 0, touches)
        ho = L["host_offset"].cpu().numpy()
        for hh in range(H):     # rows of host hh: its range, in token order
            r = rs[:, hh][touches[:, hh]]
            assert np.array_equal(r, np.arange(ho[hh], ho[hh + 1], dtype=np.int32))
        del touches, rs

    # dispatch and combine, checked on sampled tokens
    x = W.f32_to_bf16_bits(rng.standard_normal((T, h), dtype=np.float32))
    cap = epx.relay_capacity(p) if relay else T * k
    recv = torch.empty((cap, h), dtype=torch.bfloat16, device="cuda")
    x_dev = _dev(x.view(np.int16)).view(torch.bfloat16)
    epx.epx_dispatch(p, L, x_dev, epx.BF16, recv)

    # the fused call (count, scan, then assignment and copies in one launch)
    # gives the same layout and rows
    L2 = epx.Layout(p)
    recv2 = torch.empty_like(recv)
    epx.epx_layout_dispatch(p, _dev(idx), L2, x_dev, epx.BF16, recv2)
    torch.cuda.synchronize()
    used = int(L["totals"][1 if relay else 0])
    for name in ("slot", "row_token", "expert_offset", "totals") + (("relay_slot", "relay_token") if relay else ()):
        assert torch.equal(L2[name], L[name]), name
    assert torch.equal(recv2[:used].view(torch.int16), recv[:used].view(torch.int16))
    del L2, recv2
    y = W.f32_to_bf16_bits(rng.standard_normal((T * k, h), dtype=np.float32))
    w = rng.random((T, k), dtype=np.float32)
    out = torch.empty((T, h), dtype=torch.bfloat16, device="cuda")
    epx.epx_combine(p, L, _dev(y.view(np.int16)).view(torch.bfloat16), _dev(w), out)
    torch.cuda.synchronize()
    sample = np.unique(np.concatenate([rng.integers(0, T, 4096), [0, 1, T - 2, T - 1]]))
    got_recv = _bits(recv)
    if relay:
        rs = L["relay_slot"].cpu().numpy().reshape(T, H)[sample]
        for i, t in enumerate(sample):
            for hh in range(H):
                if rs[i, hh] >= 0:
                    assert np.array_equal(got_recv[rs[i, hh]], x[t]), (t, hh)
    else:
        sl = slot.reshape(T, k)[sample]
        for j in range(k):
            assert np.array_equal(got_recv[sl[:, j]], x[sample]), j
    n = sample.size
    sub = {"slot": np.arange(n * k, dtype=np.int32)}
    want = oracle.combine(y[slot.reshape(T, k)[sample].ravel()], sub, w[sample])
    assert np.array_equal(_bits(out)[sample], want)
