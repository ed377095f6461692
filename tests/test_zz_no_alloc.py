"""epx_layout_dispatch_noalloc against epx_layout_dispatch, through the C ABI.

The no-alloc call takes the layout kernels' scratch from a static device
array of the library instead of the layout's workspace; everything else is
the same call. Each case runs two calls in a row, the second on a smaller
problem, so the second finds the first one's contents in the shared array.
Every layout array, row, code and scale must equal what epx_layout_dispatch
writes on separate arrays. The cases take each path that uses the scratch:
count + scan + assign-and-copy (bf16, per-expert and relay; fp8 relay),
count + scan + assign then the fp8 dispatch, count + assign summing the
columns itself, and the single-launch decode path (no scratch).
"""
import numpy as np
import pytest
import torch

from combine_epx_get_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def epx():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    from combine_epx_get_amd import epx as mod
    return mod


def _arrays(epx, L, relay):
    out = {}
    for name in epx.LAYOUT_FIELDS:
        if name == "workspace" or (name in epx.RELAY_FIELDS and not relay):
            continue
        out[name] = L[name].cpu().numpy()
    return out


def _run(epx, call, p, idx, x, relay, fp8, layout_arg, L):
    T, k, h = p.num_tokens, p.topk, x.shape[1]
    cap = epx.relay_capacity(p) if relay else T * k
    if fp8:
        recv = torch.full((cap, h), 0xA5, dtype=torch.uint8, device="cuda")
        sc = torch.full((cap, h // 128), -1.0, dtype=torch.float32, device="cuda")
        call(p, idx, layout_arg, x, epx.FP8_E4M3, recv, sc)
    else:
        recv = torch.full((cap, h), 0x7FBF, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        sc = None
        call(p, idx, layout_arg, x, epx.BF16, recv)
    torch.cuda.synchronize()
    got = {"recv": recv.view(torch.uint8).cpu().numpy()}
    if sc is not None:
        got["scales"] = sc.cpu().numpy().view(np.uint32)
    got.update(_arrays(epx, L, relay))
    return got


CASES = [
    # name, (T, k, E, R, H, s, hidden, relay, fp8)
    ("assign_copy per-expert bf16", (4096, 8, 256, 16, 2, 0, 7168, False, False),
     (1500, 8, 256, 16, 2, 0, 7168, False, False)),
    ("assign_copy relay bf16 / fp8", (4096, 8, 256, 32, 4, 5, 2048, True, False),
     (700, 8, 256, 32, 4, 5, 2048, True, True)),
    ("count+scan+assign, fp8 dispatch", (4096, 8, 256, 16, 2, 0, 1024, False, True),
     (2000, 8, 128, 16, 2, 0, 1024, False, True)),
    ("count+assign summing columns", (500, 16, 64, 8, 2, 1, 512, False, True),
     (300, 16, 64, 8, 2, 1, 256, False, True)),
    ("decode single launch, both modes", (128, 8, 256, 32, 4, 0, 7168, False, False),
     (64, 8, 256, 32, 4, 0, 7168, True, False)),
]


@pytest.mark.parametrize("name,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_layout_dispatch_two_calls(epx, name, first, second):
    for shape in (first, second):
        T, k, E, R, H, s, h, relay, fp8 = shape
        print(f"[noalloc] {name} T={T} k={k} E={E} R={R} H={H} h={h} relay={relay} fp8={fp8}", flush=True)
        rng = np.random.Generator(np.random.PCG64(T + 7 * k + h))
        xb = W.f32_to_bf16_bits(rng.standard_normal((T, h), dtype=np.float32))
        idx_np = W.draw_routing(rng, T, E, k, "uniform")
        mode = epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT
        p = epx.make_problem(T, k, E, R, H, s, mode)
        idx = torch.from_numpy(idx_np).to("cuda")
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to("cuda")
        L_ref = epx.Layout(p)
        want = _run(epx, epx.epx_layout_dispatch, p, idx, x, relay, fp8, L_ref, L_ref)
        L = epx.Layout(p)
        struct = epx.epx_layout(*[None if n == "workspace" else getattr(L.struct, n)
                                  for n in epx.LAYOUT_FIELDS])
        got = _run(epx, epx.epx_layout_dispatch_noalloc, p, idx, x, relay, fp8, struct, L)
        assert epx.epx_read_error(L) == 0
        for key in want:
            assert got[key].shape == want[key].shape, (name, shape, key)
            bad = np.nonzero(got[key].ravel() != want[key].ravel())[0]
            assert bad.size == 0, (name, shape, key, int(bad[0]), bad.size)
