"""The C ABI from a host program with no Python in its process.

tests/c_abi/epx_abi_driver (built by build()) allocates with the HIP runtime,
calls epx_layout_sizes, epx_get_layout, epx_dispatch, epx_combine and
epx_read_error on a stream of its own and writes every result to files; it
also checks documented argument errors (short capacity, null x, misaligned
out, my_rank out of range), which return before anything launches. This
test writes the seeded inputs, runs the program as a child process and
compares what it wrote with the oracle: layout arrays, rows (bf16, or fp8
codes and scales) and the combine, bit for bit.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from combine_epx_get_amd import workloads as W
from tests.c_abi import EXE
from tests.test_parity_gpu import assert_layout_parity, expert_outputs

pytestmark = pytest.mark.gpu

# the layout arrays in the order of the header's EPX_L_* indices
FIELDS = ["expert_count", "expert_offset", "rank_rows", "rank_tokens", "rank_offset",
          "host_tokens", "host_offset", "slot", "row_token", "relay_slot", "relay_token",
          "fanout_expert", "fanout_rank_mask", "relay_dst_rank", "totals", "group_offset"]
RELAY = {"relay_slot", "relay_token", "fanout_expert", "fanout_rank_mask"}

CASES = [
    # T, k, E, R, H, s, relay, hidden, fp8, routing
    (64, 2, 16, 4, 2, 0, False, 256, False, "uniform"),        # the tiny workload's shape
    (128, 8, 256, 32, 4, 5, True, 7168, True, "zipf"),         # decode, relay fp8
    (1500, 8, 64, 8, 2, 3, False, 1024, False, "uniform"),     # count + scan + assign launches
    (200, 32, 64, 8, 4, 1, True, 136, False, "zipf"),          # k > 16, ragged hidden
    (0, 4, 16, 4, 2, 0, True, 128, True, "uniform"),           # empty batch
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}k{c[1]}E{c[2]}R{c[3]}H{c[4]}{'relay' if c[6] else 'pe'}"
                                             f"{'fp8' if c[8] else 'bf16'}" for c in CASES])
def test_driver_through_the_c_abi(case, tmp_path):
    T, k, E, R, H, s, relay, h, fp8, routing = case
    if not os.path.exists(EXE):
        raise RuntimeError(f"{EXE} is not built (build() builds it)")
    rng = np.random.Generator(np.random.PCG64(4242 + T + k))
    x = W.f32_to_bf16_bits(rng.standard_normal((T, h), dtype=np.float32))
    idx = W.draw_routing(rng, T, E, k, routing, 1.2)
    w = W.draw_gate_weights(rng, T, k)
    ora = oracle.layout(idx, E, R, H, s, relay=relay)
    y = expert_outputs(W.bf16_bits_to_f32(x), idx, ora["slot"])

    d = str(tmp_path)
    with open(os.path.join(d, "problem.txt"), "w") as f:
        f.write(f"{T} {k} {E} {R} {H} {s} {int(relay)} {h} {int(fp8)}\n")
    idx.astype(np.int32).tofile(os.path.join(d, "topk_idx.bin"))
    x.tofile(os.path.join(d, "x.bin"))
    w.astype(np.float32).tofile(os.path.join(d, "w.bin"))
    y.tofile(os.path.join(d, "y.bin"))
    print(f"[c abi] {case}", flush=True)
    r = subprocess.run([EXE, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)

    statuses = dict(line.split() for line in open(os.path.join(d, "statuses.txt")))
    assert statuses["get_layout"] == "0" and statuses["dispatch"] == "0" and statuses["combine"] == "0"
    assert statuses["layout_bad_rank"] == "1" and statuses["bad_ids"] == "0"
    if T > 0:
        assert statuses["dispatch_capacity_short"] == "3"
        assert statuses["dispatch_null_x"] == "1" and statuses["combine_misaligned_out"] == "1"

    got = {}
    for i, name in enumerate(FIELDS):
        if name in RELAY and not relay:
            continue
        a = np.fromfile(os.path.join(d, f"layout_{i}.bin"), dtype=np.int32)
        got[name] = a.view(np.uint32) if name == "fanout_rank_mask" else a
    assert_layout_parity(got, ora, relay, str(case))

    rows = int(ora["totals"][1] if relay else ora["totals"][0])
    cap = T * min(k, H) if relay else T * k
    if fp8:
        q = np.fromfile(os.path.join(d, "recv.bin"), dtype=np.uint8).reshape(cap, h)
        sc = np.fromfile(os.path.join(d, "scales.bin"), dtype=np.uint32).reshape(cap, h // 128)
        wq, ws = oracle.dispatch_fp8(x, ora, k, H, relay)
        assert np.array_equal(q[:rows], wq)
        assert np.array_equal(sc[:rows], ws.view(np.uint32))
        assert np.all(q[rows:] == 0x5A) and np.all(sc[rows:] == 0xFFFFFFFF)   # untouched
    else:
        got_rows = np.fromfile(os.path.join(d, "recv.bin"), dtype=np.uint16).reshape(cap, h)
        assert np.array_equal(got_rows[:rows], oracle.dispatch_bf16(x, ora, k, H, relay))
        assert np.all(got_rows[rows:] == 0x5A5A)
    out = np.fromfile(os.path.join(d, "out.bin"), dtype=np.uint16)
    assert np.array_equal(out[:T * h].reshape(T, h), oracle.combine(y, ora, w))
    assert np.all(out[T * h:] == 0x5A5A)   # the 16 bytes past the output stay untouched
