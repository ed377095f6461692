"""CPU oracle for MoE expert-parallel dispatch/combine (ctypes over epx_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product library never imports,
links or executes anything here, and nothing here imports the product.

Each wrapper takes and returns numpy arrays; the arithmetic lives in
``epx_oracle.c`` (plain scalar loops written from the definitions in the
digest "Balancing and Beyond: Communication-Centric Optimizations in Expert
Parallelism", sections 1-3, and in the DeepEP issue "[GH-ISSUE #250]
Profiling when rank unbalance").

Parity status of each function (what pins it, in tests/test_oracle_*.py):
  layout         -- brute-force enumeration of the order definitions on small
                    inputs; invariants; the copy-count closed forms of digest
                    section 3.2; the worked example of the DeepEP issue.
  dispatch_bf16  -- row equality with the token's row (definition) on small inputs.
  dispatch_fp8   -- converter exhaustive vs torch's float8_e4m3fn cast; block
                    properties (amax code is 448, error bound of a 3-bit mantissa);
                    scale and quotient by golden blocks whose codes are derived in
                    exact rational arithmetic (s = RNE32(amax/448), RNE32(x/s)) and
                    that x*(448/amax), x*(1/s) and amax*(1/448) all fail
                    (tests/golden/fp8_quotient_blocks.json).
  combine        -- float64 sum within the float32 error bound; exact special cases.
  relay_fanout   -- equals the per-expert dispatch row for row (two independent
                    definitions); membership by host brute force.
  relay_partials / relay_finish -- one host reduces to the flat combine bit for
                    bit; partial membership by exact power-of-two tagging;
                    float64 sum within the float32 bound.
  layout_grouped -- m = 1 equals the plain layout; brute-force sort by
                    (group, expert, token, j) on small inputs; block offsets.
  group_slots    -- the union over groups is the full slot array, groups disjoint.
  combine_grouped -- m = 1 equals the plain combine bit for bit; an order
                    case whose float32 result differs between j order and
                    group order (exact expected values); float64 bound.
  plan_swaps     -- the worked example of digest Figure 2(b) (160/100 -> 130/130);
                    optimality of every chosen swap by enumeration; pairing,
                    threshold and conservation invariants.
  Where the pages leave a choice open (relay row order, the all-zero block,
  the fma order of combine), the oracle takes the reading recorded in the
  design notes, and tests pin that reading: the row order by brute force, the
  all-zero and signed-zero blocks by exact cases, the fma order by exact order
  cases and planted mutants (tests/test_oracle_mutants.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "epx_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11"]

_lib: Optional[ctypes.CDLL] = None


def build(out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (plain C, libm only)."""
    cmd = ["gcc", *_CFLAGS, *extra_flags, "-o", out, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = _LIB) -> ctypes.CDLL:
    """Load the oracle library, compiling it first if it is missing or stale."""
    global _lib
    if path == _LIB and _lib is not None:
        return _lib
    if (not os.path.exists(path)) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        if path != _LIB:
            raise FileNotFoundError(path)
        build(path)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.oracle_layout.argtypes = [i32] * 7 + [P] * 16
    lib.oracle_layout.restype = ctypes.c_int
    lib.oracle_dispatch_bf16.argtypes = [i32] * 5 + [P] * 4
    lib.oracle_dispatch_bf16.restype = ctypes.c_int
    lib.oracle_dispatch_fp8.argtypes = [i32] * 5 + [P] * 5
    lib.oracle_dispatch_fp8.restype = ctypes.c_int
    lib.oracle_combine.argtypes = [i32] * 3 + [P] * 4
    lib.oracle_combine.restype = ctypes.c_int
    lib.oracle_relay_fanout.argtypes = [i32] * 5 + [ctypes.c_int64, i32] + [P] * 7
    lib.oracle_relay_fanout.restype = ctypes.c_int
    lib.oracle_relay_partials.argtypes = [i32] * 7 + [P] * 6
    lib.oracle_relay_partials.restype = ctypes.c_int
    lib.oracle_relay_finish.argtypes = [i32] * 4 + [P] * 3
    lib.oracle_relay_finish.restype = ctypes.c_int
    lib.oracle_layout_grouped.argtypes = [i32] * 5 + [P] * 7
    lib.oracle_layout_grouped.restype = ctypes.c_int
    lib.oracle_group_slots.argtypes = [i32] * 6 + [P] * 3
    lib.oracle_group_slots.restype = ctypes.c_int
    lib.oracle_combine_grouped.argtypes = [i32] * 6 + [P] * 5
    lib.oracle_combine_grouped.restype = ctypes.c_int
    lib.oracle_plan_swaps.argtypes = [i32] * 3 + [P] * 2 + [i32] + [P] * 5
    lib.oracle_plan_swaps.restype = ctypes.c_int
    for name in ("oracle_f32_to_e4m3_array", "oracle_f32_to_bf16_array", "oracle_e4m3_to_f32_array"):
        getattr(lib, name).argtypes = [P, P, ctypes.c_int64]
        getattr(lib, name).restype = None
    if path == _LIB:
        _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


def layout(topk_idx: np.ndarray, num_experts: int, num_ranks: int, num_hosts: int,
           my_rank: int = 0, relay: bool = False, lib: Optional[ctypes.CDLL] = None) -> dict:
    """All layout arrays for one source rank (see oracle_layout in epx_oracle.c)."""
    lib = lib or load()
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    E, R, H = num_experts, num_ranks, num_hosts
    cap = T * min(k, H)
    out = {
        "expert_count": np.zeros(E, np.int32), "expert_offset": np.zeros(E + 1, np.int32),
        "rank_rows": np.zeros(R, np.int32), "rank_tokens": np.zeros(R, np.int32),
        "rank_offset": np.zeros(R + 1, np.int32), "host_tokens": np.zeros(H, np.int32),
        "host_offset": np.zeros(H + 1, np.int32), "slot": np.zeros(T * k, np.int32),
        "row_token": np.zeros(T * k, np.int32), "relay_slot": np.zeros(T * H, np.int32),
        "relay_token": np.zeros(cap, np.int32), "fanout_expert": np.zeros(cap * k, np.int32),
        "fanout_rank_mask": np.zeros(cap, np.uint32), "relay_dst_rank": np.zeros(H, np.int32),
        "totals": np.zeros(4, np.int32),
    }
    rc = lib.oracle_layout(T, k, E, R, H, my_rank, int(relay), _p(idx),
                           *[_p(out[n]) for n in (
                               "expert_count", "expert_offset", "rank_rows", "rank_tokens",
                               "rank_offset", "host_tokens", "host_offset", "slot", "row_token",
                               "relay_slot", "relay_token", "fanout_expert", "fanout_rank_mask",
                               "relay_dst_rank", "totals")])
    out["status"] = rc
    if rc != 0:
        raise OracleError(rc, "oracle_layout")
    if not relay:
        for n in ("relay_slot", "relay_token", "fanout_expert", "fanout_rank_mask"):
            out.pop(n)
    return out


def dispatch_bf16(x_bits: np.ndarray, lay: dict, topk: int, num_hosts: int, relay: bool,
                  rows: Optional[int] = None, lib=None, out: Optional[np.ndarray] = None) -> np.ndarray:
    """recv rows (uint16 bf16 bits) for per-expert or relay mode. With `out`
    (a C-contiguous uint16 [rows, h] array) the rows are written there: x and
    the slot arrays may then be a slice of the tokens, whose rows are still
    addressed by the full layout's row numbers."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, hidden = x.shape
    if rows is None:
        rows = int(lay["totals"][1] if relay else lay["totals"][0])
    recv = np.zeros((max(rows, 0), hidden), np.uint16) if out is None else out
    slot = lay["slot"]
    rslot = lay.get("relay_slot", np.zeros(1, np.int32)) if relay else np.zeros(1, np.int32)
    rc = lib.oracle_dispatch_bf16(T, topk, num_hosts, int(relay), hidden, _p(slot), _p(rslot),
                                  _p(x), _p(recv))
    if rc != 0:
        raise OracleError(rc, "oracle_dispatch_bf16")
    return recv


def dispatch_fp8(x_bits: np.ndarray, lay: dict, topk: int, num_hosts: int, relay: bool,
                 rows: Optional[int] = None, lib=None, out=None):
    """(codes uint8 [rows, h], scales float32 [rows, h/128]). With `out` =
    (codes, scales) arrays the rows are written there (as dispatch_bf16)."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, hidden = x.shape
    if rows is None:
        rows = int(lay["totals"][1] if relay else lay["totals"][0])
    if out is None:
        q = np.zeros((rows, hidden), np.uint8)
        sc = np.zeros((rows, hidden // 128), np.float32)
    else:
        q, sc = out
    slot = lay["slot"]
    rslot = lay.get("relay_slot", np.zeros(1, np.int32)) if relay else np.zeros(1, np.int32)
    rc = lib.oracle_dispatch_fp8(T, topk, num_hosts, int(relay), hidden, _p(slot), _p(rslot),
                                 _p(x), _p(q), _p(sc))
    if rc != 0:
        raise OracleError(rc, "oracle_dispatch_fp8")
    return q, sc


def combine(y_bits: np.ndarray, lay: dict, topk_weights: np.ndarray, lib=None,
            out: Optional[np.ndarray] = None) -> np.ndarray:
    """out [T, h] uint16 bf16 bits. With `out` (C-contiguous uint16 [T, h] for
    the T rows of topk_weights) the result is written there: topk_weights and
    lay["slot"] may then be a slice of the tokens, y stays whole."""
    lib = lib or load()
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    T, k = w.shape
    hidden = y.shape[1]
    if out is None:
        out = np.zeros((T, hidden), np.uint16)
    assert out.shape == (T, hidden) and out.dtype == np.uint16
    rc = lib.oracle_combine(T, k, hidden, _p(lay["slot"]), _p(w), _p(y), _p(out))
    if rc != 0:
        raise OracleError(rc, "oracle_combine")
    return out


def layout_grouped(topk_idx: np.ndarray, num_experts: int, num_ranks: int, num_groups: int,
                   lib=None) -> dict:
    """Per-expert layout with rows ordered by (expert group, expert, token, j)."""
    lib = lib or load()
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    E, R, m = num_experts, num_ranks, num_groups
    out = {"expert_count": np.zeros(E, np.int32), "expert_offset": np.zeros(E + 1, np.int32),
           "group_offset": np.zeros(m * R + 1, np.int32), "slot": np.zeros(T * k, np.int32),
           "row_token": np.zeros(T * k, np.int32), "totals": np.zeros(4, np.int32)}
    rc = lib.oracle_layout_grouped(T, k, E, R, m, _p(idx), *[_p(out[n]) for n in (
        "expert_count", "expert_offset", "group_offset", "slot", "row_token", "totals")])
    if rc != 0:
        raise OracleError(rc, "oracle_layout_grouped")
    return out


def group_slots(topk_idx: np.ndarray, lay: dict, num_experts: int, num_ranks: int, num_groups: int,
                group: int, lib=None) -> np.ndarray:
    """slot[t, j] where expert idx[t, j] is in the group, -1 elsewhere."""
    lib = lib or load()
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    out = np.zeros(T * k, np.int32)
    rc = lib.oracle_group_slots(T, k, num_experts, num_ranks, num_groups, group, _p(idx),
                                _p(lay["slot"]), _p(out))
    if rc != 0:
        raise OracleError(rc, "oracle_group_slots")
    return out


def dispatch_group(x_bits: np.ndarray, lay: dict, topk_idx: np.ndarray, num_experts: int,
                   num_ranks: int, num_groups: int, group: int, fp8: bool = False, lib=None):
    """Rows [T*k, ...] of one group's dispatch (other groups' rows zero): the
    per-expert dispatch over that group's destinations only."""
    k = topk_idx.shape[1]
    sub = {"slot": group_slots(topk_idx, lay, num_experts, num_ranks, num_groups, group, lib),
           "totals": lay["totals"]}
    if fp8:
        return dispatch_fp8(x_bits, sub, k, 1, False, lib=lib)
    return dispatch_bf16(x_bits, sub, k, 1, False, lib=lib)


def combine_grouped(y_bits: np.ndarray, lay: dict, topk_idx: np.ndarray, topk_weights: np.ndarray,
                    num_experts: int, num_ranks: int, num_groups: int, lib=None) -> np.ndarray:
    """out [T, h] bf16 bits after the m group combines (float32 carried across groups)."""
    lib = lib or load()
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = w.shape
    hidden = y.shape[1]
    out = np.zeros((T, hidden), np.uint16)
    rc = lib.oracle_combine_grouped(T, k, num_experts, num_ranks, num_groups, hidden, _p(idx),
                                    _p(lay["slot"]), _p(w), _p(y), _p(out))
    if rc != 0:
        raise OracleError(rc, "oracle_combine_grouped")
    return out


def relay_fanout(relay_rows: np.ndarray, lay: dict, topk_idx: np.ndarray, num_experts: int,
                 num_ranks: int, num_hosts: int, relay_scales: Optional[np.ndarray] = None,
                 lib=None):
    """Per-expert rows [T*k, ...] (same dtype as relay_rows) built from relay
    rows by the fan-out definition; with relay_scales also the scales."""
    lib = lib or load()
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    rows = np.ascontiguousarray(relay_rows)
    row_bytes = rows.shape[1] * rows.itemsize
    recv = np.zeros((T * k,) + rows.shape[1:], rows.dtype)
    nsc = 0 if relay_scales is None else relay_scales.shape[1]
    sc_in = np.ascontiguousarray(relay_scales if relay_scales is not None else np.zeros((1, 1), np.float32),
                                 dtype=np.float32)
    sc_out = np.zeros((T * k, max(nsc, 1)), np.float32)
    rc = lib.oracle_relay_fanout(T, k, num_experts, num_ranks, num_hosts, row_bytes, nsc, _p(idx),
                                 _p(lay["slot"]), _p(lay["relay_slot"]), _p(rows), _p(sc_in), _p(recv),
                                 _p(sc_out))
    if rc != 0:
        raise OracleError(rc, "oracle_relay_fanout")
    return (recv, sc_out[:, :nsc]) if relay_scales is not None else recv


def relay_partials(y_bits: np.ndarray, lay: dict, topk_idx: np.ndarray, topk_weights: np.ndarray,
                   num_experts: int, num_ranks: int, num_hosts: int, bf16: bool = False, lib=None):
    """Per relay row fp32 (or bf16-bit) partial sums [relay_rows, h]."""
    lib = lib or load()
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    hidden = y.shape[1]
    rows = int(lay["totals"][1])
    part = np.zeros((rows, hidden), np.uint16 if bf16 else np.float32)
    rc = lib.oracle_relay_partials(T, k, num_experts, num_ranks, num_hosts, hidden, int(bf16), _p(idx),
                                   _p(lay["slot"]), _p(lay["relay_slot"]), _p(w), _p(y), _p(part))
    if rc != 0:
        raise OracleError(rc, "oracle_relay_partials")
    return part


def relay_finish(partials: np.ndarray, lay: dict, num_tokens: int, num_hosts: int, lib=None) -> np.ndarray:
    """out [T, h] bf16 bits from the per-host partials."""
    lib = lib or load()
    part = np.ascontiguousarray(partials)
    bf16 = part.dtype == np.uint16
    hidden = part.shape[1]
    out = np.zeros((num_tokens, hidden), np.uint16)
    rc = lib.oracle_relay_finish(num_tokens, num_hosts, hidden, int(bf16), _p(lay["relay_slot"]), _p(part),
                                 _p(out))
    if rc != 0:
        raise OracleError(rc, "oracle_relay_finish")
    return out


def plan_swaps(counts: np.ndarray, num_ranks: int, num_hosts: int, tau: int,
               slot_expert: Optional[np.ndarray] = None, lib=None) -> dict:
    """Intra-host swap plan (see oracle_plan_swaps). Returns the placement
    after the swaps, loads before/after, the per-pair records [.., 7] and
    host_bad [H] (ids outside [0, E) per host; such a host is not planned)."""
    lib = lib or load()
    c = np.ascontiguousarray(counts, dtype=np.int32)
    E, R, H = c.size, num_ranks, num_hosts
    se = np.arange(E, dtype=np.int32) if slot_expert is None else np.ascontiguousarray(slot_expert, np.int32)
    out = np.zeros(E, np.int32)
    lb = np.zeros(R, np.int32)
    la = np.zeros(R, np.int32)
    npair = (R // H) // 2
    sw = np.full((H * max(npair, 0), 7), -1, np.int32)
    hb = np.zeros(max(H, 1), np.int32)
    rc = lib.oracle_plan_swaps(E, R, H, _p(c), _p(se), tau, _p(out), _p(lb), _p(la),
                               _p(sw if sw.size else np.zeros(7, np.int32)), _p(hb))
    if rc != 0:
        raise OracleError(rc, "oracle_plan_swaps")
    return {"slot_expert": out, "load_before": lb, "load_after": la, "swaps": sw, "host_bad": hb[:H]}


def f32_to_e4m3(a: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib.oracle_f32_to_e4m3_array(_p(a), _p(out), a.size)
    return out


def e4m3_to_f32(q: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(q.shape, np.float32)
    lib.oracle_e4m3_to_f32_array(_p(q), _p(out), q.size)
    return out


def f32_to_bf16(a: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    lib.oracle_f32_to_bf16_array(_p(a), _p(out), a.size)
    return out


def expert_of_rows(lay: dict) -> np.ndarray:
    """Expert id of each per-expert row, read off the offsets (row r belongs to
    the expert e with expert_offset[e] <= r < expert_offset[e+1])."""
    off = lay["expert_offset"]
    rows = int(off[-1])
    return (np.searchsorted(off, np.arange(rows), side="right") - 1).astype(np.int32)
