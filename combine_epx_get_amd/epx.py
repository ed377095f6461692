"""Thin ctypes binding over libepx.so (the C ABI in include/epx.h).

Argument marshalling only: tensors are checked for dtype, shape, device and
contiguity, and their data pointers and the current HIP stream are passed to
the library. Every step of dispatch and combine runs in the library's HIP
kernels; there is no fallback of any kind. Importing this module fails when
the library has not been built (``python -m combine_epx_get_amd.build``).

PyTorch serves as the device allocator and stream provider only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional

import torch

# The release library, or the one EPX_LIBRARY names (e.g. the bounds-checked
# libepx_checked.so built beside it).
_LIB_PATH = os.environ.get("EPX_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libepx.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run `python -m combine_epx_get_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

MODE_PER_EXPERT = 0
MODE_HOST_RELAY = 1
BF16 = 0
FP8_E4M3 = 1
F32 = 2

STATUS = {0: "EPX_OK", 1: "EPX_ERR_ARG", 2: "EPX_ERR_INDEX", 3: "EPX_ERR_CAPACITY", 4: "EPX_ERR_DEVICE",
          5: "EPX_ERR_SCRATCH"}

LAYOUT_FIELDS = ["expert_count", "expert_offset", "rank_rows", "rank_tokens", "rank_offset",
                 "host_tokens", "host_offset", "slot", "row_token", "relay_slot", "relay_token",
                 "fanout_expert", "fanout_rank_mask", "relay_dst_rank", "totals", "group_offset",
                 "workspace"]
RELAY_FIELDS = ("relay_slot", "relay_token", "fanout_expert", "fanout_rank_mask")


class epx_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("num_tokens", "topk", "num_experts", "num_ranks", "num_hosts", "my_rank", "mode",
                 "num_groups")]


class epx_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYOUT_FIELDS]


_P = ctypes.c_void_p
_lib.epx_layout_sizes.argtypes = [ctypes.POINTER(epx_problem), ctypes.POINTER(ctypes.c_int64)]
_lib.epx_get_layout.argtypes = [ctypes.POINTER(epx_problem), _P, ctypes.POINTER(epx_layout), _P]
_lib.epx_dispatch.argtypes = [ctypes.POINTER(epx_problem), ctypes.POINTER(epx_layout), _P,
                              ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int64, _P]
_lib.epx_combine.argtypes = [ctypes.POINTER(epx_problem), ctypes.POINTER(epx_layout), _P,
                             ctypes.c_int64, _P, ctypes.c_int32, _P, _P]
_lib.epx_read_error.argtypes = [ctypes.POINTER(epx_layout), ctypes.POINTER(ctypes.c_int32), _P]
_lib.epx_f32_to_e4m3.argtypes = [_P, _P, ctypes.c_int64, _P]
_lib.epx_relay_fanout.argtypes = [ctypes.POINTER(epx_problem), ctypes.POINTER(epx_layout), _P, _P,
                                  ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int64, _P]
_lib.epx_combine_relay_partials.argtypes = [ctypes.POINTER(epx_problem), ctypes.POINTER(epx_layout), _P,
                                            ctypes.c_int64, _P, ctypes.c_int32, ctypes.c_int32, _P,
                                            ctypes.c_int64, _P]
_lib.epx_combine_relay_finish.argtypes = [ctypes.POINTER(epx_problem), ctypes.POINTER(epx_layout), _P,
                                          ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P]
_lib.epx_layout_dispatch.argtypes = [ctypes.POINTER(epx_problem), _P, ctypes.POINTER(epx_layout), _P,
                                     ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int64, _P]
_lib.epx_layout_dispatch_noalloc.argtypes = [ctypes.POINTER(epx_problem), _P, ctypes.POINTER(epx_layout), _P,
                                             ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int64, _P]
_lib.epx_dispatch_group.argtypes = [ctypes.POINTER(epx_problem), ctypes.POINTER(epx_layout), ctypes.c_int32,
                                    _P, ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int64, _P]
_lib.epx_combine_group.argtypes = [ctypes.POINTER(epx_problem), ctypes.POINTER(epx_layout), ctypes.c_int32,
                                   _P, ctypes.c_int64, _P, ctypes.c_int32, _P, _P, _P]
_lib.epx_plan_swaps.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32,
                                _P, _P, _P, _P, _P, _P]
_lib.epx_time_next_call.argtypes = [_P, _P]
_lib.epx_checked_violations.argtypes = [ctypes.POINTER(ctypes.c_int64), _P]
_lib.epx_status_string.argtypes = [ctypes.c_int]
_lib.epx_status_string.restype = ctypes.c_char_p
for _f in ("epx_layout_sizes", "epx_get_layout", "epx_dispatch", "epx_combine", "epx_read_error",
           "epx_f32_to_e4m3", "epx_relay_fanout", "epx_combine_relay_partials",
           "epx_combine_relay_finish", "epx_plan_swaps", "epx_dispatch_group", "epx_combine_group",
           "epx_layout_dispatch", "epx_time_next_call", "epx_layout_dispatch_noalloc",
           "epx_checked_violations"):
    getattr(_lib, _f).restype = ctypes.c_int
_lib.epx_abi_version.restype = ctypes.c_int32
NARRAYS = len(LAYOUT_FIELDS)


class EpxError(RuntimeError):
    def __init__(self, code: int, call: str):
        msg = _lib.epx_status_string(code).decode()
        super().__init__(f"{call}: {STATUS.get(code, code)} ({msg})")
        self.code = code


def _check(code: int, call: str) -> None:
    if code != 0:
        raise EpxError(code, call)


def abi_version() -> int:
    return int(_lib.epx_abi_version())


def make_problem(num_tokens: int, topk: int, num_experts: int, num_ranks: int, num_hosts: int,
                 my_rank: int = 0, mode: int = MODE_PER_EXPERT, num_groups: int = 1) -> epx_problem:
    return epx_problem(num_tokens, topk, num_experts, num_ranks, num_hosts, my_rank, mode, num_groups)


def epx_layout_sizes(problem: epx_problem) -> List[int]:
    sizes = (ctypes.c_int64 * NARRAYS)()
    _check(_lib.epx_layout_sizes(ctypes.byref(problem), sizes), "epx_layout_sizes")
    return list(sizes)


class Layout:
    """Device arrays of one layout (torch tensors) and the matching C struct."""

    def __init__(self, problem: epx_problem, device="cuda"):
        sizes = epx_layout_sizes(problem)
        relay = problem.mode == MODE_HOST_RELAY
        self.problem = problem
        self.tensors: Dict[str, torch.Tensor] = {}
        ptrs = []
        for name, n in zip(LAYOUT_FIELDS, sizes):
            if name in RELAY_FIELDS and not relay:
                ptrs.append(None)
                continue
            t = torch.empty(max(int(n), 1), dtype=torch.int32, device=device)
            self.tensors[name] = t
            ptrs.append(t.data_ptr())
        self.struct = epx_layout(*ptrs)
        self.sizes = dict(zip(LAYOUT_FIELDS, sizes))

    def __getitem__(self, name: str) -> torch.Tensor:
        return self.tensors[name][: self.sizes[name]]


# The current stream's raw handle: torch's own accessor costs about 0.1 us
# per call against about 3 us for torch.cuda.current_stream() (measured on
# MI355X), which is a third of a decode-sized call's host time.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    if stream is None:
        if _raw_current_stream is not None:
            return _raw_current_stream(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, dtype, name: str, ndim: Optional[int] = None) -> None:
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous {dtype} CUDA tensor")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: need {ndim} dimensions, got {tuple(t.shape)}")


def epx_get_layout(problem: epx_problem, topk_idx: torch.Tensor, layout: Layout, stream=None) -> None:
    _need(topk_idx, torch.int32, "topk_idx", 2)
    if tuple(topk_idx.shape) != (problem.num_tokens, problem.topk):
        raise ValueError(f"topk_idx shape {tuple(topk_idx.shape)} != (T, k)")
    _check(_lib.epx_get_layout(ctypes.byref(problem), topk_idx.data_ptr(), ctypes.byref(layout.struct),
                               _stream(stream)), "epx_get_layout")


def _dispatch_args(problem, x, out_dtype, recv, recv_scales):
    _need(x, torch.bfloat16, "x", 2)
    if x.shape[0] != problem.num_tokens:
        raise ValueError("x: first dimension must be num_tokens")
    hidden = x.shape[1]
    if out_dtype == BF16:
        _need(recv, torch.bfloat16, "recv", 2)
        scales_ptr = None
    else:
        _need(recv, torch.uint8, "recv", 2)
        _need(recv_scales, torch.float32, "recv_scales", 2)
        if recv_scales.shape != (recv.shape[0], hidden // 128):
            raise ValueError("recv_scales: need [capacity_rows, hidden/128]")
        scales_ptr = recv_scales.data_ptr()
    if recv.shape[1] != hidden:
        raise ValueError("recv: second dimension must be hidden")
    return hidden, scales_ptr


def epx_dispatch(problem: epx_problem, layout: Layout, x: torch.Tensor, out_dtype: int,
                 recv: torch.Tensor, recv_scales: Optional[torch.Tensor] = None, stream=None) -> None:
    hidden, scales_ptr = _dispatch_args(problem, x, out_dtype, recv, recv_scales)
    _check(_lib.epx_dispatch(ctypes.byref(problem), ctypes.byref(layout.struct), x.data_ptr(), hidden,
                             out_dtype, recv.data_ptr(), scales_ptr, recv.shape[0], _stream(stream)),
           "epx_dispatch")


def epx_layout_dispatch(problem: epx_problem, topk_idx: torch.Tensor, layout: Layout, x: torch.Tensor,
                        out_dtype: int, recv: torch.Tensor, recv_scales: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """epx_get_layout then epx_dispatch in one call: one launch for decode-sized
    batches, the row assignment and the copies in one launch for larger ones."""
    _need(topk_idx, torch.int32, "topk_idx", 2)
    if tuple(topk_idx.shape) != (problem.num_tokens, problem.topk):
        raise ValueError(f"topk_idx shape {tuple(topk_idx.shape)} != (T, k)")
    hidden, scales_ptr = _dispatch_args(problem, x, out_dtype, recv, recv_scales)
    _check(_lib.epx_layout_dispatch(ctypes.byref(problem), topk_idx.data_ptr(), ctypes.byref(layout.struct),
                                    x.data_ptr(), hidden, out_dtype, recv.data_ptr(), scales_ptr,
                                    recv.shape[0], _stream(stream)),
           "epx_layout_dispatch")


def epx_layout_dispatch_noalloc(problem: epx_problem, topk_idx: torch.Tensor, layout, x: torch.Tensor,
                                out_dtype: int, recv: torch.Tensor, recv_scales: Optional[torch.Tensor] = None,
                                stream=None) -> None:
    """epx_layout_dispatch with the library's static scratch in place of the
    layout's workspace. `layout` is a Layout or an epx_layout struct (its
    workspace may be NULL)."""
    _need(topk_idx, torch.int32, "topk_idx", 2)
    if tuple(topk_idx.shape) != (problem.num_tokens, problem.topk):
        raise ValueError(f"topk_idx shape {tuple(topk_idx.shape)} != (T, k)")
    hidden, scales_ptr = _dispatch_args(problem, x, out_dtype, recv, recv_scales)
    struct = layout.struct if isinstance(layout, Layout) else layout
    _check(_lib.epx_layout_dispatch_noalloc(ctypes.byref(problem), topk_idx.data_ptr(), ctypes.byref(struct),
                                            x.data_ptr(), hidden, out_dtype, recv.data_ptr(), scales_ptr,
                                            recv.shape[0], _stream(stream)),
           "epx_layout_dispatch_noalloc")


def epx_dispatch_group(problem: epx_problem, layout: Layout, group: int, x: torch.Tensor, out_dtype: int,
                       recv: torch.Tensor, recv_scales: Optional[torch.Tensor] = None, stream=None) -> None:
    """Dispatch of one expert group's rows (recv is the whole [T*k, ...] buffer)."""
    hidden, scales_ptr = _dispatch_args(problem, x, out_dtype, recv, recv_scales)
    _check(_lib.epx_dispatch_group(ctypes.byref(problem), ctypes.byref(layout.struct), group, x.data_ptr(),
                                   hidden, out_dtype, recv.data_ptr(), scales_ptr, recv.shape[0],
                                   _stream(stream)),
           "epx_dispatch_group")


def epx_combine(problem: epx_problem, layout: Layout, y: torch.Tensor, topk_weights: torch.Tensor,
                out: torch.Tensor, stream=None) -> None:
    _need(y, torch.bfloat16, "y", 2)
    _need(topk_weights, torch.float32, "topk_weights", 2)
    _need(out, torch.bfloat16, "out", 2)
    if tuple(topk_weights.shape) != (problem.num_tokens, problem.topk):
        raise ValueError("topk_weights: need [T, k]")
    if tuple(out.shape) != (problem.num_tokens, y.shape[1]):
        raise ValueError("out: need [T, hidden]")
    _check(_lib.epx_combine(ctypes.byref(problem), ctypes.byref(layout.struct), y.data_ptr(), y.shape[0],
                            topk_weights.data_ptr(), y.shape[1], out.data_ptr(), _stream(stream)),
           "epx_combine")


def epx_combine_group(problem: epx_problem, layout: Layout, group: int, y: torch.Tensor,
                      topk_weights: torch.Tensor, carry: Optional[torch.Tensor], out: torch.Tensor,
                      stream=None) -> None:
    """One expert group's combine; call for groups 0..m-1 in order on one
    float32 [T, hidden] carry."""
    _need(y, torch.bfloat16, "y", 2)
    _need(topk_weights, torch.float32, "topk_weights", 2)
    _need(out, torch.bfloat16, "out", 2)
    if tuple(topk_weights.shape) != (problem.num_tokens, problem.topk):
        raise ValueError("topk_weights: need [T, k]")
    if tuple(out.shape) != (problem.num_tokens, y.shape[1]):
        raise ValueError("out: need [T, hidden]")
    if carry is not None:
        _need(carry, torch.float32, "carry", 2)
        if tuple(carry.shape) != tuple(out.shape):
            raise ValueError("carry: need [T, hidden]")
    _check(_lib.epx_combine_group(ctypes.byref(problem), ctypes.byref(layout.struct), group, y.data_ptr(),
                                  y.shape[0], topk_weights.data_ptr(), y.shape[1],
                                  carry.data_ptr() if carry is not None else None, out.data_ptr(),
                                  _stream(stream)),
           "epx_combine_group")


def epx_read_error(layout: Layout, stream=None) -> int:
    """Synchronising read of the layout's bad-id count (0 = all ids valid)."""
    bad = ctypes.c_int32(0)
    code = _lib.epx_read_error(ctypes.byref(layout.struct), ctypes.byref(bad), _stream(stream))
    if code not in (0, 2):
        _check(code, "epx_read_error")
    return int(bad.value)


def epx_time_next_call(start_event: Optional[int], stop_event: Optional[int]) -> None:
    """Bind two raw hipEvent_t handles to the kernels of the next library call
    from this thread (start: its first kernel's start, stop: its last kernel's
    end); None, None disarms."""
    _check(_lib.epx_time_next_call(start_event, stop_event), "epx_time_next_call")


def epx_checked_violations(stream=None) -> int:
    """Bounds-checked library only: accesses its checks skipped since the last
    call (synchronises the stream and resets the count)."""
    n = ctypes.c_int64(-1)
    _check(_lib.epx_checked_violations(ctypes.byref(n), _stream(stream)), "epx_checked_violations")
    return int(n.value)


def epx_f32_to_e4m3(inp: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _need(inp, torch.float32, "in")
    _need(out, torch.uint8, "out")
    if inp.numel() != out.numel():
        raise ValueError("in/out sizes differ")
    _check(_lib.epx_f32_to_e4m3(inp.data_ptr(), out.data_ptr(), inp.numel(), _stream(stream)),
           "epx_f32_to_e4m3")


def epx_relay_fanout(problem: epx_problem, layout: Layout, relay_rows: torch.Tensor, recv: torch.Tensor,
                     relay_scales: Optional[torch.Tensor] = None, recv_scales: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """Relay rows -> per-expert rows (bf16 rows, or fp8 codes with scales)."""
    fp8 = relay_rows.dtype == torch.uint8
    _need(relay_rows, torch.uint8 if fp8 else torch.bfloat16, "relay_rows", 2)
    _need(recv, relay_rows.dtype, "recv", 2)
    hidden = relay_rows.shape[1]
    if recv.shape[1] != hidden:
        raise ValueError("recv: hidden differs from relay_rows")
    if fp8:
        _need(relay_scales, torch.float32, "relay_scales", 2)
        _need(recv_scales, torch.float32, "recv_scales", 2)
        # the kernel reads relay_scales[r] for relay rows r and writes
        # recv_scales[o] for per-expert rows o: one scale per 128 channels
        if tuple(relay_scales.shape) != (relay_rows.shape[0], hidden // 128):
            raise ValueError("relay_scales: need [relay_rows, hidden/128]")
        if tuple(recv_scales.shape) != (recv.shape[0], hidden // 128):
            raise ValueError("recv_scales: need [capacity_rows, hidden/128]")
    _check(_lib.epx_relay_fanout(ctypes.byref(problem), ctypes.byref(layout.struct), relay_rows.data_ptr(),
                                 relay_scales.data_ptr() if fp8 else None, relay_rows.shape[0], hidden,
                                 FP8_E4M3 if fp8 else BF16, recv.data_ptr(),
                                 recv_scales.data_ptr() if fp8 else None, recv.shape[0], _stream(stream)),
           "epx_relay_fanout")


def epx_combine_relay_partials(problem: epx_problem, layout: Layout, y: torch.Tensor,
                               topk_weights: torch.Tensor, partials: torch.Tensor, stream=None) -> None:
    """Per relay row fp32 (float32 tensor) or bf16 (bfloat16 tensor) partial sums."""
    _need(y, torch.bfloat16, "y", 2)
    _need(topk_weights, torch.float32, "topk_weights", 2)
    if partials.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("partials: float32 or bfloat16")
    _need(partials, partials.dtype, "partials", 2)
    if partials.shape[1] != y.shape[1]:
        raise ValueError("partials: hidden differs from y")
    pd = F32 if partials.dtype == torch.float32 else BF16
    _check(_lib.epx_combine_relay_partials(ctypes.byref(problem), ctypes.byref(layout.struct), y.data_ptr(),
                                           y.shape[0], topk_weights.data_ptr(), y.shape[1], pd,
                                           partials.data_ptr(), partials.shape[0], _stream(stream)),
           "epx_combine_relay_partials")


def epx_combine_relay_finish(problem: epx_problem, layout: Layout, partials: torch.Tensor,
                             out: torch.Tensor, stream=None) -> None:
    if partials.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("partials: float32 or bfloat16")
    _need(partials, partials.dtype, "partials", 2)
    _need(out, torch.bfloat16, "out", 2)
    if tuple(out.shape) != (problem.num_tokens, partials.shape[1]):
        raise ValueError("out: need [T, hidden]")
    pd = F32 if partials.dtype == torch.float32 else BF16
    _check(_lib.epx_combine_relay_finish(ctypes.byref(problem), ctypes.byref(layout.struct),
                                         partials.data_ptr(), partials.shape[0], pd, partials.shape[1],
                                         out.data_ptr(), _stream(stream)),
           "epx_combine_relay_finish")


def epx_plan_swaps(num_experts: int, num_ranks: int, num_hosts: int, expert_count: torch.Tensor,
                   slot_expert: torch.Tensor, tau: int, out: Optional[dict] = None, stream=None) -> dict:
    """Per-step intra-host expert swaps. Returns (and fills, if given) the
    int32 tensors slot_expert [E], load_before [R], load_after [R],
    swaps [H * (R/H)//2, 7] and host_bad [H]."""
    E, R, H = num_experts, num_ranks, num_hosts
    _need(expert_count, torch.int32, "expert_count", 1)
    _need(slot_expert, torch.int32, "slot_expert", 1)
    if expert_count.numel() < E or slot_expert.numel() != E:
        raise ValueError("expert_count needs >= E entries, slot_expert exactly E")
    npair = H * ((R // H) // 2) if H > 0 and R % H == 0 else 0
    shapes = {"slot_expert": (E,), "load_before": (R,), "load_after": (R,), "swaps": (npair, 7),
              "host_bad": (H,)}
    if out is None:
        out = {n: torch.empty(sh, dtype=torch.int32, device=slot_expert.device) for n, sh in shapes.items()}
    for n, sh in shapes.items():
        _need(out[n], torch.int32, n)
        if tuple(out[n].shape) != sh:
            raise ValueError(f"{n}: need shape {sh}")
    _check(_lib.epx_plan_swaps(E, R, H, expert_count.data_ptr(), slot_expert.data_ptr(), tau,
                               out["slot_expert"].data_ptr(), out["load_before"].data_ptr(),
                               out["load_after"].data_ptr(), out["swaps"].data_ptr() if npair else None,
                               out["host_bad"].data_ptr(), _stream(stream)),
           "epx_plan_swaps")
    return out


def relay_capacity(problem: epx_problem) -> int:
    return problem.num_tokens * min(problem.topk, problem.num_hosts)
