"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

epx_api.hip (every entry point's argument checks, sizes and status strings)
is rebuilt with the sanitizers on its host code only (hipcc -Xarch_host
-fsanitize=...; the device code is built as usual), linked with the
library's other objects into a small driver program, and the driver calls
every entry point on every host-side error path: null and misaligned
pointers, bad geometry, unsupported sizes, short capacities, a problem too
large for the no-alloc scratch, bad measurement-hook arguments. Each call
must return its documented status. None of these calls reaches a HIP launch
(a call that fails a host check launches nothing), so the driver needs no
GPU; the pointers it passes point into a host buffer and are only checked
for null and alignment. Any out-of-bounds access or undefined arithmetic in
the host code aborts the driver.
"""
import glob
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_epx_get_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DRIVER = r'''
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "epx.h"

static int checks = 0;
#define EXPECT(call, want)                                                                    \
    do {                                                                                      \
        const int got_ = (int)(call);                                                         \
        if (got_ != (int)(want)) {                                                            \
            std::printf("FAIL line %d: %s -> %d, want %d\n", __LINE__, #call, got_, (int)(want)); \
            return 1;                                                                         \
        }                                                                                     \
        ++checks;                                                                             \
    } while (0)

alignas(256) static unsigned char buf[1 << 16];

static epx_problem prob(int T, int k, int E, int R, int H, int s, int mode, int m = 1)
{
    epx_problem p;
    p.num_tokens = T; p.topk = k; p.num_experts = E; p.num_ranks = R; p.num_hosts = H;
    p.my_rank = s; p.mode = mode; p.num_groups = m;
    return p;
}

static epx_layout layout(bool relay)
{
    epx_layout L;
    int32_t *a = (int32_t *)buf;
    L.expert_count = a; L.expert_offset = a; L.rank_rows = a; L.rank_tokens = a;
    L.rank_offset = a; L.host_tokens = a; L.host_offset = a; L.slot = a; L.row_token = a;
    L.relay_slot = relay ? a : nullptr; L.relay_token = relay ? a : nullptr;
    L.fanout_expert = relay ? a : nullptr; L.fanout_rank_mask = relay ? (uint32_t *)a : nullptr;
    L.relay_dst_rank = a; L.totals = a; L.group_offset = a; L.workspace = a;
    return L;
}

int main()
{
    void *A = buf;                 // 256-byte aligned
    void *A2 = buf + 2, *A4 = buf + 4, *A8 = buf + 8;
    const epx_problem p = prob(64, 2, 16, 4, 2, 0, EPX_MODE_PER_EXPERT);
    const epx_problem pr = prob(64, 2, 16, 4, 2, 0, EPX_MODE_HOST_RELAY);
    const epx_problem pg = prob(64, 2, 16, 4, 2, 0, EPX_MODE_PER_EXPERT, 2);
    epx_layout L = layout(false), LR = layout(true);
    int64_t sizes[EPX_LAYOUT_NARRAYS];

    // sizes and geometry
    EXPECT(epx_layout_sizes(&p, sizes), EPX_OK);
    EXPECT(sizes[EPX_L_SLOT] == 128, 1);
    EXPECT(epx_layout_sizes(nullptr, sizes), EPX_ERR_ARG);
    EXPECT(epx_layout_sizes(&p, nullptr), EPX_ERR_ARG);
    const epx_problem bad[] = {
        prob(-1, 2, 16, 4, 2, 0, 0), prob((1 << 24) + 1, 2, 16, 4, 2, 0, 0), prob(64, 0, 16, 4, 2, 0, 0),
        prob(64, 65, 128, 4, 2, 0, 0), prob(64, 2, 0, 1, 1, 0, 0), prob(64, 2, 4096, 4, 2, 0, 0),
        prob(64, 2, 16, 0, 1, 0, 0), prob(64, 2, 16, 4, 0, 0, 0), prob(64, 2, 128, 128, 128, 0, 0),
        prob(64, 2, 16, 3, 1, 0, 0), prob(64, 2, 16, 4, 3, 0, 0), prob(64, 17, 16, 4, 2, 0, 0),
        prob(64, 2, 128, 64, 1, 0, 0), prob(64, 2, 16, 4, 2, -1, 0), prob(64, 2, 16, 4, 2, 4, 0),
        prob(64, 2, 16, 4, 2, 0, 7),
        prob(64, 2, 16, 4, 2, 0, 0, 3), prob(64, 2, 16, 4, 2, 0, EPX_MODE_HOST_RELAY, 2),
        prob(64, 2, 16, 4, 2, 0, 0, -1)};
    for (const epx_problem &b : bad) {
        EXPECT(epx_layout_sizes(&b, sizes), EPX_ERR_ARG);
        EXPECT(epx_get_layout(&b, (const int32_t *)A, &L, nullptr), EPX_ERR_ARG);
        EXPECT(epx_dispatch(&b, &L, A, 256, EPX_BF16, A, nullptr, 1 << 20, nullptr), EPX_ERR_ARG);
        EXPECT(epx_combine(&b, &L, A, 1 << 20, (const float *)A, 256, A, nullptr), EPX_ERR_ARG);
        EXPECT(epx_layout_dispatch(&b, (const int32_t *)A, &L, A, 256, EPX_BF16, A, nullptr, 1 << 20, nullptr),
               EPX_ERR_ARG);
        EXPECT(epx_layout_dispatch_noalloc(&b, (const int32_t *)A, &L, A, 256, EPX_BF16, A, nullptr, 1 << 20,
                                           nullptr), EPX_ERR_ARG);
    }

    // layout: the struct, its arrays, alignment, the routing ids
    EXPECT(epx_get_layout(&p, (const int32_t *)A, nullptr, nullptr), EPX_ERR_ARG);
    EXPECT(epx_get_layout(&p, nullptr, &L, nullptr), EPX_ERR_ARG);
    EXPECT(epx_get_layout(&p, (const int32_t *)A2, &L, nullptr), EPX_ERR_ARG);
    EXPECT(epx_get_layout(&pr, (const int32_t *)A, &L, nullptr), EPX_ERR_ARG);   // relay arrays missing
    {
        epx_layout M = L;
        M.slot = nullptr;
        EXPECT(epx_get_layout(&p, (const int32_t *)A, &M, nullptr), EPX_ERR_ARG);
        M = L;
        M.totals = (int32_t *)A2;
        EXPECT(epx_get_layout(&p, (const int32_t *)A, &M, nullptr), EPX_ERR_ARG);
        M = L;
        M.workspace = (int32_t *)A8;
        EXPECT(epx_get_layout(&p, (const int32_t *)A, &M, nullptr), EPX_ERR_ARG);
    }

    // dispatch: dtype, hidden, capacity, pointers, alignment, scales, groups
    EXPECT(epx_dispatch(&p, &L, A, 256, 9, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch(&p, &L, A, 4, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch(&p, &L, A, 252, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch(&p, &L, A, 264, EPX_FP8_E4M3, A, (float *)A, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch(&p, &L, A, 256, EPX_BF16, A, nullptr, 127, nullptr), EPX_ERR_CAPACITY);
    EXPECT(epx_dispatch(&pr, &LR, A, 256, EPX_BF16, A, nullptr, 127, nullptr), EPX_ERR_CAPACITY);
    EXPECT(epx_dispatch(&p, &L, nullptr, 256, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch(&p, &L, A8, 256, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch(&p, &L, A, 256, EPX_BF16, A4, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch(&p, &L, A, 256, EPX_FP8_E4M3, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch(&p, &L, A, 256, EPX_FP8_E4M3, A, (float *)A2, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch(&p, nullptr, A, 256, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch_group(&pg, &L, -1, A, 256, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_dispatch_group(&pg, &L, 2, A, 256, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    {   // an empty batch moves nothing and launches nothing
        const epx_problem p0 = prob(0, 2, 16, 4, 2, 0, EPX_MODE_PER_EXPERT);
        EXPECT(epx_dispatch(&p0, &L, nullptr, 256, EPX_BF16, nullptr, nullptr, 0, nullptr), EPX_OK);
        EXPECT(epx_combine(&p0, &L, nullptr, 0, nullptr, 256, nullptr, nullptr), EPX_OK);
    }

    // layout + dispatch in one call, and its no-alloc variant
    EXPECT(epx_layout_dispatch(&p, nullptr, &L, A, 256, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_layout_dispatch(&p, (const int32_t *)A, nullptr, A, 256, EPX_BF16, A, nullptr, 128, nullptr),
           EPX_ERR_ARG);
    EXPECT(epx_layout_dispatch(&p, (const int32_t *)A, &L, A, 256, EPX_BF16, A, nullptr, 127, nullptr),
           EPX_ERR_CAPACITY);
    EXPECT(epx_layout_dispatch(&pr, (const int32_t *)A, &L, A, 256, EPX_BF16, A, nullptr, 128, nullptr),
           EPX_ERR_ARG);
    {
        const epx_problem big = prob(1 << 20, 8, 2048, 64, 2, 0, EPX_MODE_PER_EXPERT);
        EXPECT(epx_layout_dispatch_noalloc(&big, (const int32_t *)A, &L, A, 256, EPX_BF16, A, nullptr,
                                           (int64_t)1 << 23, nullptr), EPX_ERR_SCRATCH);
        EXPECT(epx_layout_dispatch_noalloc(&p, (const int32_t *)A, nullptr, A, 256, EPX_BF16, A, nullptr, 128,
                                           nullptr), EPX_ERR_ARG);
    }

    // combine and group combine
    EXPECT(epx_combine(&p, &L, A, 128, (const float *)A, 4, A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine(&p, &L, A, 127, (const float *)A, 256, A, nullptr), EPX_ERR_CAPACITY);
    EXPECT(epx_combine(&p, &L, nullptr, 128, (const float *)A, 256, A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine(&p, &L, A, 128, nullptr, 256, A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine(&p, &L, A, 128, (const float *)A2, 256, A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine(&p, &L, A, 128, (const float *)A, 256, A8, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine_group(&pg, &L, -1, A, 128, (const float *)A, 256, (float *)A, A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine_group(&pg, &L, 2, A, 128, (const float *)A, 256, (float *)A, A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine_group(&pg, &L, 0, A, 128, (const float *)A, 256, nullptr, A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine_group(&pg, &L, 0, A, 128, (const float *)A, 256, (float *)A8, A, nullptr), EPX_ERR_ARG);

    // relay receive side
    EXPECT(epx_relay_fanout(&p, &L, A, nullptr, 128, 256, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_relay_fanout(&pr, &LR, A, nullptr, 128, 256, EPX_F32, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_relay_fanout(&pr, &LR, A, nullptr, 127, 256, EPX_BF16, A, nullptr, 128, nullptr),
           EPX_ERR_CAPACITY);
    EXPECT(epx_relay_fanout(&pr, &LR, A, nullptr, 128, 256, EPX_BF16, A, nullptr, 127, nullptr),
           EPX_ERR_CAPACITY);
    EXPECT(epx_relay_fanout(&pr, &LR, A, nullptr, 128, 264, EPX_FP8_E4M3, A, (float *)A, 128, nullptr),
           EPX_ERR_ARG);
    EXPECT(epx_relay_fanout(&pr, &LR, A, nullptr, 128, 256, EPX_FP8_E4M3, A, (float *)A, 128, nullptr),
           EPX_ERR_ARG);
    EXPECT(epx_relay_fanout(&pr, &LR, A8, nullptr, 128, 256, EPX_BF16, A, nullptr, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine_relay_partials(&p, &L, A, 128, (const float *)A, 256, EPX_F32, A, 128, nullptr),
           EPX_ERR_ARG);
    EXPECT(epx_combine_relay_partials(&pr, &LR, A, 128, (const float *)A, 256, EPX_FP8_E4M3, A, 128, nullptr),
           EPX_ERR_ARG);
    EXPECT(epx_combine_relay_partials(&pr, &LR, A, 127, (const float *)A, 256, EPX_F32, A, 128, nullptr),
           EPX_ERR_CAPACITY);
    EXPECT(epx_combine_relay_partials(&pr, &LR, A, 128, (const float *)A, 256, EPX_F32, A, 127, nullptr),
           EPX_ERR_CAPACITY);
    EXPECT(epx_combine_relay_partials(&pr, &LR, A, 128, nullptr, 256, EPX_F32, A, 128, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine_relay_finish(&p, &L, A, 128, EPX_F32, 256, A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine_relay_finish(&pr, &LR, A, 128, EPX_BF16 + 7, 256, A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_combine_relay_finish(&pr, &LR, A, 127, EPX_F32, 256, A, nullptr), EPX_ERR_CAPACITY);
    EXPECT(epx_combine_relay_finish(&pr, &LR, A, 128, EPX_F32, 256, nullptr, nullptr), EPX_ERR_ARG);

    // swap planner
    int32_t *I = (int32_t *)A;
    EXPECT(epx_plan_swaps(0, 4, 2, I, I + 64, 0, I + 128, I, I, I, I, nullptr), EPX_ERR_ARG);
    EXPECT(epx_plan_swaps(16, 4, 2, I, I + 64, -1, I + 128, I, I, I, I, nullptr), EPX_ERR_ARG);
    EXPECT(epx_plan_swaps(16, 3, 1, I, I + 64, 0, I + 128, I, I, I, I, nullptr), EPX_ERR_ARG);
    EXPECT(epx_plan_swaps(16, 4, 2, nullptr, I + 64, 0, I + 128, I, I, I, I, nullptr), EPX_ERR_ARG);
    EXPECT(epx_plan_swaps(16, 4, 2, I, I + 64, 0, I + 64, I, I, I, I, nullptr), EPX_ERR_ARG);
    EXPECT(epx_plan_swaps(16, 4, 2, I, I + 64, 0, I + 128, I, I, nullptr, I, nullptr), EPX_ERR_ARG);
    EXPECT(epx_plan_swaps(4096, 4, 2, I, I + 64, 0, I + 128, I, I, I, I, nullptr), EPX_ERR_ARG);

    // diagnostics, the measurement hook, strings
    EXPECT(epx_read_error(nullptr, nullptr, nullptr), EPX_ERR_ARG);
    {
        epx_layout M = L;
        M.totals = nullptr;
        EXPECT(epx_read_error(&M, nullptr, nullptr), EPX_ERR_ARG);
    }
    EXPECT(epx_f32_to_e4m3((const float *)A, (uint8_t *)A, -1, nullptr), EPX_ERR_ARG);
    EXPECT(epx_f32_to_e4m3(nullptr, (uint8_t *)A, 4, nullptr), EPX_ERR_ARG);
    EXPECT(epx_f32_to_e4m3((const float *)A2, (uint8_t *)A, 4, nullptr), EPX_ERR_ARG);
    EXPECT(epx_f32_to_e4m3((const float *)A, (uint8_t *)A, 0, nullptr), EPX_OK);
    EXPECT(epx_time_next_call(A, nullptr), EPX_ERR_ARG);
    EXPECT(epx_time_next_call(nullptr, A), EPX_ERR_ARG);
    EXPECT(epx_time_next_call(nullptr, nullptr), EPX_OK);
    {
        int64_t n = 5;
        EXPECT(epx_checked_violations(&n, nullptr), EPX_ERR_ARG);   // release build
        EXPECT(n, -1);
        EXPECT(epx_checked_violations(nullptr, nullptr), EPX_ERR_ARG);
    }
    EXPECT(epx_abi_version(), EPX_ABI_VERSION);
    for (int code = 0; code <= 6; ++code)
        EXPECT(std::strlen(epx_status_string((epx_status)code)) > 0, 1);

    std::printf("host checks ok: %d\n", checks);
    return 0;
}
'''


def _objects():
    """The library's device objects other than the API's own (built in-tree)."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs
            if os.path.basename(s) != "epx_api.hip"]
    if not all(os.path.exists(o) and os.path.getmtime(o) >= os.path.getmtime(s)
               for o, s in zip(objs, [s for s in srcs if os.path.basename(s) != "epx_api.hip"])):
        from combine_epx_get_amd import build
        build.build()
    return objs


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_every_host_check_under_asan_and_ubsan():
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    tmp = tempfile.mkdtemp(prefix="epx_host_san_")
    try:
        drv = os.path.join(tmp, "driver.cpp")
        open(drv, "w").write(DRIVER)
        api_o = os.path.join(tmp, "epx_api.o")
        exe = os.path.join(tmp, "driver")
        drv_o = os.path.join(tmp, "driver.o")
        for cmd in ([HIPCC, *common, *san, "-c", os.path.join(CSRC, "epx_api.hip"), "-o", api_o],
                    [HIPCC, *common, *san, "-c", drv, "-o", drv_o],
                    [HIPCC, "--offload-arch=gfx950", *san, "-o", exe, drv_o, api_o, *_objects()]):
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0 and "host checks ok" in r.stdout, (r.stdout[-2000:], r.stderr[-3000:])
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
