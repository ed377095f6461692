// epx_api.hip -- the C ABI of libepx: argument checks, sizes and launches.
// Every check here runs on the host before anything is launched; a call that
// fails a check launches nothing.
#include <stdint.h>

#include <mutex>

#include "epx_internal.h"

// Scratch of epx_layout_dispatch_noalloc: the layout workspace for callers
// that cannot allocate. One copy per GPU (each device holds its own at its
// own address), kept until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: host code only ever uses the
// device address that hipGetSymbolAddress returns for it.
static __device__ __align__(256) int32_t scratch[EPX_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

// Bounds-checked builds: accesses that a check skipped, on this device.
static __device__ unsigned long long violations;

namespace epx {
TimingHook &timing_hook()
{
    static thread_local TimingHook hook;
    return hook;
}
}  // namespace epx

namespace {

using epx::Geometry;

// Clears the measurement hook when an entry point returns, whatever it did:
// the hook applies to one call.
struct HookScope {
    ~HookScope() { epx::timing_hook() = epx::TimingHook{}; }
};

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Validates the problem and fills the kernel geometry.
epx_status make_geometry(const epx_problem *p, Geometry *g)
{
    if (!p)
        return EPX_ERR_ARG;
    const int32_t T = p->num_tokens, k = p->topk, E = p->num_experts, R = p->num_ranks,
                  H = p->num_hosts, s = p->my_rank;
    if (T < 0 || T > (1 << 24) || k < 1 || k > epx::kMaxTopk || E < 1 || E > epx::kMaxExperts)
        return EPX_ERR_ARG;
    if (R < 1 || H < 1 || H > epx::kMaxHosts || E % R != 0 || R % H != 0 || k > E)
        return EPX_ERR_ARG;
    if (R / H > epx::kMaxRanksPerHost || s < 0 || s >= R)
        return EPX_ERR_ARG;
    if (p->mode != EPX_MODE_PER_EXPERT && p->mode != EPX_MODE_HOST_RELAY)
        return EPX_ERR_ARG;
    if ((int64_t)T * k >= ((int64_t)1 << 31))
        return EPX_ERR_ARG;
    const int32_t m = p->num_groups == 0 ? 1 : p->num_groups;
    if (m < 1 || (E / R) % m != 0 || (m > 1 && p->mode != EPX_MODE_PER_EXPERT))
        return EPX_ERR_ARG;
    g->T = T;
    g->k = k;
    g->E = E;
    g->R = R;
    g->H = H;
    g->s = s;
    g->epr = E / R;
    g->rph = R / H;
    g->ct = k <= 16 ? 32 : epx::kChunkPairs / k;
    g->G = T > 0 ? (T + g->ct - 1) / g->ct : 1;
    g->Gs = (g->G + 3) & ~3;
    g->div_epr.init(g->epr);
    g->div_rph.init(g->rph);
    g->div_k.init(k);
    int nbits = 0;
    while ((1 << nbits) < E)
        ++nbits;
    g->nbits = nbits;
    g->relay = p->mode == EPX_MODE_HOST_RELAY;
    g->m = m;
    g->epg = g->epr / m;
    g->viol = nullptr;
    g->cap = 0;
    return EPX_OK;
}

int64_t relay_capacity(const Geometry &g) { return (int64_t)g.T * (g.k < g.H ? g.k : g.H); }

void sizes_of(const Geometry &g, int64_t s[EPX_LAYOUT_NARRAYS])
{
    const int64_t cap = relay_capacity(g);
    s[EPX_L_EXPERT_COUNT] = g.E;
    s[EPX_L_EXPERT_OFFSET] = g.E + 1;
    s[EPX_L_RANK_ROWS] = g.R;
    s[EPX_L_RANK_TOKENS] = g.R;
    s[EPX_L_RANK_OFFSET] = g.R + 1;
    s[EPX_L_HOST_TOKENS] = g.H;
    s[EPX_L_HOST_OFFSET] = g.H + 1;
    s[EPX_L_SLOT] = (int64_t)g.T * g.k;
    s[EPX_L_ROW_TOKEN] = (int64_t)g.T * g.k;
    s[EPX_L_RELAY_SLOT] = (int64_t)g.T * g.H;
    s[EPX_L_RELAY_TOKEN] = cap;
    s[EPX_L_FANOUT_EXPERT] = cap * g.k;
    s[EPX_L_FANOUT_RANK_MASK] = cap;
    s[EPX_L_RELAY_DST_RANK] = g.H;
    s[EPX_L_TOTALS] = 4;
    s[EPX_L_GROUP_OFFSET] = (int64_t)g.m * g.R + 1;
    s[EPX_L_WORKSPACE] = (int64_t)(g.Gs + 1) * (g.E + g.R + g.H + 1);
}

// Every array the layout kernels write must be present (relay arrays only in
// relay mode) and 4-byte aligned.
epx_status check_layout(const Geometry &g, const epx_layout *L)
{
    if (!L)
        return EPX_ERR_ARG;
    const void *need[] = {L->expert_count, L->expert_offset, L->rank_rows, L->rank_tokens,
                          L->rank_offset, L->host_tokens, L->host_offset, L->slot,
                          L->row_token, L->relay_dst_rank, L->totals, L->group_offset};
    for (const void *q : need)
        if (!q || !aligned(q, 4))
            return EPX_ERR_ARG;
    if (!L->workspace || !aligned(L->workspace, 16))
        return EPX_ERR_ARG;
    if (g.relay) {
        const void *rel[] = {L->relay_slot, L->relay_token, L->fanout_expert, L->fanout_rank_mask};
        for (const void *q : rel)
            if (!q || !aligned(q, 4))
                return EPX_ERR_ARG;
    }
    return EPX_OK;
}

epx_status from_hip(hipError_t e) { return e == hipSuccess ? EPX_OK : EPX_ERR_DEVICE; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
int32_t *g_scratch_ptr[kMaxDevices];

// Device address of `violations` on the current device (checked builds),
// looked up once per device and kept.
unsigned long long *g_violations_ptr[kMaxDevices];

epx_status violations_on_current_device(unsigned long long **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return EPX_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_violations_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(violations)) != hipSuccess || ptr == nullptr)
            return EPX_ERR_DEVICE;
        g_violations_ptr[dev] = (unsigned long long *)ptr;
    }
    *out = g_violations_ptr[dev];
    return EPX_OK;
}

// After a call's host checks, before its launches: checked builds point the
// kernels at the violation counter; release builds do nothing.
epx_status arm_checks(Geometry &g)
{
    if (!epx::kChecked)
        return EPX_OK;
    return violations_on_current_device(&g.viol);
}

epx_status scratch_on_current_device(int32_t **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return EPX_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return EPX_ERR_DEVICE;
        g_scratch_ptr[dev] = (int32_t *)ptr;
    }
    *out = g_scratch_ptr[dev];
    return EPX_OK;
}

// The dispatch arguments (T > 0 for the pointers).
epx_status check_dispatch(const Geometry &g, const void *x, int32_t hidden, int32_t out_dtype,
                          const void *recv, const float *recv_scales, int64_t capacity_rows)
{
    if (out_dtype != EPX_BF16 && out_dtype != EPX_FP8_E4M3)
        return EPX_ERR_ARG;
    if (hidden < 8 || hidden % 8 != 0 || (out_dtype == EPX_FP8_E4M3 && hidden % epx::kFp8Block != 0))
        return EPX_ERR_ARG;
    const int64_t need = g.relay ? relay_capacity(g) : (int64_t)g.T * g.k;
    if (capacity_rows < need)
        return EPX_ERR_CAPACITY;
    if (g.T == 0)
        return EPX_OK;   // nothing to move; the activation pointers are not used
    if (!x || !recv || !aligned(x, 16) || !aligned(recv, 16))
        return EPX_ERR_ARG;
    if (out_dtype == EPX_FP8_E4M3 && (!recv_scales || !aligned(recv_scales, 4)))
        return EPX_ERR_ARG;
    return EPX_OK;
}

// group < 0: the plain call; else one group's rows (group < m).
epx_status dispatch_impl(const epx_problem *p, const epx_layout *layout, int group, const void *x,
                         int32_t hidden, int32_t out_dtype, void *recv, float *recv_scales,
                         int64_t capacity_rows, void *stream)
{
    Geometry g;
    epx_status st = make_geometry(p, &g);
    if (st != EPX_OK)
        return st;
    if ((st = check_layout(g, layout)) != EPX_OK)
        return st;
    if (group >= g.m)
        return EPX_ERR_ARG;
    if (g.m == 1)
        group = -1;   // one group is every row (relay rows included)
    if ((st = check_dispatch(g, x, hidden, out_dtype, recv, recv_scales, capacity_rows)) != EPX_OK)
        return st;
    if (g.T == 0)
        return EPX_OK;
    if ((st = arm_checks(g)) != EPX_OK)
        return st;
    const hipStream_t s = (hipStream_t)stream;
    if (out_dtype == EPX_BF16)
        return from_hip(
            epx::launch_dispatch_bf16(g, *layout, x, hidden, recv, capacity_rows, group, s));
    return from_hip(epx::launch_dispatch_fp8(g, *layout, x, hidden, recv, recv_scales,
                                             capacity_rows, group, s));
}

// epx_layout_dispatch after the problem and layout checks; `L` carries the
// workspace to use.
epx_status layout_dispatch_checked(Geometry g, const int32_t *topk_idx, const epx_layout &L,
                                   const void *x, int32_t hidden, int32_t out_dtype, void *recv,
                                   float *recv_scales, int64_t capacity_rows, void *stream)
{
    if (g.T > 0 && (!topk_idx || !aligned(topk_idx, 4)))
        return EPX_ERR_ARG;
    epx_status st = check_dispatch(g, x, hidden, out_dtype, recv, recv_scales, capacity_rows);
    if (st != EPX_OK)
        return st;
    if ((st = arm_checks(g)) != EPX_OK)
        return st;
    g.cap = capacity_rows;
    const hipStream_t s = (hipStream_t)stream;
    const bool fp8 = out_dtype == EPX_FP8_E4M3;
    hipError_t err = hipSuccess;
    if (g.T > 0 && epx::launch_layout_dispatch(g, topk_idx, L, x, hidden, fp8, recv, recv_scales, s, &err))
        return from_hip(err);
    if (epx::launch_layout_assign_dispatch(g, topk_idx, L, x, hidden, fp8, recv, recv_scales, s, &err))
        return from_hip(err);
    if ((st = from_hip(epx::launch_layout(g, topk_idx, L, s))) != EPX_OK || g.T == 0)
        return st;
    if (!fp8)
        return from_hip(epx::launch_dispatch_bf16(g, L, x, hidden, recv, capacity_rows, -1, s));
    return from_hip(
        epx::launch_dispatch_fp8(g, L, x, hidden, recv, recv_scales, capacity_rows, -1, s));
}

epx_status combine_impl(const epx_problem *p, const epx_layout *layout, int group, const void *y,
                        int64_t y_rows, const float *topk_weights, int32_t hidden, float *carry,
                        void *out, void *stream)
{
    Geometry g;
    epx_status st = make_geometry(p, &g);
    if (st != EPX_OK)
        return st;
    if ((st = check_layout(g, layout)) != EPX_OK)
        return st;
    if (group >= g.m)
        return EPX_ERR_ARG;
    if (hidden < 8 || hidden % 8 != 0)
        return EPX_ERR_ARG;
    if (y_rows < (int64_t)g.T * g.k)
        return EPX_ERR_CAPACITY;
    if (g.T == 0)
        return EPX_OK;
    if (!y || !out || !topk_weights || !aligned(y, 16) || !aligned(out, 16) ||
        !aligned(topk_weights, 4))
        return EPX_ERR_ARG;
    const hipStream_t s = (hipStream_t)stream;
    if (!(group < 0 || g.m == 1) && (!carry || !aligned(carry, 16)))
        return EPX_ERR_ARG;
    if ((st = arm_checks(g)) != EPX_OK)
        return st;
    if (group < 0 || g.m == 1)
        return from_hip(epx::launch_combine(g, *layout, y, y_rows, topk_weights, hidden, out, s));
    return from_hip(epx::launch_combine_group(g, *layout, group, y, y_rows, topk_weights, hidden,
                                              carry, out, s));
}

}  // namespace

extern "C" {

int32_t epx_abi_version(void) { return EPX_ABI_VERSION; }

epx_status epx_time_next_call(void *start_event, void *stop_event)
{
    if ((start_event == nullptr) != (stop_event == nullptr))
        return EPX_ERR_ARG;
    epx::timing_hook() = epx::TimingHook{(hipEvent_t)start_event, (hipEvent_t)stop_event};
    return EPX_OK;
}

const char *epx_status_string(epx_status s)
{
    switch (s) {
    case EPX_OK:
        return "ok";
    case EPX_ERR_ARG:
        return "invalid argument (pointer, alignment, geometry or size)";
    case EPX_ERR_INDEX:
        return "expert id out of range in topk_idx";
    case EPX_ERR_CAPACITY:
        return "output buffer smaller than required";
    case EPX_ERR_DEVICE:
        return "HIP launch or runtime failure";
    case EPX_ERR_SCRATCH:
        return "problem too large for the library's static scratch (epx_layout_dispatch_noalloc)";
    }
    return "unknown status";
}

epx_status epx_layout_sizes(const epx_problem *p, int64_t sizes_out[EPX_LAYOUT_NARRAYS])
{
    HookScope hook_scope;
    Geometry g;
    epx_status st = make_geometry(p, &g);
    if (st != EPX_OK)
        return st;
    if (!sizes_out)
        return EPX_ERR_ARG;
    sizes_of(g, sizes_out);
    return EPX_OK;
}

epx_status epx_get_layout(const epx_problem *p, const int32_t *topk_idx, const epx_layout *layout,
                          void *stream)
{
    HookScope hook_scope;
    Geometry g;
    epx_status st = make_geometry(p, &g);
    if (st != EPX_OK)
        return st;
    if ((st = check_layout(g, layout)) != EPX_OK)
        return st;
    if (g.T > 0 && (!topk_idx || !aligned(topk_idx, 4)))
        return EPX_ERR_ARG;
    if ((st = arm_checks(g)) != EPX_OK)
        return st;
    return from_hip(epx::launch_layout(g, topk_idx, *layout, (hipStream_t)stream));
}

epx_status epx_dispatch(const epx_problem *p, const epx_layout *layout, const void *x,
                        int32_t hidden, int32_t out_dtype, void *recv, float *recv_scales,
                        int64_t capacity_rows, void *stream)
{
    HookScope hook_scope;
    return dispatch_impl(p, layout, -1, x, hidden, out_dtype, recv, recv_scales, capacity_rows,
                         stream);
}

epx_status epx_layout_dispatch(const epx_problem *p, const int32_t *topk_idx,
                               const epx_layout *layout, const void *x, int32_t hidden,
                               int32_t out_dtype, void *recv, float *recv_scales,
                               int64_t capacity_rows, void *stream)
{
    HookScope hook_scope;
    Geometry g;
    epx_status st = make_geometry(p, &g);
    if (st != EPX_OK)
        return st;
    if ((st = check_layout(g, layout)) != EPX_OK)
        return st;
    return layout_dispatch_checked(g, topk_idx, *layout, x, hidden, out_dtype, recv, recv_scales,
                                   capacity_rows, stream);
}

epx_status epx_layout_dispatch_noalloc(const epx_problem *p, const int32_t *topk_idx,
                                       const epx_layout *layout, const void *x, int32_t hidden,
                                       int32_t out_dtype, void *recv, float *recv_scales,
                                       int64_t capacity_rows, void *stream)
{
    HookScope hook_scope;
    Geometry g;
    epx_status st = make_geometry(p, &g);
    if (st != EPX_OK)
        return st;
    if (!layout)
        return EPX_ERR_ARG;
    int64_t sizes[EPX_LAYOUT_NARRAYS];
    sizes_of(g, sizes);
    if (sizes[EPX_L_WORKSPACE] * (int64_t)sizeof(int32_t) > (int64_t)EPX_NOALLOC_SCRATCH_BYTES)
        return EPX_ERR_SCRATCH;   // checked before any HIP call
    epx_layout L = *layout;
    L.workspace = nullptr;
    if ((st = scratch_on_current_device(&L.workspace)) != EPX_OK)
        return st;
    if ((st = check_layout(g, &L)) != EPX_OK)
        return st;
    return layout_dispatch_checked(g, topk_idx, L, x, hidden, out_dtype, recv, recv_scales,
                                   capacity_rows, stream);
}


epx_status epx_dispatch_group(const epx_problem *p, const epx_layout *layout, int32_t group,
                              const void *x, int32_t hidden, int32_t out_dtype, void *recv,
                              float *recv_scales, int64_t capacity_rows, void *stream)
{
    HookScope hook_scope;
    if (group < 0)
        return EPX_ERR_ARG;
    return dispatch_impl(p, layout, group, x, hidden, out_dtype, recv, recv_scales, capacity_rows,
                         stream);
}

epx_status epx_combine(const epx_problem *p, const epx_layout *layout, const void *y,
                       int64_t y_rows, const float *topk_weights, int32_t hidden, void *out,
                       void *stream)
{
    HookScope hook_scope;
    return combine_impl(p, layout, -1, y, y_rows, topk_weights, hidden, nullptr, out, stream);
}

epx_status epx_combine_group(const epx_problem *p, const epx_layout *layout, int32_t group,
                             const void *y, int64_t y_rows, const float *topk_weights,
                             int32_t hidden, float *carry, void *out, void *stream)
{
    HookScope hook_scope;
    if (group < 0)
        return EPX_ERR_ARG;
    return combine_impl(p, layout, group, y, y_rows, topk_weights, hidden, carry, out, stream);
}

epx_status epx_relay_fanout(const epx_problem *p, const epx_layout *layout,
                            const void *relay_rows, const float *relay_scales,
                            int64_t relay_capacity_rows, int32_t hidden, int32_t dtype,
                            void *recv, float *recv_scales, int64_t capacity_rows, void *stream)
{
    HookScope hook_scope;
    Geometry g;
    epx_status st = make_geometry(p, &g);
    if (st != EPX_OK)
        return st;
    if (!g.relay)
        return EPX_ERR_ARG;
    if ((st = check_layout(g, layout)) != EPX_OK)
        return st;
    if (dtype != EPX_BF16 && dtype != EPX_FP8_E4M3)
        return EPX_ERR_ARG;
    if (hidden < 8 || hidden % 8 != 0 || (dtype == EPX_FP8_E4M3 && hidden % epx::kFp8Block != 0))
        return EPX_ERR_ARG;
    if (relay_capacity_rows < relay_capacity(g) || capacity_rows < (int64_t)g.T * g.k)
        return EPX_ERR_CAPACITY;
    if (g.T == 0)
        return EPX_OK;
    if (!relay_rows || !recv || !aligned(relay_rows, 16) || !aligned(recv, 16))
        return EPX_ERR_ARG;
    const bool fp8 = dtype == EPX_FP8_E4M3;
    if (fp8 && (!relay_scales || !recv_scales || !aligned(relay_scales, 4) || !aligned(recv_scales, 4)))
        return EPX_ERR_ARG;
    const int64_t row_bytes = fp8 ? hidden : (int64_t)hidden * 2;
    if ((st = arm_checks(g)) != EPX_OK)
        return st;
    return from_hip(epx::launch_relay_fanout(g, *layout, relay_rows, relay_scales,
                                             relay_capacity_rows, row_bytes,
                                             fp8 ? hidden / epx::kFp8Block : 0, recv, recv_scales,
                                             capacity_rows, (hipStream_t)stream));
}

epx_status epx_combine_relay_partials(const epx_problem *p, const epx_layout *layout,
                                      const void *y, int64_t y_rows, const float *topk_weights,
                                      int32_t hidden, int32_t partial_dtype, void *partials,
                                      int64_t partial_capacity_rows, void *stream)
{
    HookScope hook_scope;
    Geometry g;
    epx_status st = make_geometry(p, &g);
    if (st != EPX_OK)
        return st;
    if (!g.relay)
        return EPX_ERR_ARG;
    if ((st = check_layout(g, layout)) != EPX_OK)
        return st;
    if ((partial_dtype != EPX_F32 && partial_dtype != EPX_BF16) || hidden < 8 || hidden % 8 != 0)
        return EPX_ERR_ARG;
    if (y_rows < (int64_t)g.T * g.k || partial_capacity_rows < relay_capacity(g))
        return EPX_ERR_CAPACITY;
    if (g.T == 0)
        return EPX_OK;
    if (!y || !topk_weights || !partials || !aligned(y, 16) || !aligned(topk_weights, 4) ||
        !aligned(partials, 16))
        return EPX_ERR_ARG;
    if ((st = arm_checks(g)) != EPX_OK)
        return st;
    return from_hip(epx::launch_relay_partials(g, *layout, y, y_rows, topk_weights, hidden,
                                               partial_dtype == EPX_BF16, partials,
                                               partial_capacity_rows, (hipStream_t)stream));
}

epx_status epx_combine_relay_finish(const epx_problem *p, const epx_layout *layout,
                                    const void *partials, int64_t partial_capacity_rows,
                                    int32_t partial_dtype, int32_t hidden, void *out, void *stream)
{
    HookScope hook_scope;
    Geometry g;
    epx_status st = make_geometry(p, &g);
    if (st != EPX_OK)
        return st;
    if (!g.relay)
        return EPX_ERR_ARG;
    if ((st = check_layout(g, layout)) != EPX_OK)
        return st;
    if ((partial_dtype != EPX_F32 && partial_dtype != EPX_BF16) || hidden < 8 || hidden % 8 != 0)
        return EPX_ERR_ARG;
    if (partial_capacity_rows < relay_capacity(g))
        return EPX_ERR_CAPACITY;
    if (g.T == 0)
        return EPX_OK;
    if (!partials || !out || !aligned(partials, 16) || !aligned(out, 16))
        return EPX_ERR_ARG;
    if ((st = arm_checks(g)) != EPX_OK)
        return st;
    return from_hip(epx::launch_relay_finish(g, *layout, partials, partial_capacity_rows,
                                             partial_dtype == EPX_BF16, hidden, out,
                                             (hipStream_t)stream));
}

epx_status epx_read_error(const epx_layout *layout, int32_t *bad_count, void *stream)
{
    HookScope hook_scope;
    if (!layout || !layout->totals)
        return EPX_ERR_ARG;
    int32_t totals[4];
    const hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(totals, layout->totals, sizeof totals, hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return EPX_ERR_DEVICE;
    if (bad_count)
        *bad_count = totals[3];
    return totals[3] == 0 ? EPX_OK : EPX_ERR_INDEX;
}

epx_status epx_plan_swaps(int32_t num_experts, int32_t num_ranks, int32_t num_hosts,
                          const int32_t *expert_count, const int32_t *slot_expert_in,
                          int32_t tau, int32_t *slot_expert_out, int32_t *rank_load_before,
                          int32_t *rank_load_after, int32_t *swaps, int32_t *host_bad,
                          void *stream)
{
    HookScope hook_scope;
    const int32_t E = num_experts, R = num_ranks, H = num_hosts;
    if (E < 1 || E > epx::kMaxExperts || R < 1 || H < 1 || H > epx::kMaxHosts || E % R != 0 ||
        R % H != 0 || R / H > epx::kMaxRanksPerHost || tau < 0)
        return EPX_ERR_ARG;
    const void *need[] = {expert_count, slot_expert_in, slot_expert_out, rank_load_before,
                          rank_load_after, host_bad};
    for (const void *q : need)
        if (!q || !aligned(q, 4))
            return EPX_ERR_ARG;
    if (R / H >= 2 && (!swaps || !aligned(swaps, 4)))
        return EPX_ERR_ARG;
    if (slot_expert_out == slot_expert_in)
        return EPX_ERR_ARG;
    return from_hip(epx::launch_plan_swaps(E, R, H, expert_count, slot_expert_in, tau,
                                           slot_expert_out, rank_load_before, rank_load_after,
                                           swaps, host_bad, (hipStream_t)stream));
}

epx_status epx_checked_violations(int64_t *count, void *stream)
{
    HookScope hook_scope;
    if (!count)
        return EPX_ERR_ARG;
    *count = -1;
    if (!epx::kChecked)
        return EPX_ERR_ARG;   // a release build checks nothing
    unsigned long long *ptr = nullptr;
    epx_status st = violations_on_current_device(&ptr);
    if (st != EPX_OK)
        return st;
    const hipStream_t s = (hipStream_t)stream;
    unsigned long long v = 0;
    const unsigned long long zero = 0;
    if (hipStreamSynchronize(s) != hipSuccess ||
        hipMemcpy(&v, ptr, sizeof v, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(ptr, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
        return EPX_ERR_DEVICE;
    *count = (int64_t)v;
    return EPX_OK;
}

epx_status epx_f32_to_e4m3(const float *in, uint8_t *out, int64_t n, void *stream)
{
    HookScope hook_scope;
    if (n < 0 || (n > 0 && (!in || !out || !aligned(in, 4))))
        return EPX_ERR_ARG;
    if (n == 0)
        return EPX_OK;
    return from_hip(epx::launch_f32_to_e4m3(in, out, n, (hipStream_t)stream));
}

}  // extern "C"
