// epx_internal.h -- definitions shared by the HIP translation units of libepx.
// Not installed; the public interface is include/epx.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epx.h"

namespace epx {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kChunkPairs = 1024;    // pairs staged per layout workgroup (at most 64 tokens)
constexpr int kMaxExperts = 2048;
constexpr int kMaxTopk = 64;
constexpr int kMaxHosts = 64;
constexpr int kMaxRanksPerHost = 32;
constexpr int kFp8Block = 128;       // channels per fp8 scale

// Bounds-checked builds (libepx_checked.so, compiled with EPX_CHECKED):
// every row index that a kernel computes, or reads from a layout, is checked
// against the buffer it addresses before the access; an index out of bounds
// skips the access and is counted in a device counter that
// epx_checked_violations reads. In the release build the checks compile
// away (in_bounds is constant true).
#ifdef EPX_CHECKED
constexpr bool kChecked = true;
#else
constexpr bool kChecked = false;
#endif

__device__ __forceinline__ bool in_bounds(int64_t i, int64_t n, unsigned long long *viol)
{
    if (!kChecked || (uint64_t)i < (uint64_t)n)
        return true;
    atomicAdd(viol, 1ull);
    return false;
}

// Division by a divisor fixed per call, as a multiply-high: q = umulhi(n, m)
// with m = ceil(2^32 / d) is exact whenever n * d < 2^32 (the error n*(m -
// 2^32/d)/2^32 stays below 1/d). Every use here has n, d <= 4096.
struct FastDiv {
    uint32_t mul;   // ceil(2^32 / d); unused when d == 1
    int32_t d;
    void init(int32_t divisor)
    {
        d = divisor;
        mul = divisor == 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + divisor - 1) / divisor);
    }
    __device__ __forceinline__ int32_t div(int32_t n) const
    {
        return d == 1 ? n : (int32_t)__umulhi((uint32_t)n, mul);
    }
};

// Problem geometry, validated on the host and passed by value to kernels.
struct Geometry {
    int32_t T, k, E, R, H, s;
    int32_t epr;     // experts per rank
    int32_t rph;     // ranks per host
    int32_t ct;      // tokens per layout workgroup: 32 (k <= 16), else kChunkPairs / k
    int32_t G;       // layout workgroups = max(1, ceil(T / ct))
    int32_t Gs;      // workspace column stride: G rounded up to 4 (16-byte columns)
    int32_t nbits;   // bits that distinguish expert ids (ceil(log2 E))
    int32_t relay;   // HOST_RELAY mode
    int32_t m;       // expert groups (1: none)
    int32_t epg;     // experts per rank in one group: epr / m
    FastDiv div_epr, div_rph, div_k;
    unsigned long long *viol;   // violation counter (checked builds; else null)
    int64_t cap;     // rows of the call's destination buffer (recv) for layout kernels
                     // that also dispatch (checked builds)
};

// Rows of per-expert and relay layout arrays: T*k and T*min(k, H).
__host__ __device__ inline int64_t pair_rows(const Geometry &g) { return (int64_t)g.T * g.k; }
__host__ __device__ inline int64_t relay_rows_cap(const Geometry &g)
{
    return (int64_t)g.T * (g.k < g.H ? g.k : g.H);
}

// One workgroup per item (token or row) for any item count: item i runs as
// blockIdx.x = i mod kGridX, blockIdx.z = i / kGridX (blockIdx.y stays free
// for column slices), so that no grid dimension reaches 2^32 work-items.
// Kernels return at once for i >= the item count (the last z-slab's tail).
constexpr int kGridX = 65536;

inline dim3 item_grid(int64_t items, int slices)
{
    return dim3((unsigned)(items < kGridX ? items : kGridX), (unsigned)slices,
                (unsigned)((items + kGridX - 1) / kGridX));
}

__device__ __forceinline__ int64_t item_index()
{
    return (int64_t)blockIdx.z * kGridX + blockIdx.x;
}

// 16-byte and 8-byte native vectors (global_load/store_dwordx4, dwordx2).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Measurement hook (epx_time_next_call): HIP events that the next library
// call made from this host thread binds to its kernels' dispatch packets --
// `start` to the first kernel it launches, `stop` to every kernel, so that
// it ends up marking the last one's end. Every entry point clears the hook
// when it returns.
struct TimingHook {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
TimingHook &timing_hook();

// Every kernel launch of the library. With no hook armed it is the plain
// launch; with one, the launch carries the hook's events
// (hipExtLaunchKernel), which time the kernel alone, as a profiler does.
// The caller reads the launch status with hipGetLastError().
template <typename... KArgs, typename... Args>
inline void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                   hipStream_t stream, Args... args)
{
    TimingHook &h = timing_hook();
    if (h.stop == nullptr) {
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
        return;
    }
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, h.start, h.stop, 0u,
                          args...);
    h.start = nullptr;
}

// Launchers (each returns the launch status).
hipError_t launch_layout(const Geometry &g, const int32_t *idx, const epx_layout &L,
                         hipStream_t stream);
// group < 0: every destination; else only group `group`'s rows.
// cap: rows of recv (and of the scales).
hipError_t launch_dispatch_bf16(const Geometry &g, const epx_layout &L, const void *x,
                                int32_t hidden, void *recv, int64_t cap, int group,
                                hipStream_t stream);
hipError_t launch_dispatch_fp8(const Geometry &g, const epx_layout &L, const void *x,
                               int32_t hidden, void *recv, float *scales, int64_t cap, int group,
                               hipStream_t stream);
// Layout and dispatch in one launch; false (nothing launched) when the batch
// is too large for it. *err receives the launch status otherwise.
bool launch_layout_dispatch(const Geometry &g, const int32_t *idx, const epx_layout &L,
                            const void *x, int32_t hidden, bool fp8, void *recv, float *scales,
                            hipStream_t stream, hipError_t *err);
// Layout and dispatch above the single-launch sizes (k <= 16, one expert
// group; bf16, or fp8 in relay mode): count, scan, then one launch that
// assigns the rows and copies the tokens. False (nothing launched) when it does not apply; *err receives the
// status otherwise.
bool launch_layout_assign_dispatch(const Geometry &g, const int32_t *idx, const epx_layout &L,
                                   const void *x, int32_t hidden, bool fp8, void *recv,
                                   float *scales, hipStream_t stream, hipError_t *err);
// y_rows: rows of y.
hipError_t launch_combine(const Geometry &g, const epx_layout &L, const void *y, int64_t y_rows,
                          const float *w, int32_t hidden, void *out, hipStream_t stream);
hipError_t launch_combine_group(const Geometry &g, const epx_layout &L, int group,
                                const void *y, int64_t y_rows, const float *w, int32_t hidden,
                                float *carry, void *out, hipStream_t stream);
hipError_t launch_f32_to_e4m3(const float *in, uint8_t *out, int64_t n, hipStream_t stream);
// relay_cap, cap, y_rows, part_cap: rows of relay_rows, recv, y and partials.
hipError_t launch_relay_fanout(const Geometry &g, const epx_layout &L, const void *relay_rows,
                               const float *relay_scales, int64_t relay_cap, int64_t row_bytes,
                               int nsc, void *recv, float *recv_scales, int64_t cap,
                               hipStream_t stream);
hipError_t launch_relay_partials(const Geometry &g, const epx_layout &L, const void *y,
                                 int64_t y_rows, const float *w, int32_t hidden, bool bf16_out,
                                 void *partials, int64_t part_cap, hipStream_t stream);
hipError_t launch_relay_finish(const Geometry &g, const epx_layout &L, const void *partials,
                               int64_t part_cap, bool bf16_in, int32_t hidden, void *out,
                               hipStream_t stream);
hipError_t launch_plan_swaps(int E, int R, int H, const int32_t *count, const int32_t *slot_in,
                             int tau, int32_t *slot_out, int32_t *load_before,
                             int32_t *load_after, int32_t *swaps, int32_t *host_bad,
                             hipStream_t stream);

}  // namespace epx
