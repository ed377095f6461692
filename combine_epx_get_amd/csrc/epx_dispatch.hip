// epx_dispatch.hip -- token rows -> destination rows on gfx950.
//
// Per-expert mode writes one copy of a token's row per destination expert
// (DeepEP's default, Mode 1 of the digest "Balancing and Beyond:
// Communication-Centric Optimizations in Expert Parallelism", section 3.2);
// relay mode writes one copy per destination host (Mode 2 with
// de-redundancy). Both read x once per token and store it to each of the
// token's destination rows, so the kernel moves T*h*2 bytes in and
// (rows)*h*2 bytes out: an HBM-bound scatter.
//
// The fp8 variant is the BF16-to-FP8 conversion that dispatch performs
// (digest section 3.1): per token and 128-channel block, scale = amax/448 and
// code = E4M3(x / scale), quantised once per token and stored to every row.
// One 16-lane group holds a 128-channel block (8 bf16 per lane, one 16-byte
// load), reduces the block maximum with lane shuffles and writes 8 code bytes
// per lane (128 contiguous bytes per group).
#include "epx_internal.h"

namespace epx {
namespace {

constexpr int kThreads = 256;

// Destination rows of token t: the layout's slots or relay slots.
__device__ __forceinline__ void load_destinations(const int32_t *__restrict__ dest, int D,
                                                  int64_t t, int32_t *s_dst)
{
    if (threadIdx.x < D)
        s_dst[threadIdx.x] = dest[t * D + threadIdx.x];
    __syncthreads();
}

__global__ __launch_bounds__(kThreads) void dispatch_bf16_kernel(
    const u32x4 *__restrict__ x, int nvec, const int32_t *__restrict__ dest, int D,
    u32x4 *__restrict__ recv, const int32_t *__restrict__ totals)
{
    __shared__ int32_t s_dst[kMaxTopk];
    if (totals[3] != 0)
        return;   // the layout saw out-of-range expert ids
    const int64_t t = blockIdx.x;
    load_destinations(dest, D, t, s_dst);
    const u32x4 *xr = x + t * nvec;
    for (int c = threadIdx.x; c < nvec; c += kThreads) {
        const u32x4 v = __builtin_nontemporal_load(xr + c);
        for (int d = 0; d < D; ++d) {
            const int64_t r = s_dst[d];
            if (r >= 0)
                __builtin_nontemporal_store(v, recv + r * nvec + c);
        }
    }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> OCP E4M3FN, round to nearest even, finite values beyond +-448
// saturate to +-448, NaN -> NaN. Normal range: round the 23-bit mantissa to 3
// bits on the integer pattern and rebias the exponent (127 -> 7); below 2^-6
// the codes are the integers rint(|v| * 2^9) (2^-9 steps; 8 is 2^-6 itself).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return sign | 0x7Fu;
    if (a >= 0x43E00000u)           // >= 448.0f
        return sign | 0x7Eu;
    if (a < 0x3C800000u)            // < 2^-6
        return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((r >> 20) - (120u << 3));
}

__device__ __forceinline__ uint32_t quantize4(float a, float b, float c, float d, float s, bool zero)
{
    if (zero) {   // all-zero block: scale 0, codes keep the sign of each zero
        return ((__float_as_uint(a) >> 24) & 0x80u) | (((__float_as_uint(b) >> 24) & 0x80u) << 8) |
               (((__float_as_uint(c) >> 24) & 0x80u) << 16) |
               (((__float_as_uint(d) >> 24) & 0x80u) << 24);
    }
    return f32_to_e4m3(a / s) | (f32_to_e4m3(b / s) << 8) | (f32_to_e4m3(c / s) << 16) |
           (f32_to_e4m3(d / s) << 24);
}

__global__ __launch_bounds__(kThreads) void dispatch_fp8_kernel(
    const u32x4 *__restrict__ x, int nvec, const int32_t *__restrict__ dest, int D,
    u32x2 *__restrict__ recv, float *__restrict__ scales, const int32_t *__restrict__ totals)
{
    __shared__ int32_t s_dst[kMaxTopk];
    if (totals[3] != 0)
        return;
    const int64_t t = blockIdx.x;
    load_destinations(dest, D, t, s_dst);
    const int nblk = nvec / 16;                     // 128-channel blocks per row
    const u32x4 *xr = x + t * nvec;
    const int sub = threadIdx.x & 15;               // lane within the 16-lane group
    for (int c = threadIdx.x; c < nvec; c += kThreads) {
        const u32x4 v = __builtin_nontemporal_load(xr + c);
        const float f0 = bf16_lo(v.x), f1 = bf16_hi(v.x), f2 = bf16_lo(v.y), f3 = bf16_hi(v.y);
        const float f4 = bf16_lo(v.z), f5 = bf16_hi(v.z), f6 = bf16_lo(v.w), f7 = bf16_hi(v.w);
        float m = fmaxf(fmaxf(fmaxf(fabsf(f0), fabsf(f1)), fmaxf(fabsf(f2), fabsf(f3))),
                        fmaxf(fmaxf(fabsf(f4), fabsf(f5)), fmaxf(fabsf(f6), fabsf(f7))));
#pragma unroll
        for (int d = 8; d > 0; d >>= 1)
            m = fmaxf(m, __shfl_xor(m, d, 16));
        const float s = m / 448.0f;
        const bool zero = (m == 0.0f);
        u32x2 q;
        q.x = quantize4(f0, f1, f2, f3, s, zero);
        q.y = quantize4(f4, f5, f6, f7, s, zero);
        const int blk = c >> 4;
        for (int d = 0; d < D; ++d) {
            const int64_t r = s_dst[d];
            if (r < 0)
                continue;
            __builtin_nontemporal_store(q, recv + r * nvec + c);
            if (sub == 0)
                scales[r * nblk + blk] = s;
        }
    }
}

__global__ void f32_to_e4m3_kernel(const float *__restrict__ in, uint8_t *__restrict__ out,
                                   int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = (uint8_t)f32_to_e4m3(in[i]);
}

}  // namespace

hipError_t launch_dispatch_bf16(const Geometry &g, const epx_layout &L, const void *x,
                                int32_t hidden, void *recv, hipStream_t stream)
{
    const int32_t *dest = g.relay ? L.relay_slot : L.slot;
    const int D = g.relay ? g.H : g.k;
    hipLaunchKernelGGL(dispatch_bf16_kernel, dim3(g.T), dim3(kThreads), 0, stream,
                       (const u32x4 *)x, hidden / 8, dest, D, (u32x4 *)recv,
                       (const int32_t *)L.totals);
    return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const Geometry &g, const epx_layout &L, const void *x,
                               int32_t hidden, void *recv, float *scales, hipStream_t stream)
{
    const int32_t *dest = g.relay ? L.relay_slot : L.slot;
    const int D = g.relay ? g.H : g.k;
    hipLaunchKernelGGL(dispatch_fp8_kernel, dim3(g.T), dim3(kThreads), 0, stream,
                       (const u32x4 *)x, hidden / 8, dest, D, (u32x2 *)recv, scales,
                       (const int32_t *)L.totals);
    return hipGetLastError();
}

hipError_t launch_f32_to_e4m3(const float *in, uint8_t *out, int64_t n, hipStream_t stream)
{
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(f32_to_e4m3_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace epx
