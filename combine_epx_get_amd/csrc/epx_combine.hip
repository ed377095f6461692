// epx_combine.hip -- k expert outputs per token -> weighted sum on gfx950.
//
// Combine gathers each token's k expert results back and sums them (digest
// "Balancing and Beyond: Communication-Centric Optimizations in Expert
// Parallelism", section 3.2 "Combine sums", and section 3.4: combine buffers
// hold batch x k rows). The sum is weighted by the gate weights, accumulated
// in float32 as acc = fma(w_j, y_j, acc) for j = 0..k-1 from +0 and rounded
// once to bf16, nearest even: the same order on every element, so results
// are deterministic and independent of the launch shape.
//
// One workgroup per token; each lane owns 8 channels (one 16-byte vector per
// row). A lane issues the loads of up to 8 expert rows before its first FMA,
// so 8 x 16 bytes per lane are in flight: an HBM-bound gather that reads
// T*k*h*2 bytes and writes T*h*2.
#include "epx_internal.h"

namespace epx {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;    // expert rows loaded before the FMAs

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return ((u >> 16) & 0x8000u) | 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const u32x4 *__restrict__ y, int nvec, const int32_t *__restrict__ slot,
    const float *__restrict__ w, int k, u32x4 *__restrict__ out,
    const int32_t *__restrict__ totals)
{
    __shared__ int32_t s_row[kMaxTopk];
    __shared__ float s_w[kMaxTopk];
    if (totals[3] != 0)
        return;   // the layout saw out-of-range expert ids
    const int64_t t = blockIdx.x;
    if (threadIdx.x < k) {
        s_row[threadIdx.x] = slot[t * k + threadIdx.x];
        s_w[threadIdx.x] = w[t * k + threadIdx.x];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < nvec; c += kThreads) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += kBatch) {
            u32x4 v[kBatch];
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj)
                if (j0 + jj < k)
                    v[jj] = __builtin_nontemporal_load(y + (int64_t)s_row[j0 + jj] * nvec + c);
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                if (j0 + jj >= k)
                    break;
                const float wj = s_w[j0 + jj];
                acc[0] = __builtin_fmaf(wj, bf16_lo(v[jj].x), acc[0]);
                acc[1] = __builtin_fmaf(wj, bf16_hi(v[jj].x), acc[1]);
                acc[2] = __builtin_fmaf(wj, bf16_lo(v[jj].y), acc[2]);
                acc[3] = __builtin_fmaf(wj, bf16_hi(v[jj].y), acc[3]);
                acc[4] = __builtin_fmaf(wj, bf16_lo(v[jj].z), acc[4]);
                acc[5] = __builtin_fmaf(wj, bf16_hi(v[jj].z), acc[5]);
                acc[6] = __builtin_fmaf(wj, bf16_lo(v[jj].w), acc[6]);
                acc[7] = __builtin_fmaf(wj, bf16_hi(v[jj].w), acc[7]);
            }
        }
        u32x4 o;
        o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
        o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
        __builtin_nontemporal_store(o, out + t * nvec + c);
    }
}

}  // namespace

hipError_t launch_combine(const Geometry &g, const epx_layout &L, const void *y, const float *w,
                          int32_t hidden, void *out, hipStream_t stream)
{
    hipLaunchKernelGGL(combine_kernel, dim3(g.T), dim3(kThreads), 0, stream, (const u32x4 *)y,
                       hidden / 8, (const int32_t *)L.slot, w, g.k, (u32x4 *)out,
                       (const int32_t *)L.totals);
    return hipGetLastError();
}

}  // namespace epx
