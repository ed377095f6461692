// epx_combine.hip -- k expert outputs per token -> weighted sum on gfx950.
//
// Combine gathers each token's k expert results back and sums them (digest
// "Balancing and Beyond: Communication-Centric Optimizations in Expert
// Parallelism", section 3.2, the combine step, and section 3.4: combine
// buffers hold batch x k rows). The sum is weighted by the gate weights, accumulated
// in float32 as acc = fma(w_j, y_j, acc) for j = 0..k-1 from +0 and rounded
// once to bf16, nearest even: the same order on every element, so results
// are deterministic and independent of the launch shape.
//
// One workgroup per (token, column slice); each lane owns 8 channels in each
// of its 16-byte chunks (two per lane from 256 tokens on, one below) and
// issues the loads of up to 8 expert rows for all its chunks before the
// first fma (up to 16 x 16 bytes in flight per lane).
// Reads T*k*h*2 bytes and writes T*h*2: an HBM-bound gather.
#include "epx_device.h"

namespace epx {
namespace {

constexpr int kBatch = 8;    // expert rows loaded before the fmas
constexpr int kChunks = 2;   // 16-byte chunks per lane (group combine)

template <int CHUNKS>
__global__ __launch_bounds__(1024) void combine_kernel(
    const u32x4 *__restrict__ y, int nvec, int slice, const int32_t *__restrict__ slot,
    const float *__restrict__ w, int k, u32x4 *__restrict__ out, int64_t y_rows,
    unsigned long long *viol, const int32_t *__restrict__ totals, int64_t T)
{
    __shared__ int32_t s_row[kMaxTopk];
    __shared__ float s_w[kMaxTopk];
    const int64_t t = item_index();
    if (t >= T)
        return;   // past the last token
    const int c_beg = blockIdx.y * slice;
    const int c_end = min(nvec, c_beg + slice);
    // the error word, the slots and the weights in one round trip
    const int bad = totals[3];
    if ((int)threadIdx.x < k) {
        const int r = slot[t * k + threadIdx.x];
        s_row[threadIdx.x] = in_bounds(r, y_rows, viol) ? r : 0;   // checked builds only
        s_w[threadIdx.x] = w[t * k + threadIdx.x];
    }
    __syncthreads();
    if (bad != 0)
        return;   // the layout saw out-of-range expert ids: the slots are undefined
    for (int c0 = c_beg + threadIdx.x; c0 < c_end; c0 += blockDim.x * CHUNKS) {
        float acc[CHUNKS][8];
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[i][q] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += kBatch) {
            u32x4 v[CHUNKS][kBatch];
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj)
#pragma unroll
                for (int i = 0; i < CHUNKS; ++i) {
                    const int c = c0 + i * blockDim.x;
                    if (j0 + jj < k && c < c_end)
                        v[i][jj] = __builtin_nontemporal_load(y + (int64_t)s_row[j0 + jj] * nvec + c);
                }
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                if (j0 + jj >= k)
                    break;
                const float wj = s_w[j0 + jj];
#pragma unroll
                for (int i = 0; i < CHUNKS; ++i) {
                    acc[i][0] = __builtin_fmaf(wj, bf16_lo(v[i][jj].x), acc[i][0]);
                    acc[i][1] = __builtin_fmaf(wj, bf16_hi(v[i][jj].x), acc[i][1]);
                    acc[i][2] = __builtin_fmaf(wj, bf16_lo(v[i][jj].y), acc[i][2]);
                    acc[i][3] = __builtin_fmaf(wj, bf16_hi(v[i][jj].y), acc[i][3]);
                    acc[i][4] = __builtin_fmaf(wj, bf16_lo(v[i][jj].z), acc[i][4]);
                    acc[i][5] = __builtin_fmaf(wj, bf16_hi(v[i][jj].z), acc[i][5]);
                    acc[i][6] = __builtin_fmaf(wj, bf16_lo(v[i][jj].w), acc[i][6]);
                    acc[i][7] = __builtin_fmaf(wj, bf16_hi(v[i][jj].w), acc[i][7]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = c0 + i * blockDim.x;
            if (c >= c_end)
                continue;
            u32x4 o;
            o.x = f32_to_bf16(acc[i][0]) | (f32_to_bf16(acc[i][1]) << 16);
            o.y = f32_to_bf16(acc[i][2]) | (f32_to_bf16(acc[i][3]) << 16);
            o.z = f32_to_bf16(acc[i][4]) | (f32_to_bf16(acc[i][5]) << 16);
            o.w = f32_to_bf16(acc[i][6]) | (f32_to_bf16(acc[i][7]) << 16);
            __builtin_nontemporal_store(o, out + t * nvec + c);
        }
    }
}

// One expert group's combine (per-expert overlap, digest section 3.3): the
// token's pairs whose rows lie in the group's range [*lo_p, *hi_p) are
// compacted in ascending j; the sum starts from the float32 carry when the
// token had rows in an earlier group (rows below lo), else from +0, and goes
// to the carry when the token has rows in a later group (rows at or above
// hi), else to out as bf16. Groups' row ranges are ordered, so the three
// cases follow from comparing the token's rows with the range.
__global__ __launch_bounds__(1024) void combine_group_kernel(
    const u32x4 *__restrict__ y, int nvec, int slice, const int32_t *__restrict__ slot,
    const float *__restrict__ w, int k, const int32_t *lo_p, const int32_t *hi_p,
    float4 *__restrict__ carry, u32x4 *__restrict__ out, int64_t y_rows,
    unsigned long long *viol, const int32_t *__restrict__ totals, int64_t T)
{
    __shared__ int32_t s_row[kMaxTopk];
    __shared__ float s_w[kMaxTopk];
    __shared__ int32_t s_n, s_prior, s_later;
    const int64_t t = item_index();
    if (t >= T || totals[3] != 0)
        return;
    const int c_beg = blockIdx.y * slice;
    const int c_end = min(nvec, c_beg + slice);
    if (threadIdx.x < kWave) {   // k <= 64: one wave sees every pair
        const int j = threadIdx.x;
        const int lo = *lo_p, hi = *hi_p;
        const int r = j < k ? slot[t * k + j] : lo;
        const bool in = j < k && r >= lo && r < hi && in_bounds(r, y_rows, viol);
        const uint64_t bal_in = __ballot(in);
        const uint64_t bal_prior = __ballot(j < k && r < lo);
        const uint64_t bal_later = __ballot(j < k && r >= hi);
        if (in) {
            const int pos = __popcll(bal_in & ((1ull << j) - 1ull));
            s_row[pos] = r;
            s_w[pos] = w[t * k + j];
        }
        if (j == 0) {
            s_n = __popcll(bal_in);
            s_prior = bal_prior != 0ull;
            s_later = bal_later != 0ull;
        }
    }
    __syncthreads();
    const int n = s_n;
    if (n == 0)
        return;   // no row of this token in the group
    const bool prior = s_prior, later = s_later;
    for (int c0 = c_beg + threadIdx.x; c0 < c_end; c0 += blockDim.x * kChunks) {
        float acc[kChunks][8];
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = c0 + i * blockDim.x;
            if (prior && c < c_end) {
                const float4 a = carry[(t * nvec + c) * 2], b = carry[(t * nvec + c) * 2 + 1];
                acc[i][0] = a.x; acc[i][1] = a.y; acc[i][2] = a.z; acc[i][3] = a.w;
                acc[i][4] = b.x; acc[i][5] = b.y; acc[i][6] = b.z; acc[i][7] = b.w;
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[i][q] = 0.0f;
            }
        }
        for (int j0 = 0; j0 < n; j0 += kBatch) {
            u32x4 v[kChunks][kBatch];
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj)
#pragma unroll
                for (int i = 0; i < kChunks; ++i) {
                    const int c = c0 + i * blockDim.x;
                    if (j0 + jj < n && c < c_end)
                        v[i][jj] = __builtin_nontemporal_load(y + (int64_t)s_row[j0 + jj] * nvec + c);
                }
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                if (j0 + jj >= n)
                    break;
                const float wj = s_w[j0 + jj];
#pragma unroll
                for (int i = 0; i < kChunks; ++i) {
                    acc[i][0] = __builtin_fmaf(wj, bf16_lo(v[i][jj].x), acc[i][0]);
                    acc[i][1] = __builtin_fmaf(wj, bf16_hi(v[i][jj].x), acc[i][1]);
                    acc[i][2] = __builtin_fmaf(wj, bf16_lo(v[i][jj].y), acc[i][2]);
                    acc[i][3] = __builtin_fmaf(wj, bf16_hi(v[i][jj].y), acc[i][3]);
                    acc[i][4] = __builtin_fmaf(wj, bf16_lo(v[i][jj].z), acc[i][4]);
                    acc[i][5] = __builtin_fmaf(wj, bf16_hi(v[i][jj].z), acc[i][5]);
                    acc[i][6] = __builtin_fmaf(wj, bf16_lo(v[i][jj].w), acc[i][6]);
                    acc[i][7] = __builtin_fmaf(wj, bf16_hi(v[i][jj].w), acc[i][7]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = c0 + i * blockDim.x;
            if (c >= c_end)
                continue;
            if (later) {
                carry[(t * nvec + c) * 2] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
                carry[(t * nvec + c) * 2 + 1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
            } else {
                u32x4 o;
                o.x = f32_to_bf16(acc[i][0]) | (f32_to_bf16(acc[i][1]) << 16);
                o.y = f32_to_bf16(acc[i][2]) | (f32_to_bf16(acc[i][3]) << 16);
                o.z = f32_to_bf16(acc[i][4]) | (f32_to_bf16(acc[i][5]) << 16);
                o.w = f32_to_bf16(acc[i][6]) | (f32_to_bf16(acc[i][7]) << 16);
                __builtin_nontemporal_store(o, out + t * nvec + c);
            }
        }
    }
}

// Column slices so that small batches still give ~2048 workgroups, and the
// threads that cover one slice at `chunks` chunks per lane.
void combine_shape(const Geometry &g, int nvec, int chunks, int &slice, int &threads)
{
    int want = g.T >= 2048 ? 1 : (2048 + g.T - 1) / g.T;
    slice = (nvec + want - 1) / want;
    const int unit = kWave * chunks;
    slice = ((slice + unit - 1) / unit) * unit;
    if (slice > nvec)
        slice = nvec;
    threads = ((slice + chunks - 1) / chunks + kWave - 1) / kWave * kWave;
    if (threads > 1024)
        threads = 1024;
    if (threads < kWave)
        threads = kWave;
}

}  // namespace

hipError_t launch_combine_group(const Geometry &g, const epx_layout &L, int group, const void *y,
                                int64_t y_rows, const float *w, int32_t hidden, float *carry,
                                void *out, hipStream_t stream)
{
    const int nvec = hidden / 8;
    int slice, threads;
    combine_shape(g, nvec, kChunks, slice, threads);
    const dim3 grid = item_grid(g.T, (nvec + slice - 1) / slice);
    launch(combine_group_kernel, grid, dim3(threads), 0, stream, (const u32x4 *)y,
                       nvec, slice, (const int32_t *)L.slot, w, g.k,
                       (const int32_t *)L.group_offset + group * g.R,
                       (const int32_t *)L.group_offset + (group + 1) * g.R, (float4 *)carry,
                       (u32x4 *)out, y_rows, g.viol, (const int32_t *)L.totals, (int64_t)g.T);
    return hipGetLastError();
}

hipError_t launch_combine(const Geometry &g, const epx_layout &L, const void *y, int64_t y_rows,
                          const float *w, int32_t hidden, void *out, hipStream_t stream)
{
    const int nvec = hidden / 8;
    // Below 256 tokens one 16-byte chunk per lane: twice the workgroups for
    // the few tokens there are (HIP-graph layers at 128 tokens x 7168:
    // 13.3 -> 12.7 us); from 256 tokens on, two chunks (4096 tokens: 198.1
    // against 201.3 us with one).
    const int chunks = g.T < 256 ? 1 : 2;
    int slice, threads;
    combine_shape(g, nvec, chunks, slice, threads);
    const dim3 grid = item_grid(g.T, (nvec + slice - 1) / slice);
    if (chunks == 1)
        launch(combine_kernel<1>, grid, dim3(threads), 0, stream, (const u32x4 *)y,
                           nvec, slice, (const int32_t *)L.slot, w, g.k, (u32x4 *)out, y_rows,
                           g.viol, (const int32_t *)L.totals, (int64_t)g.T);
    else
        launch(combine_kernel<2>, grid, dim3(threads), 0, stream, (const u32x4 *)y,
                           nvec, slice, (const int32_t *)L.slot, w, g.k, (u32x4 *)out, y_rows,
                           g.viol, (const int32_t *)L.totals, (int64_t)g.T);
    return hipGetLastError();
}

}  // namespace epx
