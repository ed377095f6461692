// epx_relay.hip -- receive side of the host relay and the two-level combine.
//
// Mode 2 of the digest "Balancing and Beyond: Communication-Centric
// Optimizations in Expert Parallelism" (section 3.2, Figure 3): a token goes
// to each destination host once, to the GPU there whose local index equals
// the sender's, which hands it on to the token's experts on that host; the
// results come back the same way, pre-summed over that host's experts into
// one partial per token, and the source adds the partials of its hosts.
//
//   relay_fanout:   relay row r -> per-expert rows slot[t, j] of every j with
//                   fanout_expert[r, j] >= 0 (bf16 rows, or fp8 codes +
//                   scales); one workgroup reads the row once and its waves
//                   stream whole destination rows, 16 KiB per wave in flight
//                   (the relay rows come from HBM: 4 KiB bursts measured
//                   125.5 us at 4096 x 7168 bf16, 16 KiB 121.3 us).
//   relay_partials: relay row r = (t, h) -> partial[r] = sum over those j,
//                   ascending, of w[t, j] * y[slot[t, j]] in fp32 fma from +0,
//                   stored as fp32 or rounded to bf16 (the return wire form).
//   relay_finish:   out[t] = bf16(sum over h ascending of partial[relay_slot[t, h]]),
//                   fp32 adds from +0.
//
// All three are HBM-bound gathers/scatters like dispatch and combine. Relay
// rows are visited up to the row capacity; workgroups past totals[1] (the
// rows in use) return at once.
#include "epx_device.h"

namespace epx {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBurst = 16;   // fan-out: row vectors per lane loaded before its stores

// The fan-out list of relay row r in ascending j: (destination slot, j).
// Returns its length; s_dst / s_j hold up to k entries. Every thread calls it.
// (Checked builds drop slots at or past dst_rows, counted.)
__device__ __forceinline__ int fanout_list(const epx_layout &L, int k, int64_t r, int t,
                                           int32_t *s_dst, int32_t *s_j, int32_t *s_n,
                                           int64_t dst_rows, unsigned long long *viol)
{
    if (threadIdx.x < kWave) {
        // k <= 64: one lane per j, compacted in j order with a ballot prefix
        const int j = threadIdx.x;
        bool on = j < k && L.fanout_expert[r * k + j] >= 0;
        const int o = on ? L.slot[(int64_t)t * k + j] : 0;
        on = on && in_bounds(o, dst_rows, viol);
        const uint64_t bal = __ballot(on);
        if (on) {
            const int pos = __popcll(bal & ((1ull << j) - 1ull));
            s_dst[pos] = o;
            s_j[pos] = j;
        }
        if (j == 0)
            *s_n = __popcll(bal);
    }
    __syncthreads();
    return *s_n;
}

// Rows are row_vec 16-byte vectors; nsc float32 scales per row (fp8) or 0.
__global__ __launch_bounds__(kThreads) void relay_fanout_kernel(
    const u32x4 *__restrict__ src, const float *__restrict__ src_sc, int row_vec, int nsc,
    int slice, int k, epx_layout L, u32x4 *__restrict__ dst, float *__restrict__ dst_sc,
    int64_t T, int64_t relay_cap, int64_t cap, unsigned long long *viol)
{
    __shared__ int32_t s_dst[kMaxTopk], s_j[kMaxTopk], s_n;
    if (L.totals[3] != 0)
        return;
    const int64_t r = item_index();
    if (r >= L.totals[1])
        return;   // past the relay rows in use (also past the grid's last row)
    const int t = L.relay_token[r];
    if (kChecked && ((uint64_t)r >= (uint64_t)relay_cap || (uint64_t)t >= (uint64_t)T)) {
        if (threadIdx.x == 0)
            atomicAdd(viol, 1ull);   // checked builds: a relay row or token out of range
        return;
    }
    const int n = fanout_list(L, k, r, t, s_dst, s_j, &s_n, cap, viol);
    const int c_beg = blockIdx.y * slice;
    const int c_end = min(row_vec, c_beg + slice);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const u32x4 *row = src + r * row_vec;
    for (int d = wave; d < n; d += kWaves) {
        const int64_t o = s_dst[d];
        u32x4 *out = dst + o * row_vec;
        for (int c0 = c_beg + lane; c0 < c_end; c0 += kWave * kBurst) {
            u32x4 v[kBurst];
#pragma unroll
            for (int i = 0; i < kBurst; ++i) {
                const int c = c0 + i * kWave;
                if (c < c_end)
                    v[i] = row[c];
            }
#pragma unroll
            for (int i = 0; i < kBurst; ++i) {
                const int c = c0 + i * kWave;
                if (c < c_end)
                    __builtin_nontemporal_store(v[i], out + c);
            }
        }
        if (nsc > 0 && blockIdx.y == 0)
            for (int q = lane; q < nsc; q += kWave)
                dst_sc[o * nsc + q] = src_sc[r * nsc + q];
    }
}

// Partials: lanes own 8 channels (one 16-byte bf16 vector of y) in each of
// kParChunks chunks; the loads of up to kParBatch expert rows for all of a
// lane's chunks are issued before the first fma. fp32 output is two 16-byte
// vectors per chunk, bf16 one.
constexpr int kParChunks = 4;
constexpr int kParBatch = 4;

template <bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void relay_partials_kernel(
    const u32x4 *__restrict__ y, int nvec, int slice, const float *__restrict__ w, int k,
    epx_layout L, void *__restrict__ partials, int64_t T, int64_t part_cap, int64_t y_rows,
    unsigned long long *viol)
{
    __shared__ int32_t s_dst[kMaxTopk], s_j[kMaxTopk], s_n;
    __shared__ float s_w[kMaxTopk];
    if (L.totals[3] != 0)
        return;
    const int64_t r = item_index();
    if (r >= L.totals[1])
        return;   // past the relay rows in use (also past the grid's last row)
    const int t = L.relay_token[r];
    if (kChecked && ((uint64_t)r >= (uint64_t)part_cap || (uint64_t)t >= (uint64_t)T)) {
        if (threadIdx.x == 0)
            atomicAdd(viol, 1ull);   // checked builds: a relay row or token out of range
        return;
    }
    const int n = fanout_list(L, k, r, t, s_dst, s_j, &s_n, y_rows, viol);
    if ((int)threadIdx.x < n)
        s_w[threadIdx.x] = w[(int64_t)t * k + s_j[threadIdx.x]];
    __syncthreads();
    const int c_beg = blockIdx.y * slice;
    const int c_end = min(nvec, c_beg + slice);
    for (int c0 = c_beg + threadIdx.x; c0 < c_end; c0 += kThreads * kParChunks) {
        float acc[kParChunks][8];
#pragma unroll
        for (int i = 0; i < kParChunks; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[i][q] = 0.0f;
        for (int j0 = 0; j0 < n; j0 += kParBatch) {
            u32x4 v[kParBatch][kParChunks];
#pragma unroll
            for (int jj = 0; jj < kParBatch; ++jj)
#pragma unroll
                for (int i = 0; i < kParChunks; ++i) {
                    const int c = c0 + i * kThreads;
                    if (j0 + jj < n && c < c_end)
                        v[jj][i] = __builtin_nontemporal_load(y + (int64_t)s_dst[j0 + jj] * nvec + c);
                }
#pragma unroll
            for (int jj = 0; jj < kParBatch; ++jj) {
                if (j0 + jj >= n)
                    break;
                const float wj = s_w[j0 + jj];
#pragma unroll
                for (int i = 0; i < kParChunks; ++i) {
                    acc[i][0] = __builtin_fmaf(wj, bf16_lo(v[jj][i].x), acc[i][0]);
                    acc[i][1] = __builtin_fmaf(wj, bf16_hi(v[jj][i].x), acc[i][1]);
                    acc[i][2] = __builtin_fmaf(wj, bf16_lo(v[jj][i].y), acc[i][2]);
                    acc[i][3] = __builtin_fmaf(wj, bf16_hi(v[jj][i].y), acc[i][3]);
                    acc[i][4] = __builtin_fmaf(wj, bf16_lo(v[jj][i].z), acc[i][4]);
                    acc[i][5] = __builtin_fmaf(wj, bf16_hi(v[jj][i].z), acc[i][5]);
                    acc[i][6] = __builtin_fmaf(wj, bf16_lo(v[jj][i].w), acc[i][6]);
                    acc[i][7] = __builtin_fmaf(wj, bf16_hi(v[jj][i].w), acc[i][7]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kParChunks; ++i) {
            const int c = c0 + i * kThreads;
            if (c >= c_end)
                continue;
            if (BF16_OUT) {
                u32x4 o;
                o.x = f32_to_bf16(acc[i][0]) | (f32_to_bf16(acc[i][1]) << 16);
                o.y = f32_to_bf16(acc[i][2]) | (f32_to_bf16(acc[i][3]) << 16);
                o.z = f32_to_bf16(acc[i][4]) | (f32_to_bf16(acc[i][5]) << 16);
                o.w = f32_to_bf16(acc[i][6]) | (f32_to_bf16(acc[i][7]) << 16);
                __builtin_nontemporal_store(o, (u32x4 *)partials + r * nvec + c);
            } else {
                u32x4 *o = (u32x4 *)partials + (r * nvec + c) * 2;
                const u32x4 a = {__float_as_uint(acc[i][0]), __float_as_uint(acc[i][1]),
                                 __float_as_uint(acc[i][2]), __float_as_uint(acc[i][3])};
                const u32x4 b = {__float_as_uint(acc[i][4]), __float_as_uint(acc[i][5]),
                                 __float_as_uint(acc[i][6]), __float_as_uint(acc[i][7])};
                __builtin_nontemporal_store(a, o);
                __builtin_nontemporal_store(b, o + 1);
            }
        }
    }
}

// Finish: lanes own 8 channels in each of FinShape::chunks 16-byte chunks of
// the token's output row; the loads of up to FinShape::batch partial rows
// are issued before the first add (the adds then run in ascending host
// order). Measured on MI355X: 4 chunks x 2 rows for float32 partials, 2 x 4
// for bf16 ones.
template <bool BF16_IN>
struct FinShape {
    static constexpr int chunks = BF16_IN ? 2 : 4;
    static constexpr int batch = BF16_IN ? 4 : 2;
};

template <bool BF16_IN>
__device__ __forceinline__ void load_partial(const void *partials, int64_t r, int nvec, int c,
                                             float p[8])
{
    if (BF16_IN) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4 *)partials + r * nvec + c);
        p[0] = bf16_lo(v.x); p[1] = bf16_hi(v.x); p[2] = bf16_lo(v.y); p[3] = bf16_hi(v.y);
        p[4] = bf16_lo(v.z); p[5] = bf16_hi(v.z); p[6] = bf16_lo(v.w); p[7] = bf16_hi(v.w);
    } else {
        const u32x4 *src = (const u32x4 *)partials + (r * nvec + c) * 2;
        const u32x4 a = __builtin_nontemporal_load(src), b = __builtin_nontemporal_load(src + 1);
        p[0] = __uint_as_float(a.x); p[1] = __uint_as_float(a.y);
        p[2] = __uint_as_float(a.z); p[3] = __uint_as_float(a.w);
        p[4] = __uint_as_float(b.x); p[5] = __uint_as_float(b.y);
        p[6] = __uint_as_float(b.z); p[7] = __uint_as_float(b.w);
    }
}

template <bool BF16_IN>
__global__ __launch_bounds__(kThreads) void relay_finish_kernel(
    const void *__restrict__ partials, int nvec, int slice, int H, epx_layout L,
    u32x4 *__restrict__ out, int64_t T, int64_t part_cap, unsigned long long *viol)
{
    __shared__ int32_t s_rows[kMaxHosts], s_n;
    const int64_t t = item_index();
    if (t >= T || L.totals[3] != 0)
        return;
    if (threadIdx.x < kWave) {
        const int h = threadIdx.x;
        int r = h < H ? L.relay_slot[t * H + h] : -1;
        if (r >= 0 && !in_bounds(r, part_cap, viol))
            r = -1;   // checked builds: a partial row out of range (counted)
        const uint64_t bal = __ballot(r >= 0);
        if (r >= 0)
            s_rows[__popcll(bal & ((1ull << h) - 1ull))] = r;
        if (h == 0)
            s_n = __popcll(bal);
    }
    __syncthreads();
    const int n = s_n;
    constexpr int kFinChunks = FinShape<BF16_IN>::chunks, kFinBatch = FinShape<BF16_IN>::batch;
    const int c_beg = blockIdx.y * slice;
    const int c_end = min(nvec, c_beg + slice);
    for (int c0 = c_beg + threadIdx.x; c0 < c_end; c0 += kThreads * kFinChunks) {
        float acc[kFinChunks][8];
#pragma unroll
        for (int i = 0; i < kFinChunks; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[i][q] = 0.0f;
        for (int q0 = 0; q0 < n; q0 += kFinBatch) {
            float p[kFinBatch][kFinChunks][8];
#pragma unroll
            for (int qq = 0; qq < kFinBatch; ++qq)
#pragma unroll
                for (int i = 0; i < kFinChunks; ++i) {
                    const int c = c0 + i * kThreads;
                    if (q0 + qq < n && c < c_end)
                        load_partial<BF16_IN>(partials, s_rows[q0 + qq], nvec, c, p[qq][i]);
                }
#pragma unroll
            for (int qq = 0; qq < kFinBatch; ++qq) {
                if (q0 + qq >= n)
                    break;
#pragma unroll
                for (int i = 0; i < kFinChunks; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[i][e] = acc[i][e] + p[qq][i][e];
            }
        }
#pragma unroll
        for (int i = 0; i < kFinChunks; ++i) {
            const int c = c0 + i * kThreads;
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

// Column slices so that about `target` workgroups cover `rows` rows.
int slices_for(int64_t rows, int nvec, int align, int target)
{
    int want = rows >= target ? 1 : (int)((target + rows - 1) / rows);
    int width = (nvec + want - 1) / want;
    width = ((width + align - 1) / align) * align;
    if (width < 4 * align && nvec > 4 * align)
        width = 4 * align;
    return width < nvec ? width : nvec;
}

}  // namespace

hipError_t launch_relay_fanout(const Geometry &g, const epx_layout &L, const void *relay_rows,
                               const float *relay_scales, int64_t relay_cap, int64_t row_bytes,
                               int nsc, void *recv, float *recv_scales, int64_t cap,
                               hipStream_t stream)
{
    const int64_t rows = relay_rows_cap(g);   // relay rows of the layout (<= relay_cap)
    const int row_vec = (int)(row_bytes / 16);
    const int slice = slices_for(rows, row_vec, kWave, 2048);
    const dim3 grid = item_grid(rows, (row_vec + slice - 1) / slice);
    launch(relay_fanout_kernel, grid, dim3(kThreads), 0, stream,
                       (const u32x4 *)relay_rows, relay_scales, row_vec, nsc, slice, g.k, L,
                       (u32x4 *)recv, recv_scales, (int64_t)g.T,
                       relay_cap < rows ? relay_cap : rows, cap, g.viol);
    return hipGetLastError();
}

hipError_t launch_relay_partials(const Geometry &g, const epx_layout &L, const void *y,
                                 int64_t y_rows, const float *w, int32_t hidden, bool bf16_out,
                                 void *partials, int64_t part_cap, hipStream_t stream)
{
    const int64_t rows = relay_rows_cap(g);
    const int nvec = hidden / 8;
    const int slice = slices_for(rows, nvec, kWave, 2048);
    const dim3 grid = item_grid(rows, (nvec + slice - 1) / slice);
    const int64_t pc = part_cap < rows ? part_cap : rows;
    if (bf16_out)
        launch(relay_partials_kernel<true>, grid, dim3(kThreads), 0, stream,
                           (const u32x4 *)y, nvec, slice, w, g.k, L, partials, (int64_t)g.T, pc,
                           y_rows, g.viol);
    else
        launch(relay_partials_kernel<false>, grid, dim3(kThreads), 0, stream,
                           (const u32x4 *)y, nvec, slice, w, g.k, L, partials, (int64_t)g.T, pc,
                           y_rows, g.viol);
    return hipGetLastError();
}

hipError_t launch_relay_finish(const Geometry &g, const epx_layout &L, const void *partials,
                               int64_t part_cap, bool bf16_in, int32_t hidden, void *out,
                               hipStream_t stream)
{
    const int nvec = hidden / 8;
    const int slice = slices_for(g.T, nvec, kWave, 2048);
    const dim3 grid = item_grid(g.T, (nvec + slice - 1) / slice);
    if (bf16_in)
        launch(relay_finish_kernel<true>, grid, dim3(kThreads), 0, stream, partials,
                           nvec, slice, g.H, L, (u32x4 *)out, (int64_t)g.T, part_cap, g.viol);
    else
        launch(relay_finish_kernel<false>, grid, dim3(kThreads), 0, stream, partials,
                           nvec, slice, g.H, L, (u32x4 *)out, (int64_t)g.T, part_cap, g.viol);
    return hipGetLastError();
}

}  // namespace epx
