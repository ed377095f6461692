// epx_dispatch.hip -- token rows -> destination rows on gfx950.
//
// Per-expert mode writes one copy of a token's row per destination expert
// (DeepEP's default, Mode 1 of the digest "Balancing and Beyond:
// Communication-Centric Optimizations in Expert Parallelism", section 3.2);
// relay mode writes one copy per destination host (Mode 2 with
// de-redundancy). Either way the kernel reads each token row once from HBM
// and writes it to each of the token's destination rows: T*h*2 bytes in,
// rows*h*2 bytes out, an HBM-bound scatter dominated by writes.
//
// Launch shape: one workgroup per (token, column slice); slices exist only to
// give small batches enough workgroups. Large batches whose tokens have
// fewer rows than a workgroup has waves give every wave a token of its own
// instead (below). Each wave streams whole destination
// rows (waves take the token's rows round-robin) in bursts of 16 KiB: every
// lane loads 16 x 16 bytes of the token row (L2 serves the repeats), all in
// flight together, and stores them with nontemporal 16-byte stores. Writing
// one row at a time per wave keeps each wave's write stream contiguous,
// which this memory system drains markedly faster than stores interleaved
// over all of a token's rows. The deep burst matters when x comes from HBM
// rather than from the caches: measured on MI355X at 4096 x 7168, top-8,
// 4 KiB bursts took 118.7 us after a cache flush, 16 KiB bursts 109.2 us
// (95.5 and 96.0 us with warm caches).
//
// The fp8 variant quantises bf16 to fp8 inside the dispatch (digest section
// 3.1): per token and 128-channel block, scale = amax/448 and
// code = E4M3(x / scale), the float32 quotient correctly rounded, then
// rounded to nearest even in E4M3. The workgroup quantises its slice once into LDS (a
// 16-lane group owns one 128-channel block: 8 bf16 per lane, block maximum by
// lane shuffles), then the waves stream the codes and scales from LDS to the
// destination rows.
#include "epx_device.h"

namespace epx {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBurst = 16;             // bf16: 16-byte chunks per lane per burst
constexpr int kBurstFp8 = 4;           // fp8: code vectors per lane per burst (from LDS)
constexpr int kMaxSliceVec = 4096;     // fp8 slice bound: LDS holds slice*8 code bytes
constexpr int kPre = 4;                // fp8: 16-byte chunks loaded per thread before converting

// Destination rows outside [*lo_p, *hi_p) are skipped (one expert group's
// rows); lo_p == nullptr keeps every row.
__device__ __forceinline__ void row_range(const int32_t *lo_p, const int32_t *hi_p, int &lo, int &hi)
{
    lo = 0;
    hi = 0x7FFFFFFF;
    if (lo_p) {
        lo = *lo_p;
        hi = *hi_p;
    }
}

// wave_tokens != 0: every wave takes a token of its own (kWaves tokens per
// workgroup, one column slice), loads its row once and stores it to all of
// the token's D <= 64 rows; the launch uses it only for whole rows of one
// burst, no group range, many tokens and few rows per token.
__global__ __launch_bounds__(kThreads) void dispatch_bf16_kernel(
    const u32x4 *__restrict__ x, int nvec, int slice, const int32_t *__restrict__ dest, int D,
    u32x4 *__restrict__ recv, int64_t cap, unsigned long long *viol,
    const int32_t *__restrict__ totals, const int32_t *lo_p, const int32_t *hi_p, int64_t T,
    int wave_tokens)
{
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (wave_tokens) {
        const int64_t tw = item_index() * kWaves + wave;
        if (tw >= T)
            return;   // past the last token (no barrier below)
        const u32x4 *xw = x + tw * nvec;
        u32x4 v[kBurst];
#pragma unroll
        for (int i = 0; i < kBurst; ++i) {
            const int c = lane + i * kWave;
            if (c < nvec)
                v[i] = xw[c];
        }
        // the error word and all destinations load beside the row
        const int bad = totals[3];
        const int rl = lane < D ? dest[tw * D + lane] : -1;
        if (bad != 0)
            return;   // the layout saw out-of-range expert ids: its rows are undefined
        for (int d = 0; d < D; ++d) {
            const int64_t r = __shfl(rl, d);
            if (r < 0 || !in_bounds(r, cap, viol))
                continue;   // relay: no row for this host
            u32x4 *dst = recv + r * nvec;
#pragma unroll
            for (int i = 0; i < kBurst; ++i) {
                const int c = lane + i * kWave;
                if (c < nvec)
                    __builtin_nontemporal_store(v[i], dst + c);
            }
        }
        return;
    }
    const int64_t t = item_index();
    if (t >= T)
        return;   // past the last token
    int lo, hi;
    const int c_beg = blockIdx.y * slice;
    const int c_end = min(nvec, c_beg + slice);
    const u32x4 *xr = x + t * nvec;
    if (c_end - c_beg <= kWave * kBurst) {
        // The slice fits one burst: each wave loads it once, together with
        // the error word and its destinations (no load waits for another),
        // and stores the same registers to each of its rows.
        u32x4 v[kBurst];
#pragma unroll
        for (int i = 0; i < kBurst; ++i) {
            const int c = c_beg + lane + i * kWave;
            if (c < c_end)
                v[i] = xr[c];
        }
        const int bad = totals[3];
        int64_t r0 = wave < D ? dest[t * D + wave] : -1;
        row_range(lo_p, hi_p, lo, hi);
        if (bad != 0)
            return;   // the layout saw out-of-range expert ids: its rows are undefined
        for (int d = wave; d < D; d += kWaves) {
            const int64_t r = d == wave ? r0 : dest[t * D + d];
            if (r < lo || r >= hi || !in_bounds(r, cap, viol))
                continue;
            u32x4 *dst = recv + r * nvec;
#pragma unroll
            for (int i = 0; i < kBurst; ++i) {
                const int c = c_beg + lane + i * kWave;
                if (c < c_end)
                    __builtin_nontemporal_store(v[i], dst + c);
            }
        }
        return;
    }
    if (totals[3] != 0)
        return;   // the layout saw out-of-range expert ids
    row_range(lo_p, hi_p, lo, hi);
    for (int d = wave; d < D; d += kWaves) {
        const int64_t r = dest[t * D + d];
        if (r < lo || r >= hi || !in_bounds(r, cap, viol))
            continue;
        u32x4 *dst = recv + r * nvec;
        for (int c0 = c_beg + lane; c0 < c_end; c0 += kWave * kBurst) {
            u32x4 v[kBurst];
#pragma unroll
            for (int i = 0; i < kBurst; ++i) {
                const int c = c0 + i * kWave;
                if (c < c_end)
                    v[i] = xr[c];
            }
#pragma unroll
            for (int i = 0; i < kBurst; ++i) {
                const int c = c0 + i * kWave;
                if (c < c_end)
                    __builtin_nontemporal_store(v[i], dst + c);
            }
        }
    }
}

// Slice [c_beg, c_end) of token t, in 16-byte bf16 chunks (c_beg, c_end and
// slice are multiples of 16 chunks = 128 channels). LDS: codes of the slice
// (8 bytes per chunk) then one scale per 128-channel block.
__global__ __launch_bounds__(kThreads) void dispatch_fp8_kernel(
    const u32x4 *__restrict__ x, int nvec, int slice, const int32_t *__restrict__ dest, int D,
    uint8_t *__restrict__ recv, float *__restrict__ scales, int64_t cap,
    unsigned long long *viol, const int32_t *__restrict__ totals, const int32_t *lo_p,
    const int32_t *hi_p, int64_t T)
{
    extern __shared__ u32x4 s_codes[];   // slice/2 vectors of 16 codes
    const int64_t t = item_index();
    if (t >= T || totals[3] != 0)
        return;
    int lo, hi;
    row_range(lo_p, hi_p, lo, hi);
    if (lo_p) {
        // no row of this group: skip the quantisation (every wave reads all
        // D <= 64 destinations, so the whole workgroup agrees)
        bool any = false;
        for (int d = threadIdx.x % kWave; d < D; d += kWave) {
            const int r = dest[t * D + d];
            any = any || (r >= lo && r < hi);
        }
        if (!__any(any))
            return;
    }
    const int c_beg = blockIdx.y * slice;
    const int c_end = min(nvec, c_beg + slice);
    const int n = c_end - c_beg;                       // chunks in this slice
    float *s_scale = (float *)(s_codes + (slice >> 1));
    const u32x4 *xr = x + t * nvec;

    // quantise the slice once (16 lanes per 128-channel block)
    quantize_slice_to_lds<kThreads, kPre>(xr, c_beg, n, (u32x2 *)s_codes, s_scale);
    __syncthreads();

    // stream codes (16 bytes = 16 codes per lane) and scales to each row
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nq = n >> 1;                 // 16-byte code vectors in the slice
    const int nblk = n >> 4;               // scales in the slice
    const int row_vec = nvec >> 1;         // 16-byte code vectors per row
    const int row_blk = nvec >> 4;         // scales per row
    for (int d = wave; d < D; d += kWaves) {
        const int64_t r = dest[t * D + d];
        if (r < lo || r >= hi || !in_bounds(r, cap, viol))
            continue;
        u32x4 *dst = (u32x4 *)(recv) + r * row_vec + (c_beg >> 1);
        for (int c0 = lane; c0 < nq; c0 += kWave * kBurstFp8) {
            u32x4 v[kBurstFp8];
#pragma unroll
            for (int i = 0; i < kBurstFp8; ++i) {
                const int c = c0 + i * kWave;
                if (c < nq)
                    v[i] = s_codes[c];
            }
#pragma unroll
            for (int i = 0; i < kBurstFp8; ++i) {
                const int c = c0 + i * kWave;
                if (c < nq)
                    __builtin_nontemporal_store(v[i], dst + c);
            }
        }
        for (int b = lane; b < nblk; b += kWave)
            scales[r * row_blk + (c_beg >> 4) + b] = s_scale[b];
    }
}

__global__ void f32_to_e4m3_kernel(const float *__restrict__ in, uint8_t *__restrict__ out,
                                   int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = (uint8_t)(e4m3_pair(in[i], 0.0f) & 0xFFu);
}

}  // namespace

hipError_t launch_dispatch_bf16(const Geometry &g, const epx_layout &L, const void *x,
                                int32_t hidden, void *recv, int64_t cap, int group,
                                hipStream_t stream)
{
    const int32_t *lo_p = group < 0 ? nullptr : L.group_offset + group * g.R;
    const int32_t *hi_p = group < 0 ? nullptr : L.group_offset + (group + 1) * g.R;
    const int32_t *dest = g.relay ? L.relay_slot : L.slot;
    const int D = g.relay ? g.H : g.k;
    const int nvec = hidden / 8;
    // A wave per token where a token has fewer rows than a workgroup has
    // waves (relay to at most 3 hosts), so that no wave idles, when rows fit
    // one burst and tokens are many. Measured on MI355X, 4096 x 7168, relay
    // to 2 hosts: 24.9-25.8 us against 26.2-26.4 for a workgroup per token
    // (two machines); with 4 rows per token the two shapes are even; with
    // top-8 per-expert rows the workgroup per token is faster warm (92.8
    // against 95.8 us, five repetitions on one machine) and 2 us slower
    // after a cache flush.
    const bool wave_tokens = lo_p == nullptr && nvec <= kWave * kBurst && g.T >= 2048 && D < kWaves;
    const int slice = wave_tokens ? nvec : slice_width(g.T, nvec, kWave, 1 << 30, 2048);
    const dim3 grid = wave_tokens ? item_grid((g.T + kWaves - 1) / kWaves, 1)
                                  : item_grid(g.T, (nvec + slice - 1) / slice);
    launch(dispatch_bf16_kernel, grid, dim3(kThreads), 0, stream, (const u32x4 *)x,
                       nvec, slice, dest, D, (u32x4 *)recv, cap, g.viol, (const int32_t *)L.totals,
                       lo_p, hi_p, (int64_t)g.T, (int)wave_tokens);
    return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const Geometry &g, const epx_layout &L, const void *x,
                               int32_t hidden, void *recv, float *scales, int64_t cap, int group,
                               hipStream_t stream)
{
    const int32_t *lo_p = group < 0 ? nullptr : L.group_offset + group * g.R;
    const int32_t *hi_p = group < 0 ? nullptr : L.group_offset + (group + 1) * g.R;
    const int32_t *dest = g.relay ? L.relay_slot : L.slot;
    const int D = g.relay ? g.H : g.k;
    const int nvec = hidden / 8;          // multiple of 16 (hidden % 128 == 0)
    // The fp8 workgroup quantises before it stores, so it needs more,
    // smaller workgroups to overlap the two: about 2048 * D per batch
    // (measured on MI355X: 2 slices for 4 relay rows per token at T = 4096,
    // 4 slices for 8 per-expert rows).
    // One group's dispatch writes about k/m rows per token.
    const int rows_per_token = group < 0 ? D : (D + g.m - 1) / g.m;
    const int slice = slice_width(g.T, nvec, 16, kMaxSliceVec, 2048 * rows_per_token);
    const dim3 grid = item_grid(g.T, (nvec + slice - 1) / slice);
    const size_t lds = (size_t)slice * 8 + (size_t)(slice / 16) * sizeof(float);
    launch(dispatch_fp8_kernel, grid, dim3(kThreads), lds, stream, (const u32x4 *)x,
                       nvec, slice, dest, D, (uint8_t *)recv, scales, cap, g.viol,
                       (const int32_t *)L.totals, lo_p, hi_p, (int64_t)g.T);
    return hipGetLastError();
}

hipError_t launch_f32_to_e4m3(const float *in, uint8_t *out, int64_t n, hipStream_t stream)
{
    const int64_t blocks = (n + 255) / 256;
    launch(f32_to_e4m3_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace epx
