// epx_layout.hip -- routing -> layout on gfx950.
//
// Computes, for one source rank, the counts per expert / rank / host, their
// exclusive prefixes and the destination row of every (token, expert) pair
// and of every (token, host) relay copy. The copies per expert and per host
// are the quantities the digest "Balancing and Beyond: Communication-Centric
// Optimizations in Expert Parallelism" reasons about (section 2: the busiest
// expert sets the time; section 3.2: one network copy per remote host); the
// per-rank token counts are those of the DeepEP issue "[GH-ISSUE #250]
// Profiling when rank unbalance".
//
// Three launches, no atomics on global memory and no zero-filled buffers:
//   count  (G workgroups, 64 tokens each): LDS-privatised histograms of
//          experts, of distinct ranks and hosts per token, and of bad ids;
//          each workgroup writes one column entry ws[col * G + b].
//   scan   (one wave per column): exclusive scan of every column over the G
//          workgroups with a wave-wide shuffle scan; the column total is the
//          global count.
//   assign (G workgroups): prefix of the expert counts in LDS; wave 0 walks
//          the workgroup's pairs in (token, j) order, 64 at a time, groups
//          equal expert ids with ceil(log2 E) ballots (a wave-level
//          multisplit) and takes rank-in-group = popcount(peers below me),
//          so positions are stable and independent of atomic order; wave 1
//          assigns relay rows, one token per lane, host by host with one
//          ballot each.
#include "epx_internal.h"

namespace epx {
namespace {

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int n = __shfl_up(v, d, kWave);
        if (lane >= d)
            v += n;
    }
    return v;
}

__device__ __forceinline__ int wave_max(int v)
{
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1)
        v = max(v, __shfl_xor(v, d, kWave));
    return v;
}

// ---------------------------------------------------------------- count
// LDS columns: [0, E) experts, [E, E+R) ranks, [E+R, E+R+H) hosts, E+R+H bad ids.
__global__ __launch_bounds__(256) void layout_count_kernel(const int32_t *__restrict__ idx,
                                                           Geometry g, int32_t *__restrict__ ws)
{
    extern __shared__ int32_t lds[];
    const int ncol = g.E + g.R + g.H + 1;
    int32_t *s_hist = lds;
    int32_t *s_rtok = lds + g.E;
    int32_t *s_htok = s_rtok + g.R;
    int32_t *s_bad = s_htok + g.H;

    const int b = blockIdx.x;
    const int t0 = b * kChunkTokens;
    const int nt = max(0, min(kChunkTokens, g.T - t0));
    for (int i = threadIdx.x; i < ncol; i += blockDim.x)
        lds[i] = 0;
    __syncthreads();

    const int64_t p0 = (int64_t)t0 * g.k;
    const int np = nt * g.k;
    for (int p = threadIdx.x; p < np; p += blockDim.x) {
        const int e = idx[p0 + p];
        if ((unsigned)e < (unsigned)g.E)
            atomicAdd(&s_hist[e], 1);
        else
            atomicAdd(s_bad, 1);
    }
    if (threadIdx.x < nt) {
        const int32_t *row = idx + p0 + (int64_t)threadIdx.x * g.k;
        uint64_t hosts = 0;
        for (int j = 0; j < g.k; ++j) {
            const int e = row[j];
            if ((unsigned)e >= (unsigned)g.E)
                continue;
            const int r = e / g.epr;
            bool first = true;
            for (int i = 0; i < j; ++i) {
                const int e2 = row[i];
                if ((unsigned)e2 < (unsigned)g.E && e2 / g.epr == r) {
                    first = false;
                    break;
                }
            }
            if (first)
                atomicAdd(&s_rtok[r], 1);
            const int h = r / g.rph;
            if (!((hosts >> h) & 1ull)) {
                hosts |= 1ull << h;
                atomicAdd(&s_htok[h], 1);
            }
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < ncol; c += blockDim.x)
        ws[(int64_t)c * g.G + b] = lds[c];
}

// ---------------------------------------------------------------- scan
__global__ __launch_bounds__(256) void layout_scan_kernel(Geometry g, int32_t *__restrict__ ws,
                                                          int32_t *__restrict__ expert_count,
                                                          int32_t *__restrict__ rank_tokens,
                                                          int32_t *__restrict__ host_tokens,
                                                          int32_t *__restrict__ totals)
{
    const int ncol = g.E + g.R + g.H + 1;
    const int col = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (col >= ncol)
        return;
    const int lane = lane_id();
    int32_t *c = ws + (int64_t)col * g.G;
    int carry = 0;
    for (int base = 0; base < g.G; base += kWave) {
        const int i = base + lane;
        const int v = (i < g.G) ? c[i] : 0;
        const int incl = wave_inclusive_scan(v);
        if (i < g.G)
            c[i] = carry + incl - v;
        carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
        if (col < g.E)
            expert_count[col] = carry;
        else if (col < g.E + g.R)
            rank_tokens[col - g.E] = carry;
        else if (col < g.E + g.R + g.H)
            host_tokens[col - g.E - g.R] = carry;
        else
            totals[3] = carry;
    }
}

// ---------------------------------------------------------------- assign
constexpr int kAssignThreads = 128;

// Exclusive scan of src[0, n) (global) into dst[0, n] (LDS), dst[n] = total.
__device__ void block_exclusive_scan(const int32_t *__restrict__ src, int32_t *dst, int n,
                                     int32_t *s_wsum)
{
    const int tid = threadIdx.x;
    const int per = (n + kAssignThreads - 1) / kAssignThreads;
    const int beg = min(tid * per, n), end = min(beg + per, n);
    int sum = 0;
    for (int i = beg; i < end; ++i)
        sum += src[i];
    const int incl = wave_inclusive_scan(sum);
    if (lane_id() == kWave - 1)
        s_wsum[tid / kWave] = incl;
    __syncthreads();
    int run = incl - sum + (tid >= kWave ? s_wsum[0] : 0);
    for (int i = beg; i < end; ++i) {
        dst[i] = run;
        run += src[i];
    }
    if (tid == kAssignThreads - 1)
        dst[n] = run;
}

__global__ __launch_bounds__(kAssignThreads) void layout_assign_kernel(
    const int32_t *__restrict__ idx, Geometry g, const int32_t *__restrict__ ws, epx_layout L)
{
    extern __shared__ int32_t lds[];
    int32_t *s_eoff = lds;                 // [E + 1]
    int32_t *s_base = s_eoff + g.E + 1;    // [E]  running row per expert
    int32_t *s_hoff = s_base + g.E;        // [H + 1]
    __shared__ int32_t s_wsum[2];
    __shared__ int32_t s_wmax[2];
    __shared__ int32_t s_bad;

    const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    if (tid == 0)
        s_bad = L.totals[3];
    block_exclusive_scan(L.expert_count, s_eoff, g.E, s_wsum);
    if (wave == 0) {
        const int v = lane < g.H ? L.host_tokens[lane] : 0;
        const int incl = wave_inclusive_scan(v);
        if (lane < g.H)
            s_hoff[lane] = incl - v;
        if (lane == kWave - 1)
            s_hoff[g.H] = incl;
    }
    __syncthreads();
    if (s_bad != 0)
        return;   // out-of-range ids: nothing below is defined

    if (b == 0) {
        for (int e = tid; e <= g.E; e += kAssignThreads)
            L.expert_offset[e] = s_eoff[e];
        for (int r = tid; r <= g.R; r += kAssignThreads) {
            L.rank_offset[r] = s_eoff[r * g.epr];
            if (r < g.R)
                L.rank_rows[r] = s_eoff[(r + 1) * g.epr] - s_eoff[r * g.epr];
        }
        for (int h = tid; h <= g.H; h += kAssignThreads) {
            L.host_offset[h] = s_hoff[h];
            if (h < g.H)
                L.relay_dst_rank[h] = h * g.rph + g.s % g.rph;
        }
        int m = 0;
        for (int e = tid; e < g.E; e += kAssignThreads)
            m = max(m, s_eoff[e + 1] - s_eoff[e]);
        m = wave_max(m);
        if (lane == 0)
            s_wmax[wave] = m;
        __syncthreads();
        if (tid == 0) {
            L.totals[0] = g.T * g.k;
            L.totals[1] = s_hoff[g.H];
            L.totals[2] = max(s_wmax[0], s_wmax[1]);
        }
    }

    for (int e = tid; e < g.E; e += kAssignThreads)
        s_base[e] = s_eoff[e] + ws[(int64_t)e * g.G + b];
    __syncthreads();

    const int t0 = b * kChunkTokens;
    const int nt = max(0, min(kChunkTokens, g.T - t0));
    const int64_t p0 = (int64_t)t0 * g.k;
    const uint64_t below = (1ull << lane) - 1ull;

    if (wave == 0) {
        // Stable rows: pairs in (token, j) order, 64 per step.
        const int np = nt * g.k;
        for (int base = 0; base < np; base += kWave) {
            const int p = base + lane;
            const bool act = p < np;
            const int e = act ? idx[p0 + p] : 0;
            uint64_t peers = __ballot(act);
            for (int bit = 0; bit < g.nbits; ++bit) {
                const bool on = (e >> bit) & 1;
                const uint64_t m = __ballot(on);
                peers &= on ? m : ~m;
            }
            if (act) {
                const int before = __popcll(peers & below);
                const int first = s_base[e];
                const int row = first + before;
                L.slot[p0 + p] = row;
                L.row_token[row] = t0 + p / g.k;
                if (before == 0)
                    s_base[e] = first + __popcll(peers);
            }
        }
    } else if (g.relay) {
        // Relay rows: host by host, tokens of this chunk in order (one per lane).
        const bool act = lane < nt;
        const int t = t0 + lane;
        const int32_t *row = idx + (int64_t)t * g.k;
        uint64_t hosts = 0;
        if (act)
            for (int j = 0; j < g.k; ++j)
                hosts |= 1ull << (row[j] / g.epr / g.rph);
        for (int h = 0; h < g.H; ++h) {
            const bool has = (hosts >> h) & 1ull;
            const uint64_t bal = __ballot(has);
            if (!act)
                continue;
            if (!has) {
                L.relay_slot[(int64_t)t * g.H + h] = -1;
                continue;
            }
            const int r = s_hoff[h] + ws[(int64_t)(g.E + g.R + h) * g.G + b] + __popcll(bal & below);
            L.relay_slot[(int64_t)t * g.H + h] = r;
            L.relay_token[r] = t;
            uint32_t mask = 0;
            for (int j = 0; j < g.k; ++j) {
                const int e = row[j];
                const bool here = e / g.epr / g.rph == h;
                L.fanout_expert[(int64_t)r * g.k + j] = here ? e : -1;
                if (here)
                    mask |= 1u << ((e / g.epr) % g.rph);
            }
            L.fanout_rank_mask[r] = mask;
        }
    }

    if (g.relay) {
        // Unused relay rows [relay_rows, capacity) read as empty.
        const int64_t cap = (int64_t)g.T * min(g.k, g.H);
        const int64_t used = s_hoff[g.H];
        const int64_t per = (cap + g.G - 1) / g.G;
        const int64_t beg = max(used, (int64_t)b * per), end = min(cap, (int64_t)(b + 1) * per);
        for (int64_t r = beg + tid; r < end; r += kAssignThreads) {
            L.relay_token[r] = -1;
            L.fanout_rank_mask[r] = 0u;
        }
        for (int64_t i = beg * g.k + tid; i < end * g.k; i += kAssignThreads)
            L.fanout_expert[i] = -1;
    }
}

}  // namespace

hipError_t launch_layout(const Geometry &g, const int32_t *idx, const epx_layout &L,
                         hipStream_t stream)
{
    const int ncol = g.E + g.R + g.H + 1;
    hipLaunchKernelGGL(layout_count_kernel, dim3(g.G), dim3(256), ncol * sizeof(int32_t), stream,
                       idx, g, L.workspace);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int cols_per_block = 256 / kWave;
    hipLaunchKernelGGL(layout_scan_kernel, dim3((ncol + cols_per_block - 1) / cols_per_block),
                       dim3(256), 0, stream, g, L.workspace, L.expert_count, L.rank_tokens,
                       L.host_tokens, L.totals);
    err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const size_t lds = (size_t)(2 * g.E + 1 + g.H + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(layout_assign_kernel, dim3(g.G), dim3(kAssignThreads), lds, stream, idx, g,
                       (const int32_t *)L.workspace, L);
    return hipGetLastError();
}

}  // namespace epx
