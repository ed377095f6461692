// epx_fused.hip -- layout and dispatch in one launch for small batches.
//
// At decode sizes (the digest "Balancing and Beyond: Communication-Centric
// Optimizations in Expert Parallelism" serves at most 128 tokens per GPU,
// sections 1 and 5) the layout is a few thousand (token, expert) pairs, and
// the launch boundary between the layout and the dispatch costs about as
// much as either. So one launch does both, with no workgroup waiting for
// another:
//  * item 0 (dispatched first) computes and writes the layout's global
//    arrays: counts and offsets per expert, rank, group and host, distinct
//    tokens per rank and host, totals and the relay tail;
//  * item 1 + t, one workgroup per column slice, finds the rows of token t
//    without any histogram: the row of pair (t, j) with expert e is the
//    number of pairs whose expert precedes e in row order (e's offset) plus
//    the pairs before (t, j) with expert e. Every thread compares its share
//    of the routing ids with token t's k experts in registers and one block
//    reduction adds the counts up. In relay mode the tokens' host masks are
//    counted by ballots (per host: tokens in all and before t). The slice-0
//    workgroup writes token t's layout entries; every workgroup copies its
//    slice of the token to the token's rows (bf16, or fp8 quantised once
//    into LDS).
// The result equals the layout kernels followed by the dispatch kernel, bit
// for bit, including the error path (an id outside [0, E): totals[3] = their
// number, nothing else written, nothing dispatched).
#include "epx_device.h"

namespace epx {
namespace {

constexpr int kFWaves = 8;
constexpr int kFThreads = kFWaves * kWave;
constexpr int kFBurst = 4;            // 16-byte chunks per lane per burst
constexpr int kFMaxSliceVec = 4096;   // fp8 slice bound (LDS holds slice*8 code bytes)
constexpr int kFPre = 4;              // fp8: chunks loaded per thread before converting
constexpr int kFMaxPairs = 4096;      // T * k bound of the fused path
constexpr int kFIds = kFMaxPairs / kFThreads;   // ids per thread
constexpr int kFMaxK = 16;            // k bound: per-expert counters live in registers
constexpr int kFRed = 2 * kFMaxK + 1; // reduced values: k offsets, k prior counts, bad ids
constexpr int kFTarget = 128;         // workgroups aimed at (slices for small batches)

// Position of expert e in row order (the inverse of expert_at).
__device__ __forceinline__ int row_order(const Geometry &g, int e)
{
    if (g.m == 1)
        return e;
    const int r = g.div_epr.div(e);
    const int i = e - r * g.epr;
    const int grp = i / g.epg;
    return grp * (g.R * g.epg) + r * g.epg + (i - grp * g.epg);
}

// ------------------------------------------------------------ global arrays
// One workgroup: counts per expert (LDS histogram), their scan in row order,
// distinct tokens per rank and per host, then every global array.
__device__ void layout_globals(const int32_t *__restrict__ idx, const Geometry &g,
                               const epx_layout &L, int32_t *lds)
{
    const int P = g.T * g.k;
    int32_t *s_idx = lds;                    // [P]
    int32_t *s_cnt = s_idx + P;              // [E]
    int32_t *s_eoff = s_cnt + g.E;           // [E + 1]
    int32_t *s_rtok = s_eoff + g.E + 1;      // [R]
    __shared__ int32_t s_htok[kMaxHosts];
    __shared__ int32_t s_bad, s_wsum[kFWaves], s_wmax[kFWaves];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;

    if (tid == 0)
        s_bad = 0;
    for (int i = tid; i < g.E; i += kFThreads)
        s_cnt[i] = 0;
    for (int i = tid; i < g.R; i += kFThreads)
        s_rtok[i] = 0;
    for (int i = tid; i < g.H; i += kFThreads)
        s_htok[i] = 0;
    __syncthreads();
    {
        int e[kFIds];
#pragma unroll
        for (int i = 0; i < kFIds; ++i) {
            const int p = i * kFThreads + tid;
            e[i] = p < P ? idx[p] : 0;
        }
        int bad = 0;
#pragma unroll
        for (int i = 0; i < kFIds; ++i) {
            const int p = i * kFThreads + tid;
            if (p >= P)
                break;
            s_idx[p] = e[i];
            if ((unsigned)e[i] >= (unsigned)g.E)
                ++bad;
            else
                atomicAdd(&s_cnt[e[i]], 1);
        }
        if (bad)
            atomicAdd(&s_bad, bad);
    }
    __syncthreads();
    if (s_bad != 0) {   // uniform
        if (tid == 0)
            L.totals[3] = s_bad;
        return;   // out-of-range ids: nothing else is defined
    }

    // distinct ranks and hosts of each token (a pair counts if no earlier
    // pair of its token has the same rank; hosts by their bit mask)
    for (int t = tid; t < g.T; t += kFThreads) {
        const int32_t *ids = s_idx + t * g.k;
        uint64_t hosts = 0;
        for (int j = 0; j < g.k; ++j) {
            const int r = g.div_epr.div(ids[j]);
            bool fresh = true;
            for (int q = 0; q < j; ++q)
                fresh = fresh && g.div_epr.div(ids[q]) != r;
            if (fresh)
                atomicAdd(&s_rtok[r], 1);
            hosts |= 1ull << g.div_rph.div(r);
        }
        while (hosts) {
            atomicAdd(&s_htok[__ffsll((unsigned long long)hosts) - 1], 1);
            hosts &= hosts - 1;
        }
    }

    // expert offsets: exclusive scan of the counts in row order; the maximum
    const int per = (g.E + kFThreads - 1) / kFThreads;
    const int beg = min(tid * per, g.E), end = min(beg + per, g.E);
    int sum = 0, mx = 0;
    for (int q = beg; q < end; ++q) {
        const int c = s_cnt[expert_at(g, q)];
        sum += c;
        mx = max(mx, c);
    }
    const int incl = wave_inclusive_scan(sum);
    if (lane == kWave - 1)
        s_wsum[wave] = incl;
    mx = wave_max(mx);
    if (lane == 0)
        s_wmax[wave] = mx;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w)
        run += s_wsum[w];
    for (int q = beg; q < end; ++q) {
        const int e = expert_at(g, q);
        s_eoff[e] = run;
        run += s_cnt[e];
    }
    if (tid == kFThreads - 1)
        s_eoff[g.E] = run;
    __syncthreads();

    for (int e = tid; e <= g.E; e += kFThreads) {
        L.expert_offset[e] = s_eoff[e];
        if (e < g.E)
            L.expert_count[e] = s_cnt[e];
    }
    write_rank_and_group_offsets(g, s_eoff, L, kFThreads);
    for (int r = tid; r < g.R; r += kFThreads)
        L.rank_tokens[r] = s_rtok[r];
    int used = 0;
    for (int h = 0; h < g.H; ++h)
        used += s_htok[h];
    for (int h = tid; h <= g.H; h += kFThreads) {
        int off = 0;
        for (int q = 0; q < h; ++q)
            off += s_htok[q];
        L.host_offset[h] = off;
        if (h < g.H) {
            L.host_tokens[h] = s_htok[h];
            L.relay_dst_rank[h] = h * g.rph + g.s % g.rph;
        }
    }
    if (tid == 0) {
        int mm = 0;
        for (int w = 0; w < kFWaves; ++w)
            mm = max(mm, s_wmax[w]);
        L.totals[0] = P;
        L.totals[1] = used;
        L.totals[2] = mm;
        L.totals[3] = 0;
    }
    if (g.relay)
        clear_relay_tail(g, used, 0, 1, kFThreads, L);
}

// ------------------------------------------------------------ one token
template <bool FP8>
__device__ void token_rows(int t, const int32_t *__restrict__ idx, const Geometry &g,
                           const epx_layout &L, const u32x4 *__restrict__ x, int nvec, int slice,
                           void *__restrict__ recv, float *__restrict__ scales, int32_t *lds)
{
    __shared__ int32_t s_red[kFWaves][kFRed];
    __shared__ int32_t s_slot[kFMaxK];       // rows of token t's pairs
    __shared__ int32_t s_rrow[kMaxHosts];    // relay row of token t per host, -1 if none
    __shared__ int32_t s_htot[kMaxHosts], s_hbef[kMaxHosts];
    const int P = g.T * g.k;
    const int pt = t * g.k;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;

    if (g.relay && tid < g.H) {
        s_htot[tid] = 0;
        s_hbef[tid] = 0;
    }
    // token t's experts and their positions in row order (uniform)
    int te[kFMaxK], to[kFMaxK];
#pragma unroll
    for (int j = 0; j < kFMaxK; ++j) {
        te[j] = j < g.k ? idx[pt + j] : -1;
        to[j] = j < g.k ? row_order(g, te[j]) : 0;
    }
    // this thread's share of the pairs: for each j, pairs whose expert comes
    // earlier in row order, and pairs before token t with expert te[j]; then
    // the block's sums (wave sums land in lane 63, one LDS row per wave)
    {
        int e[kFIds];
#pragma unroll
        for (int i = 0; i < kFIds; ++i) {
            const int p = i * kFThreads + tid;
            e[i] = p < P ? idx[p] : 0;
        }
        int lt[kFMaxK], pre[kFMaxK], bad = 0;
#pragma unroll
        for (int j = 0; j < kFMaxK; ++j) {
            lt[j] = 0;
            pre[j] = 0;
        }
#pragma unroll
        for (int i = 0; i < kFIds; ++i) {
            const int p = i * kFThreads + tid;
            if (p >= P)
                break;
            const bool ok = (unsigned)e[i] < (unsigned)g.E;
            bad += !ok;
            const int o = ok ? row_order(g, e[i]) : 0;
#pragma unroll
            for (int j = 0; j < kFMaxK; ++j) {
                lt[j] += o < to[j];
                pre[j] += (p < pt) & (e[i] == te[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kFMaxK; ++j) {
            if (j < g.k) {
                const int a = wave_inclusive_scan(lt[j]);
                const int b = wave_inclusive_scan(pre[j]);
                if (lane == kWave - 1) {
                    s_red[wave][j] = a;
                    s_red[wave][kFMaxK + j] = b;
                }
            }
        }
        const int nb = wave_inclusive_scan(bad);
        if (lane == kWave - 1)
            s_red[wave][2 * kFMaxK] = nb;
    }
    __syncthreads();
    int nbad = 0;
    for (int w = 0; w < kFWaves; ++w)
        nbad += s_red[w][2 * kFMaxK];
    if (nbad != 0)   // uniform
        return;      // out-of-range ids: item 0 reports them, nothing is dispatched

    // row of pair (t, j) with expert e: e's offset, the pairs of earlier
    // tokens with e, and the pairs of token t before j with e
    if (tid < g.k) {
        const int j = tid;
        int e_j = te[0];
#pragma unroll
        for (int q = 1; q < kFMaxK; ++q)
            if (q == j)
                e_j = te[q];
        int row = 0;
        for (int w = 0; w < kFWaves; ++w)
            row += s_red[w][j] + s_red[w][kFMaxK + j];
#pragma unroll
        for (int q = 0; q < kFMaxK; ++q)
            row += (q < j) & (te[q] == e_j);
        s_slot[j] = row;
    }
    if (g.relay) {
        // tokens per host, in all and before t: one ballot per host and 64 tokens
        for (int c0 = wave * kWave; c0 < g.T; c0 += kFThreads) {
            const int tt = c0 + lane;
            uint64_t m = 0;
            if (tt < g.T)
                for (int j = 0; j < g.k; ++j)
                    m |= 1ull << g.div_rph.div(g.div_epr.div(idx[tt * g.k + j]));
            const int nbef = t - c0;   // lanes below nbef hold tokens before t
            const uint64_t before = nbef >= kWave ? ~0ull : nbef <= 0 ? 0ull : (1ull << nbef) - 1ull;
            for (int h = 0; h < g.H; ++h) {
                const uint64_t bal = __ballot((m >> h) & 1ull);
                if (lane == 0 && bal != 0ull) {
                    atomicAdd(&s_htot[h], __popcll(bal));
                    if ((bal & before) != 0ull)
                        atomicAdd(&s_hbef[h], __popcll(bal & before));
                }
            }
        }
        __syncthreads();
        if (tid < g.H) {
            uint64_t mine = 0;
#pragma unroll
            for (int j = 0; j < kFMaxK; ++j)
                if (j < g.k)
                    mine |= 1ull << g.div_rph.div(g.div_epr.div(te[j]));
            int off = 0;
            for (int h = 0; h < tid; ++h)
                off += s_htot[h];
            s_rrow[tid] = ((mine >> tid) & 1ull) ? off + s_hbef[tid] : -1;
        }
    }
    __syncthreads();

    // layout entries of token t
    if (blockIdx.y == 0) {
        if (tid < g.k) {
            L.slot[pt + tid] = s_slot[tid];
            if (in_bounds(s_slot[tid], pair_rows(g), g.viol))
                L.row_token[s_slot[tid]] = t;
        }
        if (g.relay && tid < g.H) {
            const int h = tid, r = s_rrow[h];
            L.relay_slot[(int64_t)t * g.H + h] = r;
            if (r >= 0 && in_bounds(r, relay_rows_cap(g), g.viol)) {
                L.relay_token[r] = t;
                uint32_t mask = 0;
                for (int j = 0; j < g.k; ++j) {
                    const int e = idx[pt + j];
                    const int rk = g.div_epr.div(e);
                    const bool here = g.div_rph.div(rk) == h;
                    L.fanout_expert[(int64_t)r * g.k + j] = here ? e : -1;
                    if (here)
                        mask |= 1u << (rk - h * g.rph);
                }
                L.fanout_rank_mask[r] = mask;
            }
        }
    }

    // dispatch of token t's slice to its rows
    const int D = g.relay ? g.H : g.k;
    const int32_t *dst_rows = g.relay ? s_rrow : s_slot;
    const int c_beg = blockIdx.y * slice;
    const int c_end = min(nvec, c_beg + slice);
    const u32x4 *xr = x + (int64_t)t * nvec;
    // Each row goes to wpr waves, each streaming one contiguous part of it
    // (rows round-robin when there are more rows than waves).
    const int wpr = D >= kFWaves ? 1 : kFWaves / D;
    const int part = wave % wpr;
    if (!FP8) {
        const int len = ((c_end - c_beg + wpr - 1) / wpr + kWave - 1) / kWave * kWave;
        const int p_beg = c_beg + part * len, p_end = min(c_end, p_beg + len);
        for (int d = wave / wpr; d < D; d += kFWaves / wpr) {
            const int64_t r = dst_rows[d];
            if (r < 0 || !in_bounds(r, g.cap, g.viol))
                continue;
            u32x4 *dst = (u32x4 *)recv + r * nvec;
            for (int c0 = p_beg + lane; c0 < p_end; c0 += kWave * kFBurst) {
                u32x4 v[kFBurst];
#pragma unroll
                for (int i = 0; i < kFBurst; ++i) {
                    const int c = c0 + i * kWave;
                    if (c < p_end)
                        v[i] = xr[c];
                }
#pragma unroll
                for (int i = 0; i < kFBurst; ++i) {
                    const int c = c0 + i * kWave;
                    if (c < p_end)
                        __builtin_nontemporal_store(v[i], dst + c);
                }
            }
        }
        return;
    }

    // fp8: quantise the slice once into LDS (16 lanes per 128-channel
    // block), then stream codes and scales to every row
    const int n = c_end - c_beg;
    u32x4 *s_codes = (u32x4 *)lds;
    float *s_scale = (float *)(s_codes + (slice >> 1));
    quantize_slice_to_lds<kFThreads, kFPre>(xr, c_beg, n, (u32x2 *)s_codes, s_scale);
    __syncthreads();
    const int nq = n >> 1, nblk = n >> 4, row_vec = nvec >> 1, row_blk = nvec >> 4;
    const int len = ((nq + wpr - 1) / wpr + kWave - 1) / kWave * kWave;
    const int q_beg = part * len, q_end = min(nq, q_beg + len);
    for (int d = wave / wpr; d < D; d += kFWaves / wpr) {
        const int64_t r = dst_rows[d];
        if (r < 0 || !in_bounds(r, g.cap, g.viol))
            continue;
        u32x4 *dst = (u32x4 *)recv + r * row_vec + (c_beg >> 1);
        for (int c0 = q_beg + lane; c0 < q_end; c0 += kWave * kFBurst) {
            u32x4 v[kFBurst];
#pragma unroll
            for (int i = 0; i < kFBurst; ++i) {
                const int c = c0 + i * kWave;
                if (c < q_end)
                    v[i] = s_codes[c];
            }
#pragma unroll
            for (int i = 0; i < kFBurst; ++i) {
                const int c = c0 + i * kWave;
                if (c < q_end)
                    __builtin_nontemporal_store(v[i], dst + c);
            }
        }
        if (part == 0)
            for (int b = lane; b < nblk; b += kWave)
                scales[r * row_blk + (c_beg >> 4) + b] = s_scale[b];
    }
}

template <bool FP8>
__global__ __launch_bounds__(kFThreads) void layout_dispatch_kernel(
    const int32_t *__restrict__ idx, Geometry g, epx_layout L, const u32x4 *__restrict__ x,
    int nvec, int slice, void *__restrict__ recv, float *__restrict__ scales)
{
    extern __shared__ __align__(16) int32_t lds[];
    const int64_t item = item_index();
    if (item > g.T)
        return;
    if (item == 0) {
        if (blockIdx.y == 0)
            layout_globals(idx, g, L, lds);
        return;
    }
    token_rows<FP8>((int)item - 1, idx, g, L, x, nvec, slice, recv, scales, lds);
}

// LDS bytes of the fused path (0 when it does not apply): the larger of the
// global item's ids and counters and, for fp8, one slice of codes and scales.
size_t fused_lds(const Geometry &g, bool fp8, int slice)
{
    if (g.T > 1024 || (int64_t)g.T * g.k > kFMaxPairs || g.k > kFMaxK || g.E > 512)
        return 0;
    const size_t globals = ((size_t)g.T * g.k + 2 * (size_t)g.E + 1 + g.R) * 4;
    const size_t codes = fp8 ? (size_t)slice * 8 + (size_t)(slice / 16) * 4 : 0;
    const size_t bytes = globals > codes ? globals : codes;
    return bytes <= 60 * 1024 ? bytes : 0;
}

}  // namespace

bool launch_layout_dispatch(const Geometry &g, const int32_t *idx, const epx_layout &L,
                            const void *x, int32_t hidden, bool fp8, void *recv, float *scales,
                            hipStream_t stream, hipError_t *err)
{
    const int nvec = hidden / 8;
    // Every workgroup repeats the counting, so the copy is split no finer
    // than needed: one workgroup per token, column slices only below 128
    // tokens. (Measured on MI355X over 4, 8 and 16 waves and 128 to 2048
    // workgroups at decode sizes: 8 waves and 128 were best.)
    const int slice = fp8 ? slice_width(g.T, nvec, 16, kFMaxSliceVec, kFTarget)
                          : slice_width(g.T, nvec, kWave, 1 << 30, kFTarget);
    const size_t lds = g.T > 0 ? fused_lds(g, fp8, slice) : 0;
    if (lds == 0)
        return false;
    const dim3 grid = item_grid((int64_t)g.T + 1, (nvec + slice - 1) / slice);
    if (fp8)
        launch(layout_dispatch_kernel<true>, grid, dim3(kFThreads), lds, stream, idx, g,
                           L, (const u32x4 *)x, nvec, slice, recv, scales);
    else
        launch(layout_dispatch_kernel<false>, grid, dim3(kFThreads), lds, stream, idx,
                           g, L, (const u32x4 *)x, nvec, slice, recv, scales);
    *err = hipGetLastError();
    return true;
}

}  // namespace epx
