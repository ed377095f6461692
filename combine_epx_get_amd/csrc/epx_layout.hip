// epx_layout.hip -- routing -> layout on gfx950.
//
// Computes, for one source rank, the counts per expert / rank / host, their
// exclusive prefixes and the destination row of every (token, expert) pair
// and of every (token, host) relay copy. The copies per expert and per host
// are the quantities the digest "Balancing and Beyond: Communication-Centric
// Optimizations in Expert Parallelism" reasons about (section 2: the busiest
// expert sets the time; section 3.2: a single cross-host copy to each remote
// host); the per-rank token counts are those of the DeepEP issue
// "[GH-ISSUE #250] Profiling when rank unbalance".
//
// Row order: per-expert rows by (expert, token, j) -- with expert groups by
// (group, expert, token, j); relay rows by (host, token). Positions come
// from ordered wave walks, never from atomic order: a wave takes 64 pairs at
// a time in (t, j) order, groups equal expert ids with ceil(log2 E) ballots
// (a wave-level multisplit) and gives each lane base + popcount(peers below
// it); the group's first lane then advances the base. Counting may use LDS
// atomics, because counts do not depend on order.
//
// Three shapes, no global atomics and no zero-filled buffers:
//   small batches (<= 4096 pairs): one workgroup does everything in LDS;
//   up to 16 workgroups of up to 32 tokens (k <= 16; 1024 / k tokens
//     above): count, then assign (each assign workgroup sums the count
//     columns itself);
//   more: count, a column scan (one wave per counter), assign.
// Every per-pair rank and host is computed once, with division constants
// prepared on the host, and staged in LDS with the chunk's ids.
#include "epx_device.h"

namespace epx {
namespace {

// Stage pairs [0, np) of a chunk: ids, their ranks and hosts (-1 for a bad id).
__device__ __forceinline__ void stage_pairs(const int32_t *__restrict__ idx, int64_t p0, int np,
                                            const Geometry &g, int32_t *s_idx, int32_t *s_rk,
                                            int32_t *s_hk, int nthreads)
{
    for (int p = threadIdx.x; p < np; p += nthreads) {
        const int e = idx[p0 + p];
        const bool ok = (unsigned)e < (unsigned)g.E;
        const int r = ok ? g.div_epr.div(e) : -1;
        s_idx[p] = e;
        s_rk[p] = r;
        s_hk[p] = ok ? g.div_rph.div(r) : -1;
    }
}

constexpr int kRegK = 16;   // top-k up to which a token's pairs are handled in registers

// For pair p of a staged chunk (token-major, k per token): count the expert,
// and the pair's rank / host when no earlier pair of the same token has it.
__device__ __forceinline__ void count_pair(int p, const Geometry &g, const int32_t *s_idx,
                                           const int32_t *s_rk, const int32_t *s_hk,
                                           int32_t *s_hist, int32_t *s_rtok, int32_t *s_htok,
                                           int32_t *s_bad)
{
    const int r = s_rk[p];
    if (r < 0) {
        atomicAdd(s_bad, 1);
        return;
    }
    atomicAdd(&s_hist[s_idx[p]], 1);
    const int first = g.div_k.div(p) * g.k;   // first pair of the token
    const int jp = p - first;
    const int h = s_hk[p];
    bool new_rank = true, new_host = true;
    if (g.k <= kRegK) {
        // independent loads, issued together
#pragma unroll
        for (int q = 0; q < kRegK - 1; ++q)
            if (q < jp) {
                new_rank = new_rank && s_rk[first + q] != r;
                new_host = new_host && s_hk[first + q] != h;
            }
    } else {
        for (int q = first; q < p; ++q) {
            new_rank = new_rank && s_rk[q] != r;
            new_host = new_host && s_hk[q] != h;
        }
    }
    if (new_rank)
        atomicAdd(&s_rtok[r], 1);
    if (new_host)
        atomicAdd(&s_htok[h], 1);
}

// Relay rows of up to 64 consecutive tokens (one per lane: token t, its
// pairs at s_idx/s_rk/s_hk + i*k and its host mask at s_hmask[i] for the
// lane's local index i) for host h: rows in token order from `base`; the
// fan-out row is written with 16-byte stores when it is aligned. Every lane
// of the wave must call it (ballot).
__device__ __forceinline__ void relay_item(bool act, int t, int i, int h, const Geometry &g,
                                           const int32_t *s_idx, const int32_t *s_hk,
                                           const int32_t *s_rk, const uint64_t *s_hmask,
                                           int base, const epx_layout &L)
{
    const int lane = lane_id();
    const bool has = act && ((s_hmask[act ? i : 0] >> h) & 1ull);
    const uint64_t bal = __ballot(has);
    if (!act)
        return;
    if (!has) {
        L.relay_slot[(int64_t)t * g.H + h] = -1;
        return;
    }
    const int r = base + __popcll(bal & ((1ull << lane) - 1ull));
    L.relay_slot[(int64_t)t * g.H + h] = r;
    if (!in_bounds(r, relay_rows_cap(g), g.viol))
        return;   // checked builds only
    L.relay_token[r] = t;
    const int32_t *ids = s_idx + i * g.k, *hks = s_hk + i * g.k, *rks = s_rk + i * g.k;
    int32_t *fan = L.fanout_expert + (int64_t)r * g.k;
    uint32_t mask = 0;
    if ((g.k & 3) == 0 && ((uintptr_t)L.fanout_expert & 15) == 0) {
        for (int j = 0; j < g.k; j += 4) {
            int4 v;
            v.x = hks[j] == h ? ids[j] : -1;
            v.y = hks[j + 1] == h ? ids[j + 1] : -1;
            v.z = hks[j + 2] == h ? ids[j + 2] : -1;
            v.w = hks[j + 3] == h ? ids[j + 3] : -1;
            *(int4 *)(fan + j) = v;
        }
    } else {
        for (int j = 0; j < g.k; ++j)
            fan[j] = hks[j] == h ? ids[j] : -1;
    }
    for (int j = 0; j < g.k; ++j)
        if (hks[j] == h)
            mask |= 1u << (rks[j] - h * g.rph);
    L.fanout_rank_mask[r] = mask;
}

// Host mask of each of the np / k tokens staged at s_hk (threads [0, nthreads)).
__device__ __forceinline__ void token_host_masks(int ntok, const Geometry &g, const int32_t *s_hk,
                                                 uint64_t *s_hmask, int nthreads)
{
    for (int i = threadIdx.x; i < ntok; i += nthreads) {
        uint64_t hosts = 0;
        for (int j = 0; j < g.k; ++j) {
            const int h = s_hk[i * g.k + j];
            if (h >= 0)
                hosts |= 1ull << h;
        }
        s_hmask[i] = hosts;
    }
}

// ---------------------------------------------------------------- count
// Columns of the per-workgroup counts: [0, E) experts, [E, E+R) ranks,
// [E+R, E+R+H) hosts, E+R+H bad ids; column c of workgroup b at ws[c*Gs + b].
constexpr int kCountThreads = 256;

__global__ __launch_bounds__(kCountThreads) void layout_count_kernel(
    const int32_t *__restrict__ idx, Geometry g, int32_t *__restrict__ ws)
{
    extern __shared__ int32_t lds[];
    const int ncol = g.E + g.R + g.H + 1;
    int32_t *s_hist = lds;
    int32_t *s_rtok = lds + g.E;
    int32_t *s_htok = s_rtok + g.R;
    int32_t *s_bad = s_htok + g.H;
    int32_t *s_idx = lds + ncol;
    int32_t *s_rk = s_idx + g.ct * g.k;
    int32_t *s_hk = s_rk + g.ct * g.k;

    const int b = blockIdx.x;
    const int t0 = b * g.ct;
    const int nt = max(0, min(g.ct, g.T - t0));
    const int np = nt * g.k;
    for (int i = threadIdx.x; i < ncol; i += kCountThreads)
        lds[i] = 0;
    stage_pairs(idx, (int64_t)t0 * g.k, np, g, s_idx, s_rk, s_hk, kCountThreads);
    __syncthreads();
    for (int p = threadIdx.x; p < np; p += kCountThreads)
        count_pair(p, g, s_idx, s_rk, s_hk, s_hist, s_rtok, s_htok, s_bad);
    __syncthreads();
    for (int c = threadIdx.x; c < ncol; c += kCountThreads)
        ws[(int64_t)c * g.Gs + b] = lds[c];
}

// ---------------------------------------------------------------- scan
// One wave per column: exclusive scan over the G workgroups in place; the
// column total goes to ws_tot[c] (ws_tot = ws + ncol*Gs).
__global__ __launch_bounds__(256) void layout_scan_kernel(Geometry g, int32_t *__restrict__ ws)
{
    const int ncol = g.E + g.R + g.H + 1;
    const int col = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (col >= ncol)
        return;
    const int lane = lane_id();
    int32_t *c = ws + (int64_t)col * g.Gs;
    int carry = 0;
    for (int base = 0; base < g.G; base += kWave) {
        const int i = base + lane;
        const int v = (i < g.G) ? c[i] : 0;
        const int incl = wave_inclusive_scan(v);
        if (i < g.G)
            c[i] = carry + incl - v;
        carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0)
        ws[(int64_t)ncol * g.Gs + col] = carry;
}

// ---------------------------------------------------------------- assign
constexpr int kAssignThreads = 512;
// Up to this many workgroups the assign kernel sums the count columns itself
// (no scan launch); measured on MI355X, 64 workgroups summing 64-entry
// columns cost more than the scan launch they save.
constexpr int kSumsMaxG = 16;

// Exclusive scan of the expert counts src[0, E) (LDS, by expert id) in the
// row order of expert_at into dst[0, E] (LDS, by expert id), dst[E] = total.
template <int NT>
__device__ void block_exclusive_scan(const Geometry &g, const int32_t *src, int32_t *dst,
                                     int32_t *s_wsum)
{
    const int tid = threadIdx.x, n = g.E, wave = tid / kWave;
    const int per = (n + NT - 1) / NT;
    const int beg = min(tid * per, n), end = min(beg + per, n);
    int sum = 0;
    for (int i = beg; i < end; ++i)
        sum += src[expert_at(g, i)];
    const int incl = wave_inclusive_scan(sum);
    if (lane_id() == kWave - 1)
        s_wsum[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w)
        run += s_wsum[w];
    for (int i = beg; i < end; ++i) {
        const int e = expert_at(g, i);
        const int v = src[e];
        dst[e] = run;
        run += v;
    }
    if (tid == NT - 1)
        dst[n] = run;
}

// SUMS: this workgroup sums the raw count columns itself (total and the
// prefix over workgroups before it); otherwise the scan kernel has left the
// prefix in place and the totals after the columns.
//
// The chunk's pairs are split over the first nww waves in (t, j) order
// (nww = 8, fewer when the per-wave count table would not fit in LDS); each
// of them counts its pairs per expert, a scan over these waves gives each its
// first row per expert, and they then assign their rows at once. Relay rows
// are assigned host by host, one host per wave.
template <bool SUMS, int NT>
__device__ void assign_chunk(const int32_t *__restrict__ idx, const Geometry &g,
                             const int32_t *__restrict__ ws, const epx_layout &L, int nww, int b,
                             int32_t *lds)
{
    const int ncol = g.E + g.R + g.H + 1;
    const int kc = g.ct * g.k;
    const int cs = g.E + 1;                // padded per-wave stride (distinct LDS banks)
    uint64_t *s_hmask = (uint64_t *)lds;   // [ct] hosts each token touches
    int32_t *s_tot = lds + 2 * g.ct;       // [ncol] column totals
    int32_t *s_pre = s_tot + ncol;         // [ncol] this workgroup's prefix per column
    int32_t *s_eoff = s_pre + ncol;        // [E + 1]
    int32_t *s_hoff = s_eoff + g.E + 1;    // [H + 1]
    int32_t *s_idx = s_hoff + g.H + 1;     // [kc] ids, ranks, hosts of the chunk
    int32_t *s_rk = s_idx + kc;
    int32_t *s_hk = s_rk + kc;
    int32_t *s_wc = s_hk + kc;             // [nww][cs] per-wave counts, then wave bases
    __shared__ int32_t s_wsum[(NT / kWave)];
    __shared__ int32_t s_wmax[(NT / kWave)];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int t0 = b * g.ct;
    const int nt = max(0, min(g.ct, g.T - t0));
    const int np = nt * g.k;
    const int64_t p0 = (int64_t)t0 * g.k;
    const uint64_t below = (1ull << lane) - 1ull;

    stage_pairs(idx, p0, np, g, s_idx, s_rk, s_hk, NT);
    for (int i = tid; i < nww * cs; i += NT)
        s_wc[i] = 0;
    if (SUMS) {
        // each thread sums whole columns as 16-byte vectors (Gs % 4 == 0;
        // entries [G, Gs) are padding, never written)
        for (int c = tid; c < ncol; c += NT) {
            const int4 *col = (const int4 *)(ws + (int64_t)c * g.Gs);
            int tot = 0, pre = 0;
            for (int i = 0; 4 * i < g.Gs; ++i) {
                const int4 v = col[i];
                const int i0 = 4 * i;
                tot += (i0 < g.G ? v.x : 0) + (i0 + 1 < g.G ? v.y : 0) +
                       (i0 + 2 < g.G ? v.z : 0) + (i0 + 3 < g.G ? v.w : 0);
                pre += (i0 < b ? v.x : 0) + (i0 + 1 < b ? v.y : 0) + (i0 + 2 < b ? v.z : 0) +
                       (i0 + 3 < b ? v.w : 0);
            }
            s_tot[c] = tot;
            s_pre[c] = pre;
        }
    } else {
        for (int c = tid; c < ncol; c += NT) {
            s_tot[c] = ws[(int64_t)ncol * g.Gs + c];
            s_pre[c] = ws[(int64_t)c * g.Gs + b];
        }
    }
    __syncthreads();
    const int bad = s_tot[ncol - 1];
    if (bad != 0) {
        if (b == 0 && tid == 0)
            L.totals[3] = bad;
        return;   // out-of-range ids: nothing else is defined
    }

    // per-wave counts per expert (the first lane of each group adds its size)
    const int per_wave = (np + nww * kWave - 1) / (nww * kWave) * kWave;
    const int pw0 = wave < nww ? wave * per_wave : np;
    const int pw1 = wave < nww ? min(np, pw0 + per_wave) : np;
    for (int base = pw0; base < pw1; base += kWave) {
        const int p = base + lane;
        const bool act = p < pw1;
        const int e = act ? s_idx[p] : 0;
        const uint64_t peers = match_peers(act, e, g.nbits);
        if (act && (peers & below) == 0ull)
            s_wc[wave * cs + e] += __popcll(peers);
    }
    if (g.relay)
        token_host_masks(nt, g, s_hk, s_hmask, NT);
    block_exclusive_scan<NT>(g, s_tot, s_eoff, s_wsum);   // synchronises the workgroup
    if (wave == 0) {
        const int v = lane < g.H ? s_tot[g.E + g.R + lane] : 0;
        const int incl = wave_inclusive_scan(v);
        if (lane < g.H)
            s_hoff[lane] = incl - v;
        if (lane == kWave - 1)
            s_hoff[g.H] = incl;
    }
    // each wave's first row per expert: the expert's offset, the rows of
    // earlier workgroups, then those of earlier waves
    for (int e = tid; e < g.E; e += NT) {
        int run = s_pre[e];
        for (int w = 0; w < nww; ++w) {
            const int v = s_wc[w * cs + e];
            s_wc[w * cs + e] = run;
            run += v;
        }
    }
    __syncthreads();

    if (b == 0) {
        for (int e = tid; e <= g.E; e += NT) {
            L.expert_offset[e] = s_eoff[e];
            if (e < g.E)
                L.expert_count[e] = s_tot[e];
        }
        write_rank_and_group_offsets(g, s_eoff, L, NT);
        for (int r = tid; r < g.R; r += NT)
            L.rank_tokens[r] = s_tot[g.E + r];
        for (int h = tid; h <= g.H; h += NT) {
            L.host_offset[h] = s_hoff[h];
            if (h < g.H) {
                L.host_tokens[h] = s_tot[g.E + g.R + h];
                L.relay_dst_rank[h] = h * g.rph + g.s % g.rph;
            }
        }
        int m = 0;
        for (int e = tid; e < g.E; e += NT)
            m = max(m, s_tot[e]);
        m = wave_max(m);
        if (lane == 0)
            s_wmax[wave] = m;
        __syncthreads();
        if (tid == 0) {
            int mm = 0;
            for (int w = 0; w < (NT / kWave); ++w)
                mm = max(mm, s_wmax[w]);
            L.totals[0] = g.T * g.k;
            L.totals[1] = s_hoff[g.H];
            L.totals[2] = mm;
            L.totals[3] = 0;
        }
    }

    // rows per expert in (t, j) order
    for (int base = pw0; base < pw1; base += kWave) {
        const int p = base + lane;
        const bool act = p < pw1;
        const int e = act ? s_idx[p] : 0;
        const uint64_t peers = match_peers(act, e, g.nbits);
        if (act) {
            const int before = __popcll(peers & below);
            const int rel = s_wc[wave * cs + e];
            const int row = s_eoff[e] + rel + before;
            L.slot[p0 + p] = row;
            if (in_bounds(row, pair_rows(g), g.viol))
                L.row_token[row] = t0 + g.div_k.div(p);
            if (before == 0)
                s_wc[wave * cs + e] = rel + __popcll(peers);
        }
    }
    if (!g.relay)
        return;
    for (int h = wave; h < g.H; h += (NT / kWave))
        relay_item(lane < nt, t0 + lane, lane, h, g, s_idx, s_hk, s_rk, s_hmask,
                   s_hoff[h] + s_pre[g.E + g.R + h], L);
    clear_relay_tail(g, s_hoff[g.H], b, g.G, NT, L);
}

template <bool SUMS>
__global__ __launch_bounds__(kAssignThreads) void layout_assign_kernel(
    const int32_t *__restrict__ idx, Geometry g, const int32_t *__restrict__ ws, epx_layout L,
    int nww)
{
    extern __shared__ __align__(16) int32_t lds[];
    assign_chunk<SUMS, kAssignThreads>(idx, g, ws, L, nww, blockIdx.x, lds);
}

// ---------------------------------------------------------------- assign + dispatch
// Batches past the single-launch decode path (k <= 16, one expert group;
// bf16, or fp8 in relay mode):
// after the count and scan launches, one launch both assigns the rows
// (items [0, G): the chunk workgroups of the assign kernel, unchanged) and
// copies the tokens (item G + t, one per column slice), so that no copy
// waits for an assign launch to end. A token workgroup reads nothing the
// assign workgroups write; its rows equal theirs bit for bit:
//  * per-expert: the row of pair (t, j) with expert e is the rows of the
//    experts before e (an exclusive scan of the column totals), plus the
//    rows of e in earlier chunks (the scan's prefix for t's chunk), plus the
//    pairs of t's chunk before (t, j) with expert e (ballots);
//  * relay: the row of (t, host h) is the relay rows of the hosts before h,
//    plus those of h in earlier chunks, plus the tokens of t's chunk before
//    t that touch h (ballots over their host masks); -1 where t has no
//    expert on h.
// The copy is the dispatch kernel's: bf16 rows streamed 16 KiB per wave, or
// the slice quantised once into LDS (E4M3 codes, per-block scales) and then
// streamed to each row.
constexpr int kFusedThreads = 256;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedBurst = 16;     // bf16: 16-byte chunks per lane per burst
constexpr int kFusedBurstFp8 = 4;   // fp8: code vectors per lane per burst (from LDS)
constexpr int kFusedPre = 4;        // fp8: chunks loaded per thread before converting
constexpr int kFusedMaxK = 16;

template <bool FP8>
__global__ __launch_bounds__(kFusedThreads) void assign_copy_kernel(
    const int32_t *__restrict__ idx, Geometry g, const int32_t *__restrict__ ws, epx_layout L,
    int nww, const u32x4 *__restrict__ x, int nvec, int slice, void *__restrict__ recv,
    float *__restrict__ scales)
{
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int32_t s_e[kFusedMaxK];
    __shared__ int32_t s_pre[kFusedMaxK];
    __shared__ int32_t s_cnt[kFusedMaxK];
    __shared__ int32_t s_rows[kMaxHosts];   // k <= 16 expert rows or H <= 64 relay rows
    __shared__ int32_t s_wsum[kFusedWaves];
    const int64_t item = item_index();
    if (item < g.G) {
        if (blockIdx.y == 0)
            assign_chunk<false, kFusedThreads>(idx, g, ws, L, nww, (int)item, lds);
        return;
    }
    const int64_t t = item - g.G;
    if (t >= g.T)
        return;
    const int ncol = g.E + g.R + g.H + 1;
    const int32_t *tot = ws + (int64_t)ncol * g.Gs;   // column totals
    if (tot[ncol - 1] != 0)
        return;   // out-of-range ids: the assign workgroups report them, nothing moves
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int c = (int)(t / g.ct);
    const int D = g.relay ? g.H : g.k;
    if (!g.relay) {
        int32_t *s_tot = lds;           // [E] rows per expert
        int32_t *s_eoff = lds + g.E;    // [E + 1] first row per expert
        for (int e = tid; e < g.E; e += kFusedThreads)
            s_tot[e] = tot[e];
        if (tid < g.k) {
            const int e = idx[t * g.k + tid];
            s_e[tid] = e;
            s_pre[tid] = ws[(int64_t)e * g.Gs + c];
            s_cnt[tid] = 0;
        }
        __syncthreads();
        block_exclusive_scan<kFusedThreads>(g, s_tot, s_eoff, s_wsum);
        int ej[kFusedMaxK];
#pragma unroll
        for (int j = 0; j < kFusedMaxK; ++j)
            ej[j] = j < g.k ? s_e[j] : -1;
        // pairs of the chunk before (t, j) with expert e_j
        const int64_t p_beg = (int64_t)c * g.ct * g.k, p_t = t * g.k;
        for (int64_t base = p_beg; base < p_t + g.k - 1; base += kFusedThreads) {
            const int64_t p = base + tid;
            const int id = p < p_t + g.k - 1 ? idx[p] : -1;
#pragma unroll
            for (int j = 0; j < kFusedMaxK; ++j) {
                if (j < g.k) {   // uniform: every lane takes part in the ballot
                    const uint64_t bal = __ballot(p < p_t + j && id == ej[j]);
                    if (lane == 0 && bal != 0ull)
                        atomicAdd(&s_cnt[j], (int)__popcll(bal));
                }
            }
        }
        __syncthreads();
        if (tid < g.k)
            s_rows[tid] = s_eoff[s_e[tid]] + s_pre[tid] + s_cnt[tid];
    } else if (wave == 0) {
        // lane i < nb holds the host mask of the chunk's token t0 + i, lane
        // nb that of t itself (a chunk holds at most 32 tokens for k <= 16)
        const int64_t t0 = (int64_t)c * g.ct;
        const int nb = (int)(t - t0);
        uint64_t mask = 0;
        if (lane <= nb)
            for (int j = 0; j < g.k; ++j) {
                const int e = idx[(t0 + lane) * g.k + j];
                mask |= 1ull << g.div_rph.div(g.div_epr.div(e));
            }
        const uint32_t mlo = __shfl((uint32_t)mask, nb), mhi = __shfl((uint32_t)(mask >> 32), nb);
        const uint64_t mine = ((uint64_t)mhi << 32) | mlo;
        const int hv = lane < g.H ? tot[g.E + g.R + lane] : 0;
        const int hoff = wave_inclusive_scan(hv) - hv;   // relay rows of the hosts before lane's
        const int pre = lane < g.H ? ws[(int64_t)(g.E + g.R + lane) * g.Gs + c] : 0;
        int before = 0;
        for (int h = 0; h < g.H; ++h) {
            const uint64_t bal = __ballot(lane < nb && ((mask >> h) & 1ull));
            if (lane == h)
                before = (int)__popcll(bal);
        }
        if (lane < g.H)
            s_rows[lane] = ((mine >> lane) & 1ull) ? hoff + pre + before : -1;
    }
    __syncthreads();

    const int c_beg = blockIdx.y * slice;
    const int c_end = min(nvec, c_beg + slice);
    const u32x4 *xr = x + t * nvec;
    if (!FP8) {
        // a wave streams whole rows, 16 KiB per burst
        for (int d = wave; d < D; d += kFusedWaves) {
            const int r = s_rows[d];
            if (r < 0 || !in_bounds(r, g.cap, g.viol))
                continue;
            u32x4 *dst = (u32x4 *)recv + (int64_t)r * nvec;
            for (int c0 = c_beg + lane; c0 < c_end; c0 += kWave * kFusedBurst) {
                u32x4 v[kFusedBurst];
#pragma unroll
                for (int i = 0; i < kFusedBurst; ++i) {
                    const int cc = c0 + i * kWave;
                    if (cc < c_end)
                        v[i] = xr[cc];
                }
#pragma unroll
                for (int i = 0; i < kFusedBurst; ++i) {
                    const int cc = c0 + i * kWave;
                    if (cc < c_end)
                        __builtin_nontemporal_store(v[i], dst + cc);
                }
            }
        }
        return;
    }
    // fp8: the slice's codes and scales in LDS past the scan's arrays
    const int n = c_end - c_beg;
    u32x4 *s_codes = (u32x4 *)(lds + ((2 * g.E + 1 + 3) & ~3));
    float *s_scale = (float *)(s_codes + (slice >> 1));
    quantize_slice_to_lds<kFusedThreads, kFusedPre>(xr, c_beg, n, (u32x2 *)s_codes, s_scale);
    __syncthreads();
    const int nq = n >> 1, nblk = n >> 4, row_vec = nvec >> 1, row_blk = nvec >> 4;
    for (int d = wave; d < D; d += kFusedWaves) {
        const int r = s_rows[d];
        if (r < 0 || !in_bounds(r, g.cap, g.viol))
            continue;
        u32x4 *dst = (u32x4 *)recv + (int64_t)r * row_vec + (c_beg >> 1);
        for (int c0 = lane; c0 < nq; c0 += kWave * kFusedBurstFp8) {
            u32x4 v[kFusedBurstFp8];
#pragma unroll
            for (int i = 0; i < kFusedBurstFp8; ++i) {
                const int cc = c0 + i * kWave;
                if (cc < nq)
                    v[i] = s_codes[cc];
            }
#pragma unroll
            for (int i = 0; i < kFusedBurstFp8; ++i) {
                const int cc = c0 + i * kWave;
                if (cc < nq)
                    __builtin_nontemporal_store(v[i], dst + cc);
            }
        }
        for (int bk = lane; bk < nblk; bk += kWave)
            scales[(int64_t)r * row_blk + (c_beg >> 4) + bk] = s_scale[bk];
    }
}

// ---------------------------------------------------------------- single workgroup
// Small batches (decode): the whole layout in one workgroup of 16 waves, in
// LDS, in one launch. Wave w owns a contiguous range of pairs (in (t, j)
// order) and, in relay mode, tokens [64w, 64w + 64). Per-wave counts per
// expert (and per host) are scanned over the waves, which gives every wave
// the base of its first row for each expert; the ordered walk then assigns
// rows exactly as the multi-workgroup path does.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;
static_assert(kSmallWaves == 16, "per-wave columns are scanned by 16-lane groups");

__global__ __launch_bounds__(kSmallThreads) void layout_small_kernel(
    const int32_t *__restrict__ idx, Geometry g, epx_layout L)
{
    extern __shared__ __align__(16) int32_t lds[];
    const int P = g.T * g.k;
    uint64_t *s_hmask = (uint64_t *)lds;               // [T] hosts each token touches
    int32_t *s_idx = lds + 2 * g.T;                    // [P] ids, ranks, hosts
    int32_t *s_rk = s_idx + P;
    int32_t *s_hk = s_rk + P;
    // per-wave columns are padded to an odd stride so that the 16 cells of a
    // column sit in 16 different LDS banks
    const int cs = g.E + 1, hs = g.H + 1;
    int32_t *s_cnt = s_hk + P;                         // [waves][cs] counts, then wave bases
    int32_t *s_eoff = s_cnt + kSmallWaves * cs;        // [E + 1]
    int32_t *s_rtok = s_eoff + g.E + 1;                // [R]
    int32_t *s_htok = s_rtok + g.R;                    // [H]
    int32_t *s_hcnt = s_htok + g.H;                    // [waves][hs] counts, then wave bases
    int32_t *s_hoff = s_hcnt + kSmallWaves * hs;       // [H + 1]
    __shared__ int32_t s_bad;
    __shared__ int32_t s_wsum[kSmallWaves];
    __shared__ int32_t s_wmax[kSmallWaves];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const uint64_t below = (1ull << lane) - 1ull;

    stage_pairs(idx, 0, P, g, s_idx, s_rk, s_hk, kSmallThreads);
    for (int i = tid; i < kSmallWaves * cs; i += kSmallThreads)
        s_cnt[i] = 0;
    for (int i = tid; i < g.R; i += kSmallThreads)
        s_rtok[i] = 0;
    for (int i = tid; i < g.H; i += kSmallThreads)
        s_htok[i] = 0;
    if (tid == 0)
        s_bad = 0;
    __syncthreads();

    // per-wave counts per expert (the first lane of each group adds its size)
    const int per_wave = (P + kSmallThreads - 1) / kSmallThreads * kWave;
    const int pw0 = wave * per_wave, pw1 = min(P, pw0 + per_wave);
    for (int base = pw0; base < pw1; base += kWave) {
        const int p = base + lane;
        const bool act = p < pw1;
        const int e = act ? s_idx[p] : 0;
        const bool ok = act && s_rk[p] >= 0;
        const uint64_t peers = match_peers(ok, e, g.nbits);
        if (ok && (peers & below) == 0ull)
            s_cnt[wave * cs + e] += __popcll(peers);
    }
    // bad ids, distinct ranks and hosts per token
    for (int p = tid; p < P; p += kSmallThreads) {
        const int r = s_rk[p];
        if (r < 0) {
            atomicAdd(&s_bad, 1);
            continue;
        }
        const int first = g.div_k.div(p) * g.k;
        const int jp = p - first;
        const int h = s_hk[p];
        bool new_rank = true, new_host = true;
        if (g.k <= kRegK) {
#pragma unroll
            for (int q = 0; q < kRegK - 1; ++q)
                if (q < jp) {
                    new_rank = new_rank && s_rk[first + q] != r;
                    new_host = new_host && s_hk[first + q] != h;
                }
        } else {
            for (int q = first; q < p; ++q) {
                new_rank = new_rank && s_rk[q] != r;
                new_host = new_host && s_hk[q] != h;
            }
        }
        if (new_rank)
            atomicAdd(&s_rtok[r], 1);
        if (new_host)
            atomicAdd(&s_htok[h], 1);
    }
    // hosts of each token, and per-wave relay counts: tokens of wave w touching host h
    uint64_t hosts = 0;
    if (tid < g.T) {
        for (int j = 0; j < g.k; ++j) {
            const int h = s_hk[tid * g.k + j];
            if (h >= 0)
                hosts |= 1ull << h;
        }
        s_hmask[tid] = hosts;
    }
    for (int h = 0; h < g.H; ++h) {
        const uint64_t bal = __ballot((hosts >> h) & 1ull);
        if (lane == 0)
            s_hcnt[wave * hs + h] = __popcll(bal);
    }
    __syncthreads();
    if (s_bad != 0) {
        if (tid == 0)
            L.totals[3] = s_bad;
        return;   // out-of-range ids: nothing else is defined
    }

    // per column (expert, then host) an exclusive scan over the 16 waves by a
    // 16-lane group; the expert totals land in s_eoff
    for (int c = tid / kSmallWaves; c < g.E + g.H; c += kSmallThreads / kSmallWaves) {
        const int w = tid % kSmallWaves;
        int32_t *cell = c < g.E ? s_cnt + w * cs + c : s_hcnt + w * hs + (c - g.E);
        const int v = *cell;
        const int incl = row_inclusive_scan(v);   // the 16-lane group is one DPP row
        *cell = incl - v;
        if (w == kSmallWaves - 1 && c < g.E)
            s_eoff[c] = incl;
    }
    __syncthreads();
    const int e_q = tid < g.E ? expert_at(g, tid) : 0;   // expert at scan position tid
    const int cnt_e = tid < g.E ? s_eoff[e_q] : 0;
    const int incl = wave_inclusive_scan(cnt_e);
    if (lane == kWave - 1)
        s_wsum[wave] = incl;
    const int m = wave_max(cnt_e);
    if (lane == 0)
        s_wmax[wave] = m;
    __syncthreads();
    if (wave == 0) {
        const int v = lane < kSmallWaves ? s_wsum[lane] : 0;
        const int vi = wave_inclusive_scan(v);
        const int mm = wave_max(lane < kSmallWaves ? s_wmax[lane] : 0);
        if (lane < kSmallWaves)
            s_wsum[lane] = vi - v;
        if (lane == 0)
            s_wmax[0] = mm;
    } else if (wave == 1) {
        const int v = lane < g.H ? s_htok[lane] : 0;
        const int vi = wave_inclusive_scan(v);
        if (lane < g.H)
            s_hoff[lane] = vi - v;
        if (lane == kWave - 1)
            s_hoff[g.H] = vi;
    }
    __syncthreads();
    if (tid < g.E) {
        const int ex = incl - cnt_e + s_wsum[wave];
        s_eoff[e_q] = ex;
        if (tid == g.E - 1)
            s_eoff[g.E] = ex + cnt_e;
    }
    __syncthreads();

    // global counts and offsets
    for (int e = tid; e <= g.E; e += kSmallThreads)
        L.expert_offset[e] = s_eoff[e];
    if (tid < g.E)
        L.expert_count[e_q] = cnt_e;
    write_rank_and_group_offsets(g, s_eoff, L, kSmallThreads);
    for (int r = tid; r < g.R; r += kSmallThreads)
        L.rank_tokens[r] = s_rtok[r];
    for (int h = tid; h <= g.H; h += kSmallThreads) {
        L.host_offset[h] = s_hoff[h];
        if (h < g.H) {
            L.host_tokens[h] = s_htok[h];
            L.relay_dst_rank[h] = h * g.rph + g.s % g.rph;
        }
    }
    if (tid == 0) {
        L.totals[0] = P;
        L.totals[1] = s_hoff[g.H];
        L.totals[2] = s_wmax[0];
        L.totals[3] = 0;
    }

    // ordered walk: rows of each expert in (t, j) order, from the expert's
    // offset plus the rows of earlier waves
    for (int base = pw0; base < pw1; base += kWave) {
        const int p = base + lane;
        const bool act = p < pw1;
        const int e = act ? s_idx[p] : 0;
        const uint64_t peers = match_peers(act, e, g.nbits);
        if (act) {
            const int before = __popcll(peers & below);
            const int rel = s_cnt[wave * cs + e];
            const int row = s_eoff[e] + rel + before;
            L.slot[p] = row;
            if (in_bounds(row, pair_rows(g), g.viol))
                L.row_token[row] = g.div_k.div(p);
            if (before == 0)
                s_cnt[wave * cs + e] = rel + __popcll(peers);
        }
    }
    if (!g.relay)
        return;
    // relay rows: one (64-token chunk, host) item per wave
    const int nchunk = (g.T + kWave - 1) / kWave;
    for (int it = wave; it < nchunk * g.H; it += kSmallWaves) {
        const int c = it / g.H, h = it - c * g.H;
        const int t = c * kWave + lane_id();
        relay_item(t < g.T, t, t, h, g, s_idx, s_hk, s_rk, s_hmask, s_hoff[h] + s_hcnt[c * hs + h], L);
    }
    clear_relay_tail(g, s_hoff[g.H], 0, 1, kSmallThreads, L);
}

// LDS bytes of the single-workgroup path, or 0 when the batch is too large for
// it. (Expert-column scans use threads [0, E) and host-column scans the last
// wave, so E <= 512 keeps them apart.)
size_t small_layout_lds(const Geometry &g)
{
    if (g.T > kSmallThreads || g.T * g.k > 4096 || g.E > 512)
        return 0;
    const size_t ints = 2 * (size_t)g.T + 3 * (size_t)g.T * g.k + (size_t)kSmallWaves * (g.E + 1) +
                        g.E + 1 + g.R + g.H + (size_t)kSmallWaves * (g.H + 1) + g.H + 1;
    const size_t bytes = ints * sizeof(int32_t);
    return bytes <= 64 * 1024 ? bytes : 0;
}

// LDS of an assign workgroup of nt threads, and the counting waves it uses:
// nt / 64, halved until the LDS fits in 64 KB.
size_t assign_lds(const Geometry &g, int nt, int &nww)
{
    const int ncol = g.E + g.R + g.H + 1;
    const int kc = g.ct * g.k;
    nww = nt / kWave;
    for (;;) {
        const size_t bytes =
            (size_t)(2 * g.ct + 2 * ncol + g.E + 1 + g.H + 1 + 3 * kc + nww * (g.E + 1)) *
            sizeof(int32_t);
        if (bytes <= 64 * 1024 || nww == 1)
            return bytes;
        nww /= 2;
    }
}

hipError_t launch_count(const Geometry &g, const int32_t *idx, const epx_layout &L,
                        hipStream_t stream)
{
    const int ncol = g.E + g.R + g.H + 1;
    const size_t lds = (size_t)(ncol + 3 * g.ct * g.k) * sizeof(int32_t);
    launch(layout_count_kernel, dim3(g.G), dim3(kCountThreads), lds, stream, idx, g,
                       L.workspace);
    return hipGetLastError();
}

hipError_t launch_scan(const Geometry &g, const epx_layout &L, hipStream_t stream)
{
    const int ncol = g.E + g.R + g.H + 1;
    const int cols_per_block = 256 / kWave;
    launch(layout_scan_kernel, dim3((ncol + cols_per_block - 1) / cols_per_block),
                       dim3(256), 0, stream, g, L.workspace);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_layout(const Geometry &g, const int32_t *idx, const epx_layout &L,
                         hipStream_t stream)
{
    const size_t small = small_layout_lds(g);
    if (small > 0) {
        launch(layout_small_kernel, dim3(1), dim3(kSmallThreads), small, stream, idx,
                           g, L);
        return hipGetLastError();
    }
    hipError_t err = launch_count(g, idx, L, stream);
    if (err != hipSuccess)
        return err;
    int nww = 0;
    const size_t lds_assign = assign_lds(g, kAssignThreads, nww);
    if (g.G <= kSumsMaxG) {
        launch(layout_assign_kernel<true>, dim3(g.G), dim3(kAssignThreads), lds_assign,
                           stream, idx, g, (const int32_t *)L.workspace, L, nww);
        return hipGetLastError();
    }
    if ((err = launch_scan(g, L, stream)) != hipSuccess)
        return err;
    launch(layout_assign_kernel<false>, dim3(g.G), dim3(kAssignThreads), lds_assign,
                       stream, idx, g, (const int32_t *)L.workspace, L, nww);
    return hipGetLastError();
}

bool launch_layout_assign_dispatch(const Geometry &g, const int32_t *idx, const epx_layout &L,
                                   const void *x, int32_t hidden, bool fp8, void *recv,
                                   float *scales, hipStream_t stream, hipError_t *err)
{
    // Per-expert fp8 keeps the separate launches: a token's quantisation
    // followed by 8 row stores in one workgroup measured slower (4096 x 7168:
    // 156.7 against 153.4 us per layer under graph replay) than the dispatch
    // kernel's column slices, which overlap the two; relay fp8 (about 3.6
    // rows per token) gains (131.8 against 132.9 us).
    if (g.m != 1 || g.k > kFusedMaxK || g.T == 0 || small_layout_lds(g) > 0 || (fp8 && !g.relay))
        return false;
    int nww = 0;
    const size_t lds_assign = assign_lds(g, kFusedThreads, nww);
    const int nvec = hidden / 8;
    // column slices only for small batches (about 2048 workgroups): every
    // slice workgroup repeats the derivation of its token's rows
    const int slice = fp8 ? slice_width(g.T, nvec, 16, 4096, 2048)
                          : slice_width(g.T, nvec, kWave, 1 << 30, 2048);
    size_t lds_tok = (size_t)((2 * g.E + 1 + 3) & ~3) * sizeof(int32_t);
    if (fp8)
        lds_tok += (size_t)slice * 8 + (size_t)(slice / 16) * sizeof(float);
    const size_t lds = lds_assign > lds_tok ? lds_assign : lds_tok;
    if (lds > 64 * 1024)
        return false;
    if ((*err = launch_count(g, idx, L, stream)) != hipSuccess)
        return true;
    if ((*err = launch_scan(g, L, stream)) != hipSuccess)
        return true;
    const dim3 grid = item_grid((int64_t)g.G + g.T, (nvec + slice - 1) / slice);
    if (fp8)
        launch(assign_copy_kernel<true>, grid, dim3(kFusedThreads), lds, stream, idx, g,
                           (const int32_t *)L.workspace, L, nww, (const u32x4 *)x, nvec, slice,
                           recv, scales);
    else
        launch(assign_copy_kernel<false>, grid, dim3(kFusedThreads), lds, stream, idx,
                           g, (const int32_t *)L.workspace, L, nww, (const u32x4 *)x, nvec, slice,
                           recv, scales);
    *err = hipGetLastError();
    return true;
}

}  // namespace epx
