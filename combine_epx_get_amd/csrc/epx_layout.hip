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
// Row order: per-expert rows by (expert, token, j); relay rows by (host,
// token). Positions come from ordered wave walks, never from atomic order:
// a wave takes 64 pairs at a time in (t, j) order, groups equal expert ids
// with ceil(log2 E) ballots (a wave-level multisplit) and gives each lane
// base + popcount(peers below it); the group's first lane then advances the
// base. Counting may use LDS atomics, because counts do not depend on order.
//
// Three shapes, no global atomics and no zero-filled buffers:
//   small batches (<= 4096 pairs): one workgroup does everything in LDS;
//   up to 16 workgroups of up to 64 tokens: count, then assign (each assign
//     workgroup sums the count columns itself);
//   more: count, a column scan (one wave per counter), assign.
// Every per-pair rank and host is computed once, with division constants
// prepared on the host, and staged in LDS with the chunk's ids.
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

// Lanes whose `e` equals mine among the active lanes (ballot multisplit).
__device__ __forceinline__ uint64_t match_peers(bool active, int e, int nbits)
{
    uint64_t peers = __ballot(active);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool on = (e >> bit) & 1;
        const uint64_t m = __ballot(on);
        peers &= on ? m : ~m;
    }
    return peers;
}

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

// Relay rows of one token on one lane of a wave holding up to 64 consecutive
// tokens: for each host, rows of the tokens that touch it, in token order,
// from `base(h)` on. Every lane of the wave must call it (ballots). KR > 0:
// the token's ids, ranks and hosts are held in registers (k <= KR).
template <int KR, typename Base>
__device__ __forceinline__ void relay_rows(bool act, int t, const int32_t *ids, const int32_t *rks,
                                           const int32_t *hks, const Geometry &g, Base base,
                                           const epx_layout &L)
{
    const uint64_t below = (1ull << lane_id()) - 1ull;
    constexpr int N = KR > 0 ? KR : 1;
    int e_[N], r_[N], h_[N];
    uint64_t hosts = 0;
    if (KR > 0) {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const bool v = act && j < g.k;
            e_[j] = v ? ids[j] : -1;
            r_[j] = v ? rks[j] : 0;
            h_[j] = v ? hks[j] : -1;
            if (v)
                hosts |= 1ull << h_[j];
        }
    } else if (act) {
        for (int j = 0; j < g.k; ++j)
            hosts |= 1ull << hks[j];
    }
    for (int h = 0; h < g.H; ++h) {
        const bool has = (hosts >> h) & 1ull;
        const uint64_t bal = __ballot(has);
        if (!act)
            continue;
        if (!has) {
            L.relay_slot[(int64_t)t * g.H + h] = -1;
            continue;
        }
        const int r = base(h) + __popcll(bal & below);
        L.relay_slot[(int64_t)t * g.H + h] = r;
        L.relay_token[r] = t;
        int32_t *fan = L.fanout_expert + (int64_t)r * g.k;
        uint32_t mask = 0;
        if (KR > 0) {
#pragma unroll
            for (int j = 0; j < N; ++j)
                if (j < g.k) {
                    const bool here = h_[j] == h;
                    fan[j] = here ? e_[j] : -1;
                    if (here)
                        mask |= 1u << (r_[j] - h * g.rph);
                }
        } else {
            for (int j = 0; j < g.k; ++j) {
                const bool here = hks[j] == h;
                fan[j] = here ? ids[j] : -1;
                if (here)
                    mask |= 1u << (rks[j] - h * g.rph);
            }
        }
        L.fanout_rank_mask[r] = mask;
    }
}

template <typename Base>
__device__ __forceinline__ void relay_rows_any(bool act, int t, const int32_t *ids,
                                               const int32_t *rks, const int32_t *hks,
                                               const Geometry &g, Base base, const epx_layout &L)
{
    if (g.k <= kRegK)
        relay_rows<kRegK>(act, t, ids, rks, hks, g, base, L);
    else
        relay_rows<0>(act, t, ids, rks, hks, g, base, L);
}

// Relay rows past the used ones, [used, capacity) split over `parts`, read as empty.
__device__ __forceinline__ void clear_relay_tail(const Geometry &g, int64_t used, int part,
                                                 int parts, int nthreads, const epx_layout &L)
{
    const int64_t cap = (int64_t)g.T * min(g.k, g.H);
    const int64_t per = (cap + parts - 1) / parts;
    const int64_t beg = max(used, (int64_t)part * per), end = min(cap, (int64_t)(part + 1) * per);
    for (int64_t r = beg + threadIdx.x; r < end; r += nthreads) {
        L.relay_token[r] = -1;
        L.fanout_rank_mask[r] = 0u;
    }
    for (int64_t i = beg * g.k + threadIdx.x; i < end * g.k; i += nthreads)
        L.fanout_expert[i] = -1;
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

// ---------------------------------------------------------------- expert order
// Rows are ordered by expert in the scan order of this function: expert ids
// ascending, or with m > 1 expert groups (per-expert overlap) by (group,
// rank, local index in the group), so that one group's rows form one range.
__device__ __forceinline__ int expert_at(const Geometry &g, int q)
{
    if (g.m == 1)
        return q;
    const int per_group = g.R * g.epg;
    const int grp = q / per_group;
    const int rem = q - grp * per_group;
    const int r = rem / g.epg;
    return r * g.epr + grp * g.epg + (rem - r * g.epg);
}

// First row of block b = group * R + rank (b == m * R: the total), from the
// final expert offsets eoff[0, E].
__device__ __forceinline__ int block_start(const Geometry &g, const int32_t *eoff, int b)
{
    if (b >= g.m * g.R)
        return eoff[g.E];
    const int grp = b / g.R, r = b - grp * g.R;
    return eoff[r * g.epr + grp * g.epg];
}

// Per-rank and per-group offsets from the final expert offsets (threads
// [0, nthreads) of the workgroup): rank_offset (-1 with groups: a rank's rows
// are then split over the groups), rank_rows and group_offset.
__device__ void write_rank_and_group_offsets(const Geometry &g, const int32_t *eoff,
                                             const epx_layout &L, int nthreads)
{
    const int tid = threadIdx.x;
    for (int r = tid; r <= g.R; r += nthreads) {
        L.rank_offset[r] = g.m == 1 ? eoff[r * g.epr] : -1;
        if (r < g.R) {
            int rows = 0;
            for (int grp = 0; grp < g.m; ++grp)
                rows += block_start(g, eoff, grp * g.R + r + 1) - block_start(g, eoff, grp * g.R + r);
            L.rank_rows[r] = rows;
        }
    }
    for (int b = tid; b <= g.m * g.R; b += nthreads)
        L.group_offset[b] = block_start(g, eoff, b);
}

// ---------------------------------------------------------------- assign
constexpr int kAssignThreads = 128;

// Exclusive scan of the expert counts src[0, E) (LDS, by expert id) in the
// row order of expert_at into dst[0, E] (LDS, by expert id), dst[E] = total.
__device__ void block_exclusive_scan(const Geometry &g, const int32_t *src, int32_t *dst,
                                     int32_t *s_wsum)
{
    const int tid = threadIdx.x, n = g.E;
    const int per = (n + kAssignThreads - 1) / kAssignThreads;
    const int beg = min(tid * per, n), end = min(beg + per, n);
    int sum = 0;
    for (int i = beg; i < end; ++i)
        sum += src[expert_at(g, i)];
    const int incl = wave_inclusive_scan(sum);
    if (lane_id() == kWave - 1)
        s_wsum[tid / kWave] = incl;
    __syncthreads();
    int run = incl - sum + (tid >= kWave ? s_wsum[0] : 0);
    for (int i = beg; i < end; ++i) {
        const int e = expert_at(g, i);
        const int v = src[e];
        dst[e] = run;
        run += v;
    }
    if (tid == kAssignThreads - 1)
        dst[n] = run;
}

// SUMS: this workgroup sums the raw count columns itself (total and the
// prefix over workgroups before it); otherwise the scan kernel has left the
// prefix in place and the totals after the columns.
template <bool SUMS>
__global__ __launch_bounds__(kAssignThreads) void layout_assign_kernel(
    const int32_t *__restrict__ idx, Geometry g, const int32_t *__restrict__ ws, epx_layout L)
{
    extern __shared__ int32_t lds[];
    const int ncol = g.E + g.R + g.H + 1;
    const int kc = g.ct * g.k;
    int32_t *s_tot = lds;                  // [ncol] column totals
    int32_t *s_pre = s_tot + ncol;         // [ncol] this workgroup's prefix per column
    int32_t *s_eoff = s_pre + ncol;        // [E + 1]
    int32_t *s_hoff = s_eoff + g.E + 1;    // [H + 1]
    int32_t *s_idx = s_hoff + g.H + 1;     // [64 k] ids, ranks, hosts of the chunk
    int32_t *s_rk = s_idx + kc;
    int32_t *s_hk = s_rk + kc;
    __shared__ int32_t s_wsum[2];
    __shared__ int32_t s_wmax[2];

    const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int t0 = b * g.ct;
    const int nt = max(0, min(g.ct, g.T - t0));
    const int64_t p0 = (int64_t)t0 * g.k;

    stage_pairs(idx, p0, nt * g.k, g, s_idx, s_rk, s_hk, kAssignThreads);
    if (SUMS) {
        // each thread sums whole columns as 16-byte vectors (Gs % 4 == 0);
        // G <= 16 here, so a column is at most 4 vectors, all loaded at once
        for (int c = tid; c < ncol; c += kAssignThreads) {
            const int4 *col = (const int4 *)(ws + (int64_t)c * g.Gs);
            int tot = 0, pre = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (4 * i >= g.Gs)
                    break;
                const int4 v = col[i];
                const int i0 = 4 * i;   // entries [G, Gs) are padding, never written
                tot += (i0 < g.G ? v.x : 0) + (i0 + 1 < g.G ? v.y : 0) +
                       (i0 + 2 < g.G ? v.z : 0) + (i0 + 3 < g.G ? v.w : 0);
                pre += (i0 < b ? v.x : 0) + (i0 + 1 < b ? v.y : 0) + (i0 + 2 < b ? v.z : 0) +
                       (i0 + 3 < b ? v.w : 0);
            }
            s_tot[c] = tot;
            s_pre[c] = pre;
        }
    } else {
        for (int c = tid; c < ncol; c += kAssignThreads) {
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
    block_exclusive_scan(g, s_tot, s_eoff, s_wsum);
    if (wave == 0) {
        const int v = lane < g.H ? s_tot[g.E + g.R + lane] : 0;
        const int incl = wave_inclusive_scan(v);
        if (lane < g.H)
            s_hoff[lane] = incl - v;
        if (lane == kWave - 1)
            s_hoff[g.H] = incl;
    }
    __syncthreads();

    if (b == 0) {
        for (int e = tid; e <= g.E; e += kAssignThreads) {
            L.expert_offset[e] = s_eoff[e];
            if (e < g.E)
                L.expert_count[e] = s_tot[e];
        }
        write_rank_and_group_offsets(g, s_eoff, L, kAssignThreads);
        for (int r = tid; r < g.R; r += kAssignThreads)
            L.rank_tokens[r] = s_tot[g.E + r];
        for (int h = tid; h <= g.H; h += kAssignThreads) {
            L.host_offset[h] = s_hoff[h];
            if (h < g.H) {
                L.host_tokens[h] = s_tot[g.E + g.R + h];
                L.relay_dst_rank[h] = h * g.rph + g.s % g.rph;
            }
        }
        int m = 0;
        for (int e = tid; e < g.E; e += kAssignThreads)
            m = max(m, s_tot[e]);
        m = wave_max(m);
        if (lane == 0)
            s_wmax[wave] = m;
        __syncthreads();
        if (tid == 0) {
            L.totals[0] = g.T * g.k;
            L.totals[1] = s_hoff[g.H];
            L.totals[2] = max(s_wmax[0], s_wmax[1]);
            L.totals[3] = 0;
        }
    }

    if (wave == 0) {
        // rows per expert in (t, j) order: base = offset + rows of earlier workgroups
        for (int e = lane; e < g.E; e += kWave)
            s_eoff[e] += s_pre[e];
        const uint64_t below = (1ull << lane) - 1ull;
        const int np = nt * g.k;
        for (int base = 0; base < np; base += kWave) {
            const int p = base + lane;
            const bool act = p < np;
            const int e = act ? s_idx[p] : 0;
            const uint64_t peers = match_peers(act, e, g.nbits);
            if (act) {
                const int before = __popcll(peers & below);
                const int first = s_eoff[e];
                const int row = first + before;
                L.slot[p0 + p] = row;
                L.row_token[row] = t0 + g.div_k.div(p);
                if (before == 0)
                    s_eoff[e] = first + __popcll(peers);
            }
        }
    } else if (g.relay) {
        const int o = lane * g.k;
        relay_rows_any(lane < nt, t0 + lane, s_idx + o, s_rk + o, s_hk + o, g,
                   [&](int h) { return s_hoff[h] + s_pre[g.E + g.R + h]; }, L);
    }
    if (g.relay)
        clear_relay_tail(g, s_hoff[g.H], b, g.G, kAssignThreads, L);
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

__global__ __launch_bounds__(kSmallThreads) void layout_small_kernel(
    const int32_t *__restrict__ idx, Geometry g, epx_layout L)
{
    extern __shared__ int32_t lds[];
    const int P = g.T * g.k;
    int32_t *s_idx = lds;                              // [P] ids, ranks, hosts
    int32_t *s_rk = s_idx + P;
    int32_t *s_hk = s_rk + P;
    int32_t *s_cnt = s_hk + P;                         // [waves][E] counts, then row bases
    int32_t *s_eoff = s_cnt + kSmallWaves * g.E;       // [E + 1]
    int32_t *s_rtok = s_eoff + g.E + 1;                // [R]
    int32_t *s_htok = s_rtok + g.R;                    // [H]
    int32_t *s_hcnt = s_htok + g.H;                    // [waves][H] counts, then relay bases
    int32_t *s_hoff = s_hcnt + kSmallWaves * g.H;      // [H + 1]
    __shared__ int32_t s_bad;
    __shared__ int32_t s_wsum[kSmallWaves];
    __shared__ int32_t s_wmax[kSmallWaves];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const uint64_t below = (1ull << lane) - 1ull;

    stage_pairs(idx, 0, P, g, s_idx, s_rk, s_hk, kSmallThreads);
    for (int i = tid; i < kSmallWaves * g.E; i += kSmallThreads)
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
            s_cnt[wave * g.E + e] += __popcll(peers);
    }
    // bad ids, distinct ranks and hosts per token
    for (int p = tid; p < P; p += kSmallThreads) {
        const int r = s_rk[p];
        if (r < 0) {
            atomicAdd(&s_bad, 1);
            continue;
        }
        const int first = g.div_k.div(p) * g.k;
        const int h = s_hk[p];
        bool new_rank = true, new_host = true;
        for (int q = first; q < p; ++q) {
            new_rank = new_rank && s_rk[q] != r;
            new_host = new_host && s_hk[q] != h;
        }
        if (new_rank)
            atomicAdd(&s_rtok[r], 1);
        if (new_host)
            atomicAdd(&s_htok[h], 1);
    }
    // per-wave relay counts: tokens of wave w touching host h
    uint64_t hosts = 0;
    if (tid < g.T)
        for (int j = 0; j < g.k; ++j) {
            const int h = s_hk[tid * g.k + j];
            if (h >= 0)
                hosts |= 1ull << h;
        }
    for (int h = 0; h < g.H; ++h) {
        const uint64_t bal = __ballot((hosts >> h) & 1ull);
        if (lane == 0)
            s_hcnt[wave * g.H + h] = __popcll(bal);
    }
    __syncthreads();
    if (s_bad != 0) {
        if (tid == 0)
            L.totals[3] = s_bad;
        return;   // out-of-range ids: nothing else is defined
    }

    // scans over waves: each wave's base per expert / per host, and totals
    if (tid < g.E) {
        int run = 0;
        for (int w = 0; w < kSmallWaves; ++w) {
            const int c = s_cnt[w * g.E + tid];
            s_cnt[w * g.E + tid] = run;
            run += c;
        }
        s_eoff[tid] = run;
    } else if (tid >= kSmallThreads - kWave && tid - (kSmallThreads - kWave) < g.H) {
        const int h = tid - (kSmallThreads - kWave);
        int run = 0;
        for (int w = 0; w < kSmallWaves; ++w) {
            const int c = s_hcnt[w * g.H + h];
            s_hcnt[w * g.H + h] = run;
            run += c;
        }
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
    for (int w = 0; w < kSmallWaves; ++w)
        for (int e = tid; e < g.E; e += kSmallThreads)
            s_cnt[w * g.E + e] += s_eoff[e];
    __syncthreads();

    // ordered walk: rows of each expert in (t, j) order
    for (int base = pw0; base < pw1; base += kWave) {
        const int p = base + lane;
        const bool act = p < pw1;
        const int e = act ? s_idx[p] : 0;
        const uint64_t peers = match_peers(act, e, g.nbits);
        if (act) {
            const int before = __popcll(peers & below);
            const int first = s_cnt[wave * g.E + e];
            const int row = first + before;
            L.slot[p] = row;
            L.row_token[row] = g.div_k.div(p);
            if (before == 0)
                s_cnt[wave * g.E + e] = first + __popcll(peers);
        }
    }
    if (!g.relay)
        return;
    const int o = (tid < g.T ? tid : 0) * g.k;
    relay_rows_any(tid < g.T, tid, s_idx + o, s_rk + o, s_hk + o, g,
               [&](int h) { return s_hoff[h] + s_hcnt[wave * g.H + h]; }, L);
    clear_relay_tail(g, s_hoff[g.H], 0, 1, kSmallThreads, L);
}

// LDS bytes of the single-workgroup path, or 0 when the batch is too large for
// it. (Expert-column scans use threads [0, E) and host-column scans the last
// wave, so E <= 512 keeps them apart.)
size_t small_layout_lds(const Geometry &g)
{
    if (g.T > kSmallThreads || g.T * g.k > 4096 || g.E > 512)
        return 0;
    const size_t ints = 3 * (size_t)g.T * g.k + (size_t)kSmallWaves * g.E + g.E + 1 + g.R + g.H +
                        (size_t)kSmallWaves * g.H + g.H + 1;
    const size_t bytes = ints * sizeof(int32_t);
    return bytes <= 64 * 1024 ? bytes : 0;
}

}  // namespace

hipError_t launch_layout(const Geometry &g, const int32_t *idx, const epx_layout &L,
                         hipStream_t stream)
{
    const size_t small = small_layout_lds(g);
    if (small > 0) {
        hipLaunchKernelGGL(layout_small_kernel, dim3(1), dim3(kSmallThreads), small, stream, idx,
                           g, L);
        return hipGetLastError();
    }
    const int ncol = g.E + g.R + g.H + 1;
    const int kc = g.ct * g.k;
    const size_t lds_count = (size_t)(ncol + 3 * kc) * sizeof(int32_t);
    hipLaunchKernelGGL(layout_count_kernel, dim3(g.G), dim3(kCountThreads), lds_count, stream, idx,
                       g, L.workspace);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const size_t lds_assign = (size_t)(2 * ncol + g.E + 1 + g.H + 1 + 3 * kc) * sizeof(int32_t);
    if (g.G <= 16) {
        hipLaunchKernelGGL(layout_assign_kernel<true>, dim3(g.G), dim3(kAssignThreads), lds_assign,
                           stream, idx, g, (const int32_t *)L.workspace, L);
        return hipGetLastError();
    }
    const int cols_per_block = 256 / kWave;
    hipLaunchKernelGGL(layout_scan_kernel, dim3((ncol + cols_per_block - 1) / cols_per_block),
                       dim3(256), 0, stream, g, L.workspace);
    err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(layout_assign_kernel<false>, dim3(g.G), dim3(kAssignThreads), lds_assign,
                       stream, idx, g, (const int32_t *)L.workspace, L);
    return hipGetLastError();
}

}  // namespace epx
