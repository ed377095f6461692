// epx_balance.hip -- per-step intra-host expert swap planner on gfx950.
//
// Per-step expert swaps inside a host ("Balancing and Beyond:
// Communication-Centric Optimizations in Expert Parallelism", digest section
// 3.1, Figure 2(b)). Load of rank r = sum of the token counts of the experts
// in its slots. Per host: sort the ranks by load, descending; rank i of that
// order is paired with rank n-1-i; for each pair, find the one exchange of
// an expert of the heavier rank with an expert of the lighter that gives the
// smallest new pair maximum, and apply it if the maximum drops by at least
// tau tokens (tau: the weight-move time expressed in per-token time).
//
// One workgroup per host. All E counts and the host's slots (rank-major, epr
// per rank) are staged in LDS with independent loads; rank loads are summed
// there; ranks are ordered by load descending, then rank index. Pairs touch
// disjoint ranks, so they are planned at once: pair p gets a team of waves
// that scans the epr x epr candidate swaps and reduces a 64-bit key (new
// maximum, then candidate index = heavy slot * epr + light slot), so the
// smallest key is the best swap with ties to the smaller heavy slot, then the
// smaller light slot. One thread per pair then records and applies it.
//
// A host whose slots hold an expert id outside [0, E) is not planned: its
// slots are copied unchanged, its loads and pair records are written as -1
// (applied 0) and host_bad[h] gets the number of such ids; other hosts are
// planned as usual.
#include "epx_internal.h"

namespace epx {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
static_assert(kWaves >= kMaxRanksPerHost / 2, "one wave at least per pair");

// Signed order of the new maximum as unsigned order of the key's high word.
__device__ __forceinline__ uint64_t swap_key(int32_t m, int32_t cand)
{
    return ((uint64_t)((uint32_t)m ^ 0x80000000u) << 32) | (uint32_t)cand;
}

__global__ __launch_bounds__(kThreads) void plan_swaps_kernel(
    int E, int epr, int rph, const int32_t *__restrict__ count,
    const int32_t *__restrict__ slot_in, int tau, int32_t *__restrict__ slot_out,
    int32_t *__restrict__ load_before, int32_t *__restrict__ load_after,
    int32_t *__restrict__ swaps, int32_t *__restrict__ host_bad)
{
    extern __shared__ int32_t lds[];
    const int h = blockIdx.x;
    const int nslot = rph * epr, npair = rph / 2;
    int32_t *s_count = lds;          // expert_count [E]
    int32_t *s_e = s_count + E;      // experts in the host's slots [nslot]
    int32_t *s_c = s_e + nslot;      // their counts [nslot]
    __shared__ int32_t s_load[kMaxRanksPerHost], s_after[kMaxRanksPerHost];
    __shared__ int32_t s_order[kMaxRanksPerHost];
    __shared__ uint64_t s_wbest[kWaves];
    __shared__ int32_t s_bad;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int32_t *my_slots = slot_in + (int64_t)h * nslot;

    if (tid < rph)
        s_load[tid] = 0;
    if (tid == 0)
        s_bad = 0;
    const int nstage = E > nslot ? E : nslot;
    for (int i = tid; i < nstage; i += kThreads) {   // both loads in flight before either store
        const int c = i < E ? count[i] : 0;
        const int e = i < nslot ? my_slots[i] : 0;
        if (i < E)
            s_count[i] = c;
        if (i < nslot)
            s_e[i] = e;
    }
    __syncthreads();
    for (int i = tid; i < nslot; i += kThreads) {
        const int e = s_e[i];
        const bool ok = (unsigned)e < (unsigned)E;
        const int c = ok ? s_count[e] : 0;
        s_c[i] = c;
        atomicAdd(&s_load[i / epr], c);
        if (!ok)
            atomicAdd(&s_bad, 1);
    }
    __syncthreads();
    if (tid == 0)
        host_bad[h] = s_bad;
    if (s_bad != 0) {   // uniform over the workgroup
        for (int i = tid; i < nslot; i += kThreads)
            slot_out[(int64_t)h * nslot + i] = s_e[i];
        if (tid < rph) {
            load_before[h * rph + tid] = -1;
            load_after[h * rph + tid] = -1;
        }
        for (int i = tid; i < npair * 7; i += kThreads)
            swaps[(int64_t)h * npair * 7 + i] = i % 7 == 6 ? 0 : -1;
        return;
    }
    if (tid < rph) {
        const int load = s_load[tid];
        load_before[h * rph + tid] = load;
        s_after[tid] = load;
        int pos = 0;
        for (int j = 0; j < rph; ++j)
            pos += (s_load[j] > load) || (s_load[j] == load && j < tid);
        s_order[pos] = tid;
    }
    __syncthreads();

    if (npair > 0) {   // uniform
        const int wpp = kWaves / npair;   // waves per pair
        const int team = wave / wpp;
        if (team < npair) {
            const int A = s_order[team], B = s_order[rph - 1 - team];
            const int LA = s_load[A], LB = s_load[B];
            const int32_t *ca_row = s_c + A * epr, *cb_row = s_c + B * epr;
            const int ncand = epr * epr;
            uint64_t best = ~0ull;
            for (int cand = (wave - team * wpp) * kWave + lane; cand < ncand; cand += wpp * kWave) {
                const int a = cand / epr, b = cand - a * epr;
                const int ca = ca_row[a], cb = cb_row[b];
                const int m = max(LA - ca + cb, LB - cb + ca);
                best = min(best, swap_key(m, cand));
            }
#pragma unroll
            for (int d = kWave / 2; d > 0; d >>= 1) {
                const uint64_t o = __shfl_xor(best, d, kWave);
                best = o < best ? o : best;
            }
            if (lane == 0)
                s_wbest[wave] = best;
        }
        __syncthreads();
        if (tid < npair) {
            const int p = tid;
            uint64_t b0 = s_wbest[p * wpp];
            for (int w = 1; w < wpp; ++w)
                b0 = s_wbest[p * wpp + w] < b0 ? s_wbest[p * wpp + w] : b0;
            const int A = s_order[p], B = s_order[rph - 1 - p];
            const int LA = s_load[A], LB = s_load[B];
            const int cand = (int)(uint32_t)b0;
            const int m = (int)((uint32_t)(b0 >> 32) ^ 0x80000000u);
            const int a = cand / epr, b = cand - a * epr;
            const int ia = A * epr + a, ib = B * epr + b;
            const int ea = s_e[ia], eb = s_e[ib], ca = s_c[ia], cb = s_c[ib];
            const int old = max(LA, LB);
            const int applied = (old - m > 0) && (old - m >= tau);
            int32_t *rec = swaps + ((int64_t)h * npair + p) * 7;
            rec[0] = h * rph + A;
            rec[1] = ea;
            rec[2] = h * rph + B;
            rec[3] = eb;
            rec[4] = old;
            rec[5] = m;
            rec[6] = applied;
            if (applied) {   // pairs own disjoint ranks: no two threads touch one slot
                s_e[ia] = eb;
                s_e[ib] = ea;
                s_after[A] = LA - ca + cb;
                s_after[B] = LB - cb + ca;
            }
        }
        __syncthreads();
    }
    for (int i = tid; i < nslot; i += kThreads)
        slot_out[(int64_t)h * nslot + i] = s_e[i];
    if (tid < rph)
        load_after[h * rph + tid] = s_after[tid];
}

}  // namespace

hipError_t launch_plan_swaps(int E, int R, int H, const int32_t *count, const int32_t *slot_in,
                             int tau, int32_t *slot_out, int32_t *load_before,
                             int32_t *load_after, int32_t *swaps, int32_t *host_bad,
                             hipStream_t stream)
{
    const int epr = E / R, rph = R / H;
    const size_t lds = ((size_t)E + 2 * (size_t)rph * epr) * sizeof(int32_t);
    launch(plan_swaps_kernel, dim3(H), dim3(kThreads), lds, stream, E, epr, rph, count,
                       slot_in, tau, slot_out, load_before, load_after, swaps, host_bad);
    return hipGetLastError();
}

}  // namespace epx
