// epx_device.h -- device helpers shared by the kernels of libepx (internal;
// not part of the C ABI).
#pragma once

#include "epx_internal.h"

namespace epx {

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// DPP lane moves (gfx9): row_shr:n moves each 16-lane row's values n lanes
// up (lanes below n in the row read 0: bound_ctrl); row_bcast:15 / 31 hand
// lane 15 / 31 to the next row(s), written only where row_mask allows.
constexpr int kDppRowShr = 0x110;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf, bool BOUND_ZERO = true>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, BOUND_ZERO);
}

// Inclusive scan within each 16-lane row.
__device__ __forceinline__ int row_inclusive_scan(int v)
{
    v += dpp<kDppRowShr + 1>(v);
    v += dpp<kDppRowShr + 2>(v);
    v += dpp<kDppRowShr + 4>(v);
    v += dpp<kDppRowShr + 8>(v);
    return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    v = row_inclusive_scan(v);
    v += dpp<kDppRowBcast15, 0xa, false>(v);   // rows 1 and 3 add the end of rows 0 and 2
    v += dpp<kDppRowBcast31, 0xc, false>(v);   // rows 2 and 3 add the end of rows 0-1
    return v;
}

// Maximum over the wave (values >= 0), the same in every lane.
__device__ __forceinline__ int wave_max(int v)
{
    v = max(v, dpp<kDppRowShr + 1>(v));
    v = max(v, dpp<kDppRowShr + 2>(v));
    v = max(v, dpp<kDppRowShr + 4>(v));
    v = max(v, dpp<kDppRowShr + 8>(v));
    v = max(v, dpp<kDppRowBcast15, 0xa, false>(v));
    v = max(v, dpp<kDppRowBcast31, 0xc, false>(v));
    return __builtin_amdgcn_readlane(v, kWave - 1);
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
inline __device__ void write_rank_and_group_offsets(const Geometry &g, const int32_t *eoff,
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

// ---------------------------------------------------------------- bf16 and fp8
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

// float32 pair -> two OCP E4M3FN codes (a in the low byte) by the packed
// hardware conversion, which rounds to nearest even. Finite values beyond
// +-448 are clamped first so that they saturate to +-448 (the conversion on
// its own turns them into NaN); NaN stays a NaN code. Checked on every
// float32 pattern against the integer definition (round the 23-bit mantissa
// to 3 bits, rebias; below 2^-6 the codes are rint(|v| * 2^9)): identical for
// every non-NaN input.
__device__ __forceinline__ float clamp448(float v)
{
    return fabsf(v) > 448.0f ? __builtin_copysignf(448.0f, v) : v;
}

__device__ __forceinline__ uint32_t e4m3_pair(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false) & 0xFFFFu;
}

// x / s for a block scale s >= 2^-100 and |x| <= 448 s, by fma-based
// division (P. Markstein, "Computation of elementary functions on the IBM
// RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990): the hardware
// reciprocal seed of s is refined by one Newton-Raphson step once per block
// (refined_reciprocal), then each quotient q0 = x*y takes two residual
// corrections r = fma(-s, q, x), q' = fma(r, y, q). The range scaling that a
// general division needs is left out, since these operands never need it;
// the sign is restored for zero x. Over every bf16 pair (x, amax) with
// |x| <= amax and s = amax / 448 >= 2^-100 it gives the same E4M3 code as the
// correctly rounded quotient (its last bit can differ only for quotients far
// below the smallest code); tests/test_fp8_quotient_gpu.py checks every such
// pair, and the smaller scales, through the dispatch.
__device__ __forceinline__ float div_by_scale(float x, float s, float y)
{
    const float q0 = x * y;
    const float r1 = __builtin_fmaf(-s, q0, x);
    const float q1 = __builtin_fmaf(r1, y, q0);
    const float r2 = __builtin_fmaf(-s, q1, x);
    return __builtin_copysignf(__builtin_fmaf(r2, y, q1), x);
}

__device__ __forceinline__ float refined_reciprocal(float s)
{
    const float y0 = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0);
}

// Four values of one block -> four codes (a in the low byte). zero: the
// block is all zeros (scale 0), codes keep the sign of each zero.
__device__ __forceinline__ uint32_t quantize4(float a, float b, float c, float d, float s, float y,
                                              bool zero)
{
    if (zero) {
        return ((__float_as_uint(a) >> 24) & 0x80u) | (((__float_as_uint(b) >> 24) & 0x80u) << 8) |
               (((__float_as_uint(c) >> 24) & 0x80u) << 16) |
               (((__float_as_uint(d) >> 24) & 0x80u) << 24);
    }
    float qa, qb, qc, qd;
    if (s >= 0x1p-100f) {
        qa = div_by_scale(a, s, y);
        qb = div_by_scale(b, s, y);
        qc = div_by_scale(c, s, y);
        qd = div_by_scale(d, s, y);
    } else {   // tiny blocks: the full IEEE division
        qa = a / s;
        qb = b / s;
        qc = c / s;
        qd = d / s;
    }
    return e4m3_pair(qa, qb) | (e4m3_pair(qc, qd) << 16);
}

// Quantise chunks [c_beg, c_beg + n) of the bf16 row xr (8 channels per
// 16-byte chunk) into LDS: 8 code bytes per chunk at s_codes (as u32x2) and
// one scale per 128-channel block at s_scale. A 16-lane group owns one block
// (its maximum by lane shuffles); each of the NT threads issues the loads of
// up to PRE chunks before converting any. n and NT are multiples of 16, so
// a 16-lane group is either all in range or all out. The caller
// synchronises the workgroup before reading the codes.
template <int NT, int PRE>
__device__ __forceinline__ void quantize_slice_to_lds(const u32x4 *__restrict__ xr, int c_beg,
                                                      int n, u32x2 *s_codes, float *s_scale)
{
    for (int base = 0; base < n; base += NT * PRE) {
        u32x4 xv[PRE];
#pragma unroll
        for (int p = 0; p < PRE; ++p) {
            const int i = base + p * NT + (int)threadIdx.x;
            if (i < n)
                xv[p] = xr[c_beg + i];
        }
#pragma unroll
        for (int p = 0; p < PRE; ++p) {
            const int i = base + p * NT + (int)threadIdx.x;
            if (i >= n)
                break;   // uniform over each 16-lane group, and later p are out too
            const u32x4 v = xv[p];
            const float f0 = bf16_lo(v.x), f1 = bf16_hi(v.x), f2 = bf16_lo(v.y), f3 = bf16_hi(v.y);
            const float f4 = bf16_lo(v.z), f5 = bf16_hi(v.z), f6 = bf16_lo(v.w), f7 = bf16_hi(v.w);
            float m = fmaxf(fmaxf(fmaxf(fabsf(f0), fabsf(f1)), fmaxf(fabsf(f2), fabsf(f3))),
                            fmaxf(fmaxf(fabsf(f4), fabsf(f5)), fmaxf(fabsf(f6), fabsf(f7))));
#pragma unroll
            for (int dd = 8; dd > 0; dd >>= 1)
                m = fmaxf(m, __shfl_xor(m, dd, 16));
            const float s = m / 448.0f;
            const bool zero = (m == 0.0f);
            const float y = refined_reciprocal(s);
            u32x2 q;
            q.x = quantize4(f0, f1, f2, f3, s, y, zero);
            q.y = quantize4(f4, f5, f6, f7, s, y, zero);
            s_codes[i] = q;
            if ((i & 15) == 0)
                s_scale[i >> 4] = s;
        }
    }
}

// ---------------------------------------------------------------- launch shapes
// Column slices per token, each a whole number of `align` chunks: at least
// `target` workgroups in all (small batches need slices to cover the GPU).
inline int slice_width(int T, int nvec, int align, int max_width, int target)
{
    int want = T >= target ? 1 : (target + T - 1) / T;
    int width = (nvec + want - 1) / want;
    width = ((width + align - 1) / align) * align;
    if (width < 4 * align && nvec > 4 * align)
        width = 4 * align;        // no slice below 4 alignment units
    if (width > max_width)
        width = (max_width / align) * align;
    return width < nvec ? width : nvec;
}


}  // namespace epx
