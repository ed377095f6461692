/*
 * epx_oracle.c -- plain, slow CPU oracle for MoE expert-parallel dispatch and
 * combine on one rank.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. The product path
 * (the HIP library) shares no code, header, table or helper with it.
 *
 * Every function is the definition written out as scalar loops, in the order
 * the definitions are stated, single-threaded, with no blocking or fusion:
 *
 *  - Layout: counts per expert, per rank and per host, prefix offsets and the
 *    position of every (token, expert) copy. The digest "Balancing and
 *    Beyond: Communication-Centric Optimizations in Expert Parallelism"
 *    routes every token to k experts chosen for it (section 1) and measures
 *    imbalance as the largest expert count divided by the mean count
 *    (section 2);
 *    the DeepEP issue "[GH-ISSUE #250] Profiling when rank unbalance" counts
 *    the tokens each rank receives (the maintainer's estimate and the
 *    follow-up question).
 *  - Per-expert dispatch: one copy of a token's row per destination expert
 *    (digest section 3.2, Mode 1).
 *  - Relay dispatch: one copy per destination host, addressed to the
 *    same-index GPU there, with an intra-host fan-out index (digest section
 *    3.2, Mode 2, Figure 3; glossary entry "De-redundancy").
 *  - FP8 dispatch: BF16 activations converted to FP8 inside dispatch (digest
 *    section 3.1). Format OCP E4M3FN (largest finite value 448), one float32
 *    scale per 128 channels equal to the block's max |x| / 448.
 *  - Combine: gather each token's k expert outputs and sum them with the gate
 *    weights (digest section 3.2, the combine step, and section 3.4, combine
 *    buffers sized batch x k), accumulated in float32 with fmaf in ascending
 *    j from +0, rounded once to bf16 (nearest, ties to even).
 *  - Relay receive side and two-level combine (digest section 3.2, Mode 2,
 *    Figure 3), expert groups for per-expert overlap (section 3.3, Figure 4)
 *    and the per-step intra-host swap planner (section 3.1, Figure 2(b)):
 *    see each section below.
 *
 * Readings where the pages are silent (all listed with reasons in the design
 * notes of the repository): experts map to ranks in contiguous blocks and
 * ranks to hosts in contiguous blocks; per-expert rows are ordered by expert,
 * then token, then position j; relay rows are ordered by host, then token,
 * and the token's own host gets a row too; an out-of-range expert id is an
 * error; an all-zero fp8 block has scale 0 and codes +-0.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    ORC_OK = 0,
    ORC_ERR_ARG = 1,
    ORC_ERR_INDEX = 2,
    ORC_ERR_VALUE = 5 /* non-finite activation in the fp8 path */
};

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 bit pattern -> float32 (exact: bf16 is the top half of float32). */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float f32_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float32 -> bf16, round to nearest with ties to even, by comparing the
 * distances to the two neighbouring bf16 values in double precision. */
uint16_t oracle_f32_to_bf16(float v)
{
    uint32_t u = f32_bits(v);
    if (isnan(v))
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    if (isinf(v))
        return (uint16_t)(u >> 16);
    uint32_t lo_bits = u & 0xFFFF0000u;           /* toward zero */
    double lo = (double)f32_from_bits(lo_bits);
    /* spacing of bf16 values in lo's binade (subnormals share the spacing of
     * the smallest normal binade); lo + step is the next bf16 magnitude away
     * from zero, 2^128 when lo is the largest finite bf16 */
    int e = (int)((lo_bits >> 23) & 0xFFu);
    double step = ldexp(1.0, (e == 0 ? 1 : e) - 127 - 7);
    double mag = fabs((double)v), lo_mag = fabs(lo), hi_mag = lo_mag + step;
    double d_lo = mag - lo_mag, d_hi = hi_mag - mag;
    uint32_t pick_hi;
    if (d_lo < d_hi)
        pick_hi = 0;
    else if (d_hi < d_lo)
        pick_hi = 1;
    else
        pick_hi = (lo_bits >> 16) & 1u;           /* tie: keep the even one */
    uint32_t r = (lo_bits >> 16) + pick_hi;        /* +1 ulp in magnitude (may carry into the exponent or reach inf) */
    return (uint16_t)r;
}

/* float32 -> OCP E4M3FN byte: round to nearest, ties to even; finite values
 * beyond +-448 saturate to +-448. Written from the format: 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
 * subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity. */
uint8_t oracle_f32_to_e4m3(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    float a = fabsf(v);
    if (a >= 448.0f)
        return (uint8_t)(sign | 0x7E);
    if (a < 0.015625f) {                 /* below 2^-6, the smallest normal: grid step 2^-9 */
        float m = rintf(a * 512.0f);     /* exact product; rint rounds half to even */
        return (uint8_t)(sign | (uint8_t)m); /* m == 8 is the encoding of 2^-6 */
    }
    int ex;
    float f = frexpf(a, &ex);            /* a = f * 2^ex, f in [0.5, 1) */
    int unb = ex - 1;                    /* a = (2f) * 2^unb, 2f in [1, 2) */
    float m = rintf((2.0f * f - 1.0f) * 8.0f); /* exact operands; half to even */
    if (m == 8.0f) {
        m = 0.0f;
        unb += 1;
    }
    int biased = unb + 7;
    return (uint8_t)(sign | (uint8_t)(biased << 3) | (uint8_t)m);
}

/* OCP E4M3FN byte -> float32 value. */
float oracle_e4m3_to_f32(uint8_t q)
{
    int e = (q >> 3) & 0xF, m = q & 7;
    float mag;
    if (e == 0xF && m == 7)
        mag = NAN;
    else if (e == 0)
        mag = ldexpf((float)m, -9);
    else
        mag = ldexpf((float)(8 + m), e - 10);   /* (1 + m/8) * 2^(e-7) */
    return (q & 0x80) ? -mag : mag;
}

void oracle_f32_to_e4m3_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_e4m3(in[i]);
}

void oracle_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(in[i]);
}

void oracle_e4m3_to_f32_array(const uint8_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_to_f32(in[i]);
}

/* ------------------------------------------------------------------ */
/* Layout                                                              */
/* ------------------------------------------------------------------ */

/* Experts sit on ranks in contiguous blocks of epr, ranks on hosts in
 * contiguous blocks of rph. */
static int32_t rank_of(int32_t e, int32_t epr)
{
    return e / epr;
}

static int32_t host_of(int32_t e, int32_t epr, int32_t rph)
{
    return rank_of(e, epr) / rph;
}

/* Geometry checks shared by every entry point of this file. */
static int geometry_ok(int32_t T, int32_t k, int32_t E, int32_t R, int32_t H, int32_t s)
{
    if (T < 0 || k < 1 || E < 1 || R < 1 || H < 1)
        return 0;
    if (E % R != 0 || R % H != 0 || k > E || s < 0 || s >= R)
        return 0;
    if (R / H > 32) /* fan-out rank mask is 32 bits wide */
        return 0;
    return 1;
}

/*
 * oracle_layout: all counts, offsets and positions for one source rank.
 *
 * idx [T*k]: expert id of pair (t, j) at t*k + j.
 * relay != 0 additionally fills relay_slot [T*H], relay_token [cap],
 * fanout_expert [cap*k] and fanout_rank_mask [cap], cap = T*min(k, H); entries
 * of the last three beyond the used relay rows are -1, -1 and 0.
 * totals[4] = {rows, relay rows, max expert count, number of bad ids}.
 */
int oracle_layout(int32_t T, int32_t k, int32_t E, int32_t R, int32_t H, int32_t s, int32_t relay,
                  const int32_t *idx,
                  int32_t *expert_count, int32_t *expert_offset,
                  int32_t *rank_rows, int32_t *rank_tokens, int32_t *rank_offset,
                  int32_t *host_tokens, int32_t *host_offset,
                  int32_t *slot, int32_t *row_token,
                  int32_t *relay_slot, int32_t *relay_token, int32_t *fanout_expert,
                  uint32_t *fanout_rank_mask, int32_t *relay_dst_rank, int32_t *totals)
{
    if (!geometry_ok(T, k, E, R, H, s))
        return ORC_ERR_ARG;
    const int32_t epr = E / R;    /* experts per rank */
    const int32_t rph = R / H;    /* ranks per host */
    const int64_t P = (int64_t)T * k;

    /* out-of-range ids are an error: count them, compute nothing else */
    int64_t bad = 0;
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] < 0 || idx[p] >= E)
            bad += 1;
    totals[0] = 0;
    totals[1] = 0;
    totals[2] = 0;
    totals[3] = (int32_t)bad;
    if (bad)
        return ORC_ERR_INDEX;

    /* copies per expert */
    for (int32_t e = 0; e < E; ++e)
        expert_count[e] = 0;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j)
            expert_count[idx[(int64_t)t * k + j]] += 1;

    /* copies per rank: the sum over the rank's experts e in [r*epr, (r+1)*epr) */
    for (int32_t r = 0; r < R; ++r) {
        rank_rows[r] = 0;
        for (int32_t e = r * epr; e < (r + 1) * epr; ++e)
            rank_rows[r] += expert_count[e];
    }

    /* distinct tokens per rank / per host: tokens with at least one expert there */
    for (int32_t r = 0; r < R; ++r) {
        rank_tokens[r] = 0;
        for (int32_t t = 0; t < T; ++t) {
            int hit = 0;
            for (int32_t j = 0; j < k; ++j)
                if (rank_of(idx[(int64_t)t * k + j], epr) == r)
                    hit = 1;
            rank_tokens[r] += hit;
        }
    }
    for (int32_t h = 0; h < H; ++h) {
        host_tokens[h] = 0;
        for (int32_t t = 0; t < T; ++t) {
            int hit = 0;
            for (int32_t j = 0; j < k; ++j)
                if (host_of(idx[(int64_t)t * k + j], epr, rph) == h)
                    hit = 1;
            host_tokens[h] += hit;
        }
    }

    /* exclusive prefix sums */
    expert_offset[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        expert_offset[e + 1] = expert_offset[e] + expert_count[e];
    for (int32_t r = 0; r <= R; ++r)
        rank_offset[r] = expert_offset[r * epr];
    host_offset[0] = 0;
    for (int32_t h = 0; h < H; ++h)
        host_offset[h + 1] = host_offset[h] + host_tokens[h];

    /* per-expert rows: walk pairs in (t, j) order; each expert's rows fill up
     * from its offset, so rows of one expert keep token order */
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!next)
        return ORC_ERR_ARG;
    for (int32_t e = 0; e < E; ++e)
        next[e] = expert_offset[e];
    for (int32_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = idx[(int64_t)t * k + j];
            int32_t row = next[e];
            next[e] += 1;
            slot[(int64_t)t * k + j] = row;
            row_token[row] = t;
        }
    free(next);

    /* relay rows: one per (token, host it touches), ordered by host then token */
    for (int32_t h = 0; h < H; ++h)
        relay_dst_rank[h] = h * rph + (s % rph);   /* the same-index GPU on host h */
    int32_t relay_rows = host_offset[H];
    if (relay) {
        const int64_t cap = (int64_t)T * (k < H ? k : H);
        for (int64_t i = 0; i < cap; ++i) {
            relay_token[i] = -1;
            fanout_rank_mask[i] = 0;
            for (int32_t j = 0; j < k; ++j)
                fanout_expert[i * k + j] = -1;
        }
        int32_t *next_h = (int32_t *)malloc(sizeof(int32_t) * (size_t)H);
        if (!next_h)
            return ORC_ERR_ARG;
        for (int32_t h = 0; h < H; ++h)
            next_h[h] = host_offset[h];
        for (int32_t t = 0; t < T; ++t)
            for (int32_t h = 0; h < H; ++h) {
                int hit = 0;
                for (int32_t j = 0; j < k; ++j)
                    if (host_of(idx[(int64_t)t * k + j], epr, rph) == h)
                        hit = 1;
                if (!hit) {
                    relay_slot[(int64_t)t * H + h] = -1;
                    continue;
                }
                int32_t row = next_h[h];
                next_h[h] += 1;
                relay_slot[(int64_t)t * H + h] = row;
                relay_token[row] = t;
                uint32_t mask = 0;
                for (int32_t j = 0; j < k; ++j) {
                    int32_t e = idx[(int64_t)t * k + j];
                    if (host_of(e, epr, rph) == h) {
                        fanout_expert[(int64_t)row * k + j] = e;
                        mask |= 1u << (rank_of(e, epr) % rph);
                    }
                }
                fanout_rank_mask[row] = mask;
            }
        free(next_h);
    }

    int32_t mx = 0;
    for (int32_t e = 0; e < E; ++e)
        if (expert_count[e] > mx)
            mx = expert_count[e];
    totals[0] = (int32_t)P;
    totals[1] = relay_rows;
    totals[2] = mx;
    totals[3] = 0;
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Dispatch                                                            */
/* ------------------------------------------------------------------ */

/* Destination rows of token t: the k per-expert rows, or the relay rows of
 * the hosts it touches (-1 where it touches none). */
static int32_t dest_row(int32_t relay, int32_t k, int32_t H, const int32_t *slot,
                        const int32_t *relay_slot, int32_t t, int32_t d)
{
    return relay ? relay_slot[(int64_t)t * H + d] : slot[(int64_t)t * k + d];
}

/* bf16 rows: recv[row, :] = x[t, :] for every destination row of t. */
int oracle_dispatch_bf16(int32_t T, int32_t k, int32_t H, int32_t relay, int32_t hidden,
                         const int32_t *slot, const int32_t *relay_slot,
                         const uint16_t *x, uint16_t *recv)
{
    if (T < 0 || k < 1 || H < 1 || hidden < 1)
        return ORC_ERR_ARG;
    const int32_t D = relay ? H : k;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t d = 0; d < D; ++d) {
            int32_t row = dest_row(relay, k, H, slot, relay_slot, t, d);
            if (row < 0)
                continue;
            for (int32_t c = 0; c < hidden; ++c)
                recv[(int64_t)row * hidden + c] = x[(int64_t)t * hidden + c];
        }
    return ORC_OK;
}

/* fp8 rows: per token and 128-channel block b, a = max |x|, scale s = a/448
 * (float32, correctly rounded), code = e4m3(x / s) (float32 quotient, then
 * saturating round-to-nearest-even). The token is quantised once; its codes
 * and scales are stored to every destination row. */
int oracle_dispatch_fp8(int32_t T, int32_t k, int32_t H, int32_t relay, int32_t hidden,
                        const int32_t *slot, const int32_t *relay_slot,
                        const uint16_t *x, uint8_t *recv_q, float *recv_scale)
{
    if (T < 0 || k < 1 || H < 1 || hidden < 128 || hidden % 128 != 0)
        return ORC_ERR_ARG;
    const int32_t nb = hidden / 128;
    const int32_t D = relay ? H : k;
    uint8_t *q = (uint8_t *)malloc((size_t)hidden);
    float *sc = (float *)malloc(sizeof(float) * (size_t)nb);
    if (!q || !sc) {
        free(q);
        free(sc);
        return ORC_ERR_ARG;
    }
    int status = ORC_OK;
    for (int32_t t = 0; t < T && status == ORC_OK; ++t) {
        for (int32_t b = 0; b < nb; ++b) {
            float a = 0.0f;
            for (int32_t c = b * 128; c < (b + 1) * 128; ++c) {
                float v = oracle_bf16_to_f32(x[(int64_t)t * hidden + c]);
                if (!isfinite(v))
                    status = ORC_ERR_VALUE;
                if (fabsf(v) > a)
                    a = fabsf(v);
            }
            float s = a / 448.0f;
            sc[b] = s;
            for (int32_t c = b * 128; c < (b + 1) * 128; ++c) {
                float v = oracle_bf16_to_f32(x[(int64_t)t * hidden + c]);
                if (a == 0.0f)
                    q[c] = signbit(v) ? 0x80 : 0x00;   /* all-zero block keeps the sign */
                else
                    q[c] = oracle_f32_to_e4m3(v / s);
            }
        }
        for (int32_t d = 0; d < D; ++d) {
            int32_t row = dest_row(relay, k, H, slot, relay_slot, t, d);
            if (row < 0)
                continue;
            for (int32_t c = 0; c < hidden; ++c)
                recv_q[(int64_t)row * hidden + c] = q[c];
            for (int32_t b = 0; b < nb; ++b)
                recv_scale[(int64_t)row * nb + b] = sc[b];
        }
    }
    free(q);
    free(sc);
    return status;
}

/* ------------------------------------------------------------------ */
/* Combine                                                             */
/* ------------------------------------------------------------------ */

/* out[t, c] = bf16( sum_j w[t,j] * y[slot[t,j], c] ), the sum taken in
 * float32 as acc = fmaf(w, y, acc) for j = 0..k-1 starting from +0. */
int oracle_combine(int32_t T, int32_t k, int32_t hidden, const int32_t *slot,
                   const float *w, const uint16_t *y, uint16_t *out)
{
    if (T < 0 || k < 1 || hidden < 1)
        return ORC_ERR_ARG;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t c = 0; c < hidden; ++c) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
                int32_t row = slot[(int64_t)t * k + j];
                float v = oracle_bf16_to_f32(y[(int64_t)row * hidden + c]);
                acc = fmaf(w[(int64_t)t * k + j], v, acc);
            }
            out[(int64_t)t * hidden + c] = oracle_f32_to_bf16(acc);
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Relay receive side and two-level combine                            */
/* ------------------------------------------------------------------ */
/*
 * Mode 2 of the digest (section 3.2, Figure 3): the relayed copy of a token
 * arrives once at the same-index GPU of each destination host and is fanned
 * out there to the token's experts on that host; on the way back that GPU
 * sums its experts' results before sending one partial back, and the source
 * sums the partials of the hosts.
 */

/* Fan-out of relay rows (row_bytes bytes each, plus nsc float32 scales when
 * nsc > 0): for every token t and host h with a relay row r, and every j
 * whose expert idx[t,j] sits on host h, per-expert row slot[t,j] = row r. */
int oracle_relay_fanout(int32_t T, int32_t k, int32_t E, int32_t R, int32_t H,
                        int64_t row_bytes, int32_t nsc, const int32_t *idx,
                        const int32_t *slot, const int32_t *relay_slot,
                        const uint8_t *relay_rows, const float *relay_scales,
                        uint8_t *recv, float *recv_scales)
{
    if (!geometry_ok(T, k, E, R, H, 0) || row_bytes < 1 || nsc < 0)
        return ORC_ERR_ARG;
    const int32_t epr = E / R, rph = R / H;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t h = 0; h < H; ++h) {
            int32_t r = relay_slot[(int64_t)t * H + h];
            if (r < 0)
                continue;
            for (int32_t j = 0; j < k; ++j) {
                int32_t e = idx[(int64_t)t * k + j];
                if (e < 0 || e >= E)
                    return ORC_ERR_INDEX;
                if (host_of(e, epr, rph) != h)
                    continue;
                int64_t dst = slot[(int64_t)t * k + j];
                for (int64_t b = 0; b < row_bytes; ++b)
                    recv[dst * row_bytes + b] = relay_rows[(int64_t)r * row_bytes + b];
                for (int32_t q = 0; q < nsc; ++q)
                    recv_scales[dst * nsc + q] = relay_scales[(int64_t)r * nsc + q];
            }
        }
    return ORC_OK;
}

/* Level 1 (relay GPU): for relay row r = (t, h), partial[r, c] = sum over j
 * ascending with host(idx[t,j]) == h of w[t,j] * y[slot[t,j], c], in float32
 * as acc = fmaf(w, y, acc) from +0. Stored as float32 (bf16_out == 0) or
 * rounded to bf16 (bf16_out != 0; partials then hold uint16 patterns). */
int oracle_relay_partials(int32_t T, int32_t k, int32_t E, int32_t R, int32_t H,
                          int32_t hidden, int32_t bf16_out, const int32_t *idx,
                          const int32_t *slot, const int32_t *relay_slot, const float *w,
                          const uint16_t *y, void *partials)
{
    if (!geometry_ok(T, k, E, R, H, 0) || hidden < 1)
        return ORC_ERR_ARG;
    const int32_t epr = E / R, rph = R / H;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t h = 0; h < H; ++h) {
            int32_t r = relay_slot[(int64_t)t * H + h];
            if (r < 0)
                continue;
            for (int32_t c = 0; c < hidden; ++c) {
                float acc = 0.0f;
                for (int32_t j = 0; j < k; ++j) {
                    int32_t e = idx[(int64_t)t * k + j];
                    if (host_of(e, epr, rph) != h)
                        continue;
                    int32_t row = slot[(int64_t)t * k + j];
                    acc = fmaf(w[(int64_t)t * k + j], oracle_bf16_to_f32(y[(int64_t)row * hidden + c]),
                               acc);
                }
                if (bf16_out)
                    ((uint16_t *)partials)[(int64_t)r * hidden + c] = oracle_f32_to_bf16(acc);
                else
                    ((float *)partials)[(int64_t)r * hidden + c] = acc;
            }
        }
    return ORC_OK;
}

/* Level 2 (source): out[t, c] = bf16( sum over h ascending of partial of
 * relay row relay_slot[t, h] (where it exists) ), float32 adds from +0. */
int oracle_relay_finish(int32_t T, int32_t H, int32_t hidden, int32_t bf16_in,
                        const int32_t *relay_slot, const void *partials, uint16_t *out)
{
    if (T < 0 || H < 1 || hidden < 1)
        return ORC_ERR_ARG;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t c = 0; c < hidden; ++c) {
            float acc = 0.0f;
            for (int32_t h = 0; h < H; ++h) {
                int32_t r = relay_slot[(int64_t)t * H + h];
                if (r < 0)
                    continue;
                float p = bf16_in ? oracle_bf16_to_f32(((const uint16_t *)partials)[(int64_t)r * hidden + c])
                                  : ((const float *)partials)[(int64_t)r * hidden + c];
                acc = acc + p;
            }
            out[(int64_t)t * hidden + c] = oracle_f32_to_bf16(acc);
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Expert groups (per-expert overlap)                                  */
/* ------------------------------------------------------------------ */
/*
 * Digest section 3.3 and Figure 4: the split is over experts, not over the
 * batch: m groups (2 or 4) in turn, each over the whole batch, so every
 * expert's weights are read once. Every GPU must have work in every group for the
 * overlap to exist, so group g holds, on every rank, the local experts i
 * (i = e mod epr) with i / (epr / m) == g.
 *
 * Rows: per-expert rows ordered by (group, expert id, token, j). Group g's
 * rows are then one contiguous range, and inside it each rank's rows are
 * contiguous: group_offset[g * R + r] is the first row of group g on rank r,
 * group_offset[m * R] the total. With m == 1 this is the plain layout.
 *
 * Combine: each group adds its experts' weighted outputs to the float32 sum
 * the earlier groups left, in ascending j inside the group; the result is
 * rounded to bf16 once, after the last group: acc = +0, then for g = 0..m-1,
 * for j ascending with group(idx[t, j]) == g, acc = fmaf(w[t, j], y, acc).
 */

static int32_t group_of(int32_t e, int32_t epr, int32_t m)
{
    return (e % epr) / (epr / m);
}

int oracle_layout_grouped(int32_t T, int32_t k, int32_t E, int32_t R, int32_t m,
                          const int32_t *idx, int32_t *expert_count, int32_t *expert_offset,
                          int32_t *group_offset, int32_t *slot, int32_t *row_token,
                          int32_t *totals)
{
    if (T < 0 || k < 1 || E < 1 || R < 1 || m < 1 || E % R != 0 || (E / R) % m != 0)
        return ORC_ERR_ARG;
    const int32_t epr = E / R, epg = epr / m;
    const int64_t P = (int64_t)T * k;
    int64_t bad = 0;
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] < 0 || idx[p] >= E)
            bad += 1;
    totals[0] = 0;
    totals[1] = 0;
    totals[2] = 0;
    totals[3] = (int32_t)bad;
    if (bad)
        return ORC_ERR_INDEX;

    for (int32_t e = 0; e < E; ++e)
        expert_count[e] = 0;
    for (int64_t p = 0; p < P; ++p)
        expert_count[idx[p]] += 1;

    /* experts in (group, expert id) order; prefix sums in that order */
    int32_t run = 0;
    for (int32_t g = 0; g < m; ++g)
        for (int32_t r = 0; r < R; ++r) {
            group_offset[g * R + r] = run;
            for (int32_t i = g * epg; i < (g + 1) * epg; ++i) {
                int32_t e = r * epr + i;
                expert_offset[e] = run;
                run += expert_count[e];
            }
        }
    group_offset[m * R] = run;
    expert_offset[E] = run;

    /* rows of each expert fill up from its offset in (t, j) order */
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!next)
        return ORC_ERR_ARG;
    for (int32_t e = 0; e < E; ++e)
        next[e] = expert_offset[e];
    for (int32_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = idx[(int64_t)t * k + j];
            slot[(int64_t)t * k + j] = next[e];
            row_token[next[e]] = t;
            next[e] += 1;
        }
    free(next);

    int32_t mx = 0;
    for (int32_t e = 0; e < E; ++e)
        if (expert_count[e] > mx)
            mx = expert_count[e];
    totals[0] = (int32_t)P;
    totals[2] = mx;
    return ORC_OK;
}

/* The destinations of group g's dispatch: slot[t, j] where expert idx[t, j]
 * is in group g, -1 elsewhere (a per-expert dispatch over these rows copies
 * exactly group g's rows). */
int oracle_group_slots(int32_t T, int32_t k, int32_t E, int32_t R, int32_t m, int32_t g,
                       const int32_t *idx, const int32_t *slot, int32_t *slot_g)
{
    if (T < 0 || k < 1 || E < 1 || R < 1 || m < 1 || E % R != 0 || (E / R) % m != 0 || g < 0 ||
        g >= m)
        return ORC_ERR_ARG;
    const int32_t epr = E / R;
    for (int64_t p = 0; p < (int64_t)T * k; ++p)
        slot_g[p] = group_of(idx[p], epr, m) == g ? slot[p] : -1;
    return ORC_OK;
}

int oracle_combine_grouped(int32_t T, int32_t k, int32_t E, int32_t R, int32_t m,
                           int32_t hidden, const int32_t *idx, const int32_t *slot,
                           const float *w, const uint16_t *y, uint16_t *out)
{
    if (T < 0 || k < 1 || E < 1 || R < 1 || m < 1 || E % R != 0 || (E / R) % m != 0 ||
        hidden < 1)
        return ORC_ERR_ARG;
    const int32_t epr = E / R;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t c = 0; c < hidden; ++c) {
            float acc = 0.0f;
            for (int32_t g = 0; g < m; ++g)
                for (int32_t j = 0; j < k; ++j) {
                    if (group_of(idx[(int64_t)t * k + j], epr, m) != g)
                        continue;
                    int32_t row = slot[(int64_t)t * k + j];
                    float wt = w[(int64_t)t * k + j];
                    float v = oracle_bf16_to_f32(y[(int64_t)row * hidden + c]);
                    acc = fmaf(wt, v, acc);
                }
            out[(int64_t)t * hidden + c] = oracle_f32_to_bf16(acc);
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Per-step intra-host expert swap planner                             */
/* ------------------------------------------------------------------ */
/*
 * Digest section 3.1 and Figure 2(b). Load of rank r = sum over its slots of
 * the experts' token counts. Per host: ranks sorted by load, descending;
 * the i-th of that order is paired with the (n-1-i)-th; each pair gets the
 * single expert exchange with the smallest new pair maximum, applied when
 * the maximum drops by at least tau tokens.
 *
 * Placement: slot_expert[r * epr + i] is the expert in slot i of rank r.
 * Ties: ranks are ordered by load descending, then rank index ascending;
 * among equally good swaps the one with the smaller slot of the heavier rank,
 * then the smaller slot of the lighter rank, wins. A swap must lower the
 * pair's maximum strictly and by at least tau to be applied.
 *
 * Outputs: slot_expert_out (the placement after the applied swaps), loads
 * per rank before and after, and per pair (host-major, pair index within the
 * host) 7 ints: heavy rank, its expert, light rank, its expert, old maximum,
 * new maximum, applied (0/1); -1 entries when a host has no such pair.
 */
int oracle_plan_swaps(int32_t E, int32_t R, int32_t H, const int32_t *count,
                      const int32_t *slot_expert_in, int32_t tau, int32_t *slot_expert_out,
                      int32_t *load_before, int32_t *load_after, int32_t *swaps,
                      int32_t *host_bad)
{
    if (E < 1 || R < 1 || H < 1 || E % R != 0 || R % H != 0 || tau < 0)
        return ORC_ERR_ARG;
    const int32_t epr = E / R, rph = R / H, npair = rph / 2;
    /* A host whose slots hold an expert id outside [0, E) is not planned: its
     * slots are copied, its loads and pair records are -1 (applied 0) and
     * host_bad[h] is the number of such ids (0 for a planned host). */
    for (int32_t h = 0; h < H; ++h) {
        int32_t nbad = 0;
        for (int32_t i = h * rph * epr; i < (h + 1) * rph * epr; ++i)
            if (slot_expert_in[i] < 0 || slot_expert_in[i] >= E)
                nbad += 1;
        host_bad[h] = nbad;
    }
    for (int32_t i = 0; i < E; ++i)
        slot_expert_out[i] = slot_expert_in[i];
    for (int32_t r = 0; r < R; ++r) {
        int64_t load = 0;
        if (host_bad[r / rph] != 0) {
            load_before[r] = -1;
            continue;
        }
        for (int32_t i = 0; i < epr; ++i)
            load += count[slot_expert_in[r * epr + i]];
        load_before[r] = (int32_t)load;
    }
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)(rph > 0 ? rph : 1));
    if (!order)
        return ORC_ERR_ARG;
    for (int32_t h = 0; h < H; ++h) {
        /* ranks of host h by load descending, rank ascending (insertion sort) */
        for (int32_t i = 0; i < rph; ++i) {
            int32_t r = h * rph + i, pos = i;
            while (pos > 0) {
                int32_t q = order[pos - 1];
                if (load_before[q] > load_before[r] || (load_before[q] == load_before[r] && q < r))
                    break;
                order[pos] = q;
                pos -= 1;
            }
            order[pos] = r;
        }
        if (host_bad[h] != 0) {
            for (int32_t p = 0; p < npair; ++p) {
                int32_t *rec = swaps + ((int64_t)h * npair + p) * 7;
                for (int32_t f = 0; f < 6; ++f)
                    rec[f] = -1;
                rec[6] = 0;
            }
            continue;
        }
        for (int32_t p = 0; p < npair; ++p) {
            int32_t A = order[p], B = order[rph - 1 - p];
            int32_t LA = load_before[A], LB = load_before[B];
            int32_t old_max = LA > LB ? LA : LB;
            int32_t best = -1, best_a = 0, best_b = 0;
            for (int32_t a = 0; a < epr; ++a)
                for (int32_t b = 0; b < epr; ++b) {
                    int32_t ca = count[slot_expert_in[A * epr + a]];
                    int32_t cb = count[slot_expert_in[B * epr + b]];
                    int32_t na = LA - ca + cb, nb = LB - cb + ca;
                    int32_t m = na > nb ? na : nb;
                    if (best < 0 || m < best) {   /* strict: the first (a, b) keeps ties */
                        best = m;
                        best_a = a;
                        best_b = b;
                    }
                }
            int32_t applied = (old_max - best > 0) && (old_max - best >= tau);
            int32_t *rec = swaps + ((int64_t)h * npair + p) * 7;
            rec[0] = A;
            rec[1] = slot_expert_in[A * epr + best_a];
            rec[2] = B;
            rec[3] = slot_expert_in[B * epr + best_b];
            rec[4] = old_max;
            rec[5] = best;
            rec[6] = applied;
            if (applied) {
                slot_expert_out[A * epr + best_a] = slot_expert_in[B * epr + best_b];
                slot_expert_out[B * epr + best_b] = slot_expert_in[A * epr + best_a];
            }
        }
    }
    free(order);
    for (int32_t r = 0; r < R; ++r) {
        int64_t load = 0;
        if (host_bad[r / rph] != 0) {
            load_after[r] = -1;
            continue;
        }
        for (int32_t i = 0; i < epr; ++i)
            load += count[slot_expert_out[r * epr + i]];
        load_after[r] = (int32_t)load;
    }
    return ORC_OK;
}
