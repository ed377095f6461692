// epx_internal.h -- definitions shared by the HIP translation units of libepx.
// Not installed; the public interface is include/epx.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epx.h"

namespace epx {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kChunkTokens = 64;     // tokens per layout workgroup (one per lane in the relay pass)
constexpr int kMaxExperts = 2048;
constexpr int kMaxTopk = 64;
constexpr int kMaxHosts = 64;
constexpr int kMaxRanksPerHost = 32;
constexpr int kFp8Block = 128;       // channels per fp8 scale

// Problem geometry, validated on the host and passed by value to kernels.
struct Geometry {
    int32_t T, k, E, R, H, s;
    int32_t epr;     // experts per rank
    int32_t rph;     // ranks per host
    int32_t G;       // layout workgroups = max(1, ceil(T / kChunkTokens))
    int32_t nbits;   // bits that distinguish expert ids (ceil(log2 E))
    int32_t relay;   // HOST_RELAY mode
};

// 16-byte and 8-byte native vectors (global_load/store_dwordx4, dwordx2).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Launchers (each returns the launch status).
hipError_t launch_layout(const Geometry &g, const int32_t *idx, const epx_layout &L,
                         hipStream_t stream);
hipError_t launch_dispatch_bf16(const Geometry &g, const epx_layout &L, const void *x,
                                int32_t hidden, void *recv, hipStream_t stream);
hipError_t launch_dispatch_fp8(const Geometry &g, const epx_layout &L, const void *x,
                               int32_t hidden, void *recv, float *scales, hipStream_t stream);
hipError_t launch_combine(const Geometry &g, const epx_layout &L, const void *y,
                          const float *w, int32_t hidden, void *out, hipStream_t stream);
hipError_t launch_f32_to_e4m3(const float *in, uint8_t *out, int64_t n, hipStream_t stream);

}  // namespace epx
