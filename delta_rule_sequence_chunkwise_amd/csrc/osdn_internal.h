// Internal declarations shared by the libosdn host layer and its HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "osdn.h"

namespace osdn {

// ---- element access -------------------------------------------------------------------------
// bf16 is carried as its 16 raw bits.  Widening is exact; narrowing rounds to nearest even.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))  // NaN: keep it quiet
        return static_cast<uint16_t>((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    return bf16_t{f32_to_bf16_bits(x)};
}

// ---- launch arguments -----------------------------------------------------------------------
struct ChunkArgs {
    const void *q, *k, *v, *d;
    const float *beta, *alpha, *S0;
    void *o;
    float *S_T;
    int64_t BH, T;
    int32_t dk, dv, chunk;
    osdn_dtype qkv, d_dtype;
    const float *gcs = nullptr;  // [BH, nchunks, dk]: per-feature factor applied to the
                                 // state's rows after each chunk's carry (channel-wise gate)
    void *ckpt = nullptr;        // [BH, nchunks, dk, dv]: the state at every chunk start, fp32
                                 // from the fp32 forward, bf16 from the matrix-core forward
                                 // (o may then be NULL: not written; no channel gate)
    void *uout = nullptr;        // with ckpt, matrix-core forward: [BH, T, dv] bf16, the
                                 // pseudo-values U of every row (NULL: not written)
};

struct BwdArgs {
    const void *q, *k, *v, *d;
    const float *beta, *alpha, *S0;
    const void *dO;
    const float *dS_T;
    void *gq, *gk, *gv;   // qkv dtype
    float *gbeta, *galpha;
    void *gd;             // d dtype
    float *dS0;
    void *Mck, *dMck;     // [BH, nchunks, dk, dv] each, bf16 for bf16 inputs (the precision
                          // the matrix products take them in), else fp32: the workspace's, or
                          // for Mck the caller's states from the forward (states_given)
    bool states_given;    // Mck holds the forward's states: no recompute
    uint16_t *Tck;        // workspace (bf16 inputs), per chunk (bf16, row-major): the planes
                          // hi = bf16(T) and lo = bf16(T - hi) of T = (I + A)^{-1} and the
                          // scores P (64 x 64 each; P zero above the diagonal), then
                          // K~ = d (.) k (64 x dk; zero past the end)
    uint16_t *Uck, *dRck; // workspace (bf16 inputs): U from the forward and dR from the reverse
                          // pass, [BH, T, dv] bf16 each
    int64_t BH, T;
    int32_t dk, dv;
    osdn_dtype qkv, d_dtype;
};

struct KdaPrepArgs {
    const void *q, *k, *d;
    const float *alpha_ch;
    void *qp, *kp, *dp;  // workspace: q', k' (qkv dtype), d' (bf16 for OSDN_BF16, else fp32)
    float *gcs;          // workspace: [BH, nchunks, dk]
    int64_t BH, T, nchunks;
    int32_t dk, chunk;
    osdn_dtype qkv, d_dtype;
};

struct StepArgs {
    const void *q, *k, *v, *d;
    const float *beta, *alpha;
    float *S;
    void *o;
    int64_t BH;
    int32_t dk, dv;
    osdn_dtype qkv, d_dtype;
};

struct PrecondArgs {
    const void *k;
    const float *beta, *r, *d1;
    float eta;
    void *d;          // [BH, T, dk] output, may be NULL for the serial kernel only
    float *d_next;
    int64_t BH, T;
    int32_t dk, chunk;  // chunk 1: token-serial kernel; 64: chunked kernel (bf16 keys)
    osdn_dtype k_dtype, d_dtype;
};

// Each launcher enqueues its kernels on `stream` and returns the HIP error of the launch.
// Arguments were validated by the host layer.
hipError_t launch_chunk_fwd_f32math(const ChunkArgs &a, hipStream_t stream);
hipError_t launch_chunk_fwd_mfma(const ChunkArgs &a, hipStream_t stream);
hipError_t launch_step(const StepArgs &a, hipStream_t stream);
hipError_t launch_precond(const PrecondArgs &a, hipStream_t stream);
hipError_t launch_kda_prep(const KdaPrepArgs &a, hipStream_t stream);
hipError_t launch_step_kda(const StepArgs &a, hipStream_t stream);  // alpha: [BH, dk]
hipError_t launch_chunk_bwd(const BwdArgs &a, hipStream_t stream);
int32_t bwd_chunk_size(osdn_dtype qkv);  // rows per chunk of the backward

}  // namespace osdn
