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

// A decode step streams the whole state through once per token (in a model, every layer's state
// in turn), so its state accesses are non-temporal: they do not displace what the caches hold.
__device__ __forceinline__ float4 load_stream(const float4 *p) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
    return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void store_stream(float4 *p, float4 v) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f4 *>(p));
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
    const float *gcs = nullptr;  // channel-wise gate, [BH, nchunks, dk]: G_C, the product of
                                 // the chunk's gates, applied to the state's rows in the carry.
                                 // The matrix-core forward then takes q, k, d as the gate-scaled
                                 // q o G, k o G, k~ o (G_C / G) (bf16) and the chunk planes
    const uint16_t *planes = nullptr;  // [BH, nchunks, kda_planes::kElems] (matrix-core, gate)
    const float *alpha_ch = nullptr;   // fp32 forward: the channel-wise gate [BH, T, dk]
    void *ckpt = nullptr;        // [BH, nchunks, dk, dv]: the state at every chunk start, fp32
                                 // from the fp32 forward (either gate), bf16 from the
                                 // matrix-core forward (o may then be NULL: not written)
    void *uout = nullptr;        // with ckpt, matrix-core forward: the pseudo-values U of every
                                 // row, bf16 [BH, nchunks, dv/16, 64, 16] (NULL: not written)
    const float *gate_scores = nullptr;  // fp32 forward with the channel-wise gate, 32-row
                                         // chunks: the score tiles AS, P of every chunk as the
                                         // backward forms them, [BH, nchunks, 2, 32, 32]
                                         // (NULL: formed in the kernel)
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
                          // pass, bf16, [BH, nchunks, dv/16, 64, 16] each (rows_at)
    int64_t BH, T;
    int32_t dk, dv;
    osdn_dtype qkv, d_dtype;
    const float *alpha_ch = nullptr;  // the channel-wise gate [BH, T, dk] (its own backward)
    float *galpha_ch = nullptr;       // its gradient, [BH, T, dk] fp32 (NULL: not written)
    float *scores = nullptr;          // channel-wise gate: workspace for the score tiles AS and P
                                      // of every chunk, [BH, nchunks, 2, C, C] fp32
};

// The channel-wise gate's planes of one 64-row chunk (bf16 inputs): the chunk's score matrix P
// and the pieces of its UT transform, bf16, laid out exactly as the matrix-core forward keeps
// them in LDS, so that it copies them in unchanged.
namespace kda_planes {
constexpr int kRows = 64;
constexpr int kPPitch = kRows + 8;           // row pitch (bf16) of P
constexpr int kP = kRows * kPPitch;          // P: row-major, zero above the diagonal
constexpr int kDinv = 4 * 256;               // (I + A_ii)^{-1}, i = 0..3: 16 x 16 blocks
constexpr int kAneg = 6 * 256;               // -A_ik, (i, k) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
constexpr int kElems = kP + kDinv + kAneg;   // bf16 per chunk
// element (r, 4 g + e) of a 16 x 16 block: 8-byte granule g of row r sits at granule
// g ^ 2 ((r >> 3) & 1), so 16-lane reads of four-element granules touch distinct banks
__host__ __device__ constexpr int blk(int r, int g) { return r * 16 + 4 * (g ^ (((r >> 3) & 1) << 1)); }
}  // namespace kda_planes

struct KdaPrepArgs {
    const void *q, *k, *d;
    const float *alpha_ch, *beta;
    void *qp, *kp, *ktp;  // workspace [BH, T, dk] bf16: q o G, k o G, k~ o (G_C / G)
    uint16_t *planes;     // workspace [BH, nchunks, kda_planes::kElems] bf16
    float *gcs;           // workspace [BH, nchunks, dk]: G_C
    int64_t BH, T, nchunks;
    int32_t dk;
    osdn_dtype d_dtype;
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
hipError_t launch_kda_planes(const KdaPrepArgs &a, hipStream_t stream);
hipError_t launch_step_kda(const StepArgs &a, hipStream_t stream);  // alpha: [BH, dk]
hipError_t launch_chunk_bwd(const BwdArgs &a, hipStream_t stream);
// the backward with the channel-wise gate (alpha_ch set, alpha NULL): fp32 arithmetic, 32-row
// chunks, Mck and dMck fp32 [BH, nchunks, dk, dv] each, scores as above, Tck/Uck/dRck unused
hipError_t launch_chunk_bwd_gate(const BwdArgs &a, hipStream_t stream);
int32_t bwd_chunk_size(osdn_dtype qkv);  // rows per chunk of the backward

}  // namespace osdn
