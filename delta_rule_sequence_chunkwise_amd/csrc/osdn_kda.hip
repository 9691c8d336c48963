// Channel-wise (Kimi Delta Attention) gate for OSDN, gfx950: the per-token diagonal decay
// Diag(a_t) of Erase-then-Delta Attention, section 2.2, eq. 5 (section 3.2, eq. 7), with the
// OSDN write key k~ = d (.) k (OSDN technical summary, section 2.1):
//
//   M_t = Diag(a_t) M_{t-1} + b_t k~_t (v_t - (Diag(a_t) M_{t-1})^T k_t)^T ,   o_t = M_t^T q_t
//
// Chunkwise, the decay folds into the operands.  Inside a chunk let G_r = prod_{s<=r} a_s (per
// key feature, inclusive).  Unrolling the step gives M_r = Diag(G_r) M0 + sum_{s<=r}
// Diag(G_r / G_s) k~_s u_s^T, so with  q' = q G,  k' = k G,  d' = d / G^2  (hence
// k~' = d' k' = k~ / G) the chunk is the undecayed chunk algebra on (q', k', d'), except that
// the carried state becomes  Diag(G_C) (M0 + K~'^T U)  -- the forward kernels take G_C per
// chunk and scale the state's rows after each carry.  kda_prep_kernel writes q', k', d' and
// G_C into a workspace (one thread per four consecutive features of a chunk, 8- and 16-byte
// accesses); it is bound by HBM bandwidth.  G is clamped at 2^-60 inside 1/G^2,
// so a chunk whose product of gates on a feature falls below that is computed as if it were
// 2^-60 there.
//
// The decode step applies Diag(a) to the state's rows in place of the scalar gate.
#include "osdn_internal.h"
#include "osdn_mfma.h"

namespace osdn {
namespace {

constexpr float kMinGate = 0x1p-60f;

// four consecutive elements as fp32 (16 bytes of fp32, 8 bytes of bf16)
__device__ __forceinline__ float4 load4f(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 load4f(const bf16_t *p) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void store4f(float *p, float4 x) { *reinterpret_cast<float4 *>(p) = x; }
__device__ __forceinline__ void store4f(bf16_t *p, float4 x) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(
        uint32_t(f32_to_bf16_bits(x.x)) | (uint32_t(f32_to_bf16_bits(x.y)) << 16),
        uint32_t(f32_to_bf16_bits(x.z)) | (uint32_t(f32_to_bf16_bits(x.w)) << 16));
}

constexpr int kPrepThreads = 256;

// thread -> (sequence, chunk, four consecutive features); it walks the chunk's rows
template <int DK, typename TQ, typename TDI, typename TDO>
__global__ void __launch_bounds__(kPrepThreads)
kda_prep_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k, const TDI *__restrict__ d,
                const float *__restrict__ a, TQ *__restrict__ qp, TQ *__restrict__ kp,
                TDO *__restrict__ dp, float *__restrict__ gcs, int64_t T, int chunk,
                int64_t nchunks, int64_t total) {
    constexpr int QPR = DK / 4;  // feature quads per row
    const int64_t g = int64_t(blockIdx.x) * kPrepThreads + threadIdx.x;
    if (g >= total) return;
    const int64_t seg = g / QPR;  // (sequence, chunk)
    const int f = static_cast<int>(g % QPR) * 4;
    const int64_t bh = seg / nchunks, c = seg % nchunks;
    const int64_t t0 = c * chunk;
    const int n = static_cast<int>(T - t0 < chunk ? T - t0 : chunk);
    const int64_t base = (bh * T + t0) * DK + f;
    float4 G = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll 4
    for (int r = 0; r < n; ++r) {
        const int64_t i = base + int64_t(r) * DK;
        const float4 av = load4f(a + i), qv = load4f(q + i), kv = load4f(k + i), dv = load4f(d + i);
        G.x *= av.x; G.y *= av.y; G.z *= av.z; G.w *= av.w;
        store4f(qp + i, make_float4(qv.x * G.x, qv.y * G.y, qv.z * G.z, qv.w * G.w));
        store4f(kp + i, make_float4(kv.x * G.x, kv.y * G.y, kv.z * G.z, kv.w * G.w));
        const float gx = fmaxf(G.x, kMinGate), gy = fmaxf(G.y, kMinGate);
        const float gz = fmaxf(G.z, kMinGate), gw = fmaxf(G.w, kMinGate);
        store4f(dp + i, make_float4(dv.x / (gx * gx), dv.y / (gy * gy), dv.z / (gz * gz),
                                    dv.w / (gw * gw)));
    }
    store4f(gcs + seg * DK + f, G);
}

// one decode token with the channel-wise gate (same layout as step_kernel)
constexpr int kThreads = 256;

template <int DK, int DV, typename TQ, typename TD>
__global__ void __launch_bounds__(kThreads)
step_kda_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k, const TQ *__restrict__ v,
                const TD *__restrict__ d, const float *__restrict__ beta,
                const float *__restrict__ a, float *__restrict__ S, TQ *__restrict__ o) {
    constexpr int TPR = DV / 4;          // threads per key row (one float4 each)
    constexpr int RG = kThreads / TPR;   // row groups
    constexpr int RPT = DK / RG;         // key rows per thread
    static_assert(RPT * RG == DK, "dk must be a multiple of the row-group count");

    __shared__ float sak[DK], saq[DK], skt[DK], sq[DK], sa[DK];
    __shared__ float4 sy[RG][TPR], sz[RG][TPR];
    __shared__ float s_ktq;

    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % TPR, rg = tid / TPR;

    float4 *Mrow = reinterpret_cast<float4 *>(S + bh * DK * DV);
    float4 m[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) m[i] = Mrow[(rg + i * RG) * TPR + cg];

    if (tid < DK) {
        const float kv = to_f32(k[bh * DK + tid]), qv = to_f32(q[bh * DK + tid]);
        const float av = a[bh * DK + tid];
        sa[tid] = av;
        sak[tid] = av * kv;  // y = (Diag(a) M)^T k
        saq[tid] = av * qv;  // z = (Diag(a) M)^T q
        sq[tid] = qv;
        skt[tid] = to_f32(d[bh * DK + tid]) * kv;
    }
    __syncthreads();
    if (tid < 64) {  // <k~, q>
        float p = 0.f;
        for (int i = tid; i < DK; i += 64) p += skt[i] * sq[i];
        for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
        if (tid == 0) s_ktq = p;
    }
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f), z = y;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kr = sak[rg + i * RG], qr = saq[rg + i * RG];
        y.x += m[i].x * kr; y.y += m[i].y * kr; y.z += m[i].z * kr; y.w += m[i].w * kr;
        z.x += m[i].x * qr; z.y += m[i].y * qr; z.z += m[i].z * qr; z.w += m[i].w * qr;
    }
    sy[rg][cg] = y;
    sz[rg][cg] = z;
    __syncthreads();
    y = make_float4(0.f, 0.f, 0.f, 0.f);
    z = y;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const float4 p = sy[g][cg], r = sz[g][cg];
        y.x += p.x; y.y += p.y; y.z += p.z; y.w += p.w;
        z.x += r.x; z.y += r.y; z.z += r.z; z.w += r.w;
    }
    const float be = beta[bh];
    const TQ *vr = v + bh * DV + 4 * cg;
    float4 u;
    u.x = be * (to_f32(vr[0]) - y.x);
    u.y = be * (to_f32(vr[1]) - y.y);
    u.z = be * (to_f32(vr[2]) - y.z);
    u.w = be * (to_f32(vr[3]) - y.w);
    if (rg == 0) {  // o = (Diag(a) M)^T q + <k~, q> u
        const float c = s_ktq;
        TQ *orow = o + bh * DV + 4 * cg;
        orow[0] = from_f32<TQ>(z.x + c * u.x);
        orow[1] = from_f32<TQ>(z.y + c * u.y);
        orow[2] = from_f32<TQ>(z.z + c * u.z);
        orow[3] = from_f32<TQ>(z.w + c * u.w);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        const float ar = sa[row], w = skt[row];
        float4 mn;
        mn.x = ar * m[i].x + w * u.x;
        mn.y = ar * m[i].y + w * u.y;
        mn.z = ar * m[i].z + w * u.z;
        mn.w = ar * m[i].w + w * u.w;
        Mrow[row * TPR + cg] = mn;
    }
}

template <int DK, typename TQ, typename TDI, typename TDO>
hipError_t prep_typed(const KdaPrepArgs &a, hipStream_t stream) {
    const int64_t total = a.BH * a.nchunks * (DK / 4);
    const dim3 grid(static_cast<unsigned>((total + kPrepThreads - 1) / kPrepThreads));
    hipLaunchKernelGGL((kda_prep_kernel<DK, TQ, TDI, TDO>), grid, dim3(kPrepThreads), 0, stream,
                       static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),
                       static_cast<const TDI *>(a.d), a.alpha_ch, static_cast<TQ *>(a.qp),
                       static_cast<TQ *>(a.kp), static_cast<TDO *>(a.dp), a.gcs, a.T, a.chunk,
                       a.nchunks, total);
    return hipGetLastError();
}

template <int DK>
hipError_t prep_dk(const KdaPrepArgs &a, hipStream_t stream) {
    // bf16 operands: d' in bf16 (the forward rounds k~ to bf16 anyway); fp32: d' in fp32
    if (a.qkv == OSDN_BF16)
        return a.d_dtype == OSDN_F32 ? prep_typed<DK, bf16_t, float, bf16_t>(a, stream)
                                     : prep_typed<DK, bf16_t, bf16_t, bf16_t>(a, stream);
    return a.d_dtype == OSDN_F32 ? prep_typed<DK, float, float, float>(a, stream)
                                 : prep_typed<DK, float, bf16_t, float>(a, stream);
}

template <int DK, int DV>
hipError_t step_dims(const StepArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.BH));
#define OSDN_KDA_STEP(TQ, TD)                                                                 \
    hipLaunchKernelGGL((step_kda_kernel<DK, DV, TQ, TD>), grid, dim3(kThreads), 0, stream,    \
                       static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),           \
                       static_cast<const TQ *>(a.v), static_cast<const TD *>(a.d), a.beta,   \
                       a.alpha, a.S, static_cast<TQ *>(a.o))
    if (a.qkv == OSDN_F32) {
        if (a.d_dtype == OSDN_F32) OSDN_KDA_STEP(float, float);
        else OSDN_KDA_STEP(float, bf16_t);
    } else {
        if (a.d_dtype == OSDN_F32) OSDN_KDA_STEP(bf16_t, float);
        else OSDN_KDA_STEP(bf16_t, bf16_t);
    }
#undef OSDN_KDA_STEP
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kda_prep(const KdaPrepArgs &a, hipStream_t stream) {
    return a.dk == 64 ? prep_dk<64>(a, stream) : prep_dk<128>(a, stream);
}

hipError_t launch_step_kda(const StepArgs &a, hipStream_t stream) {
    if (a.dk == 64) return a.dv == 64 ? step_dims<64, 64>(a, stream) : step_dims<64, 128>(a, stream);
    return a.dv == 64 ? step_dims<128, 64>(a, stream) : step_dims<128, 128>(a, stream);
}

}  // namespace osdn
