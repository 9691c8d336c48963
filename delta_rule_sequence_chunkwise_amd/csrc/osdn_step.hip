// One recurrent OSDN decode step for every (b,h): the token step of the OSDN technical
// summary, section 2.1, with the gated-delta decay of Erase-then-Delta Attention, section
// 2.2, eq. 4, rearranged so the state is read once and written once:
//
//   y = M^T k,  z = M^T q                 (one pass over M, kept in registers)
//   u = beta (v - alpha y)                (pseudo-value: the gated residual)
//   M <- alpha M + k~ u^T                 (k~ = d (.) k), written back in place
//   o = M_new^T q = alpha z + <k~, q> u
//
// The step is bound by HBM bandwidth: M is dk*dv*4 bytes in and out per (b,h), everything
// else is a few hundred bytes.  One workgroup of 256 threads owns one (b,h); thread t holds
// four consecutive value columns (one 16-byte vector) of every (256/(dv/4))-th key row, so
// each wavefront moves whole contiguous rows per load.  The state is read and written with
// non-temporal accesses: in a model every layer's state streams through once per token, so
// none of it is worth keeping in the caches (measured at the decode shape with the state
// rotated over four buffers: 48.5 us per step against 56.7 us with ordinary accesses).
#include "osdn_internal.h"

namespace osdn {
namespace {

constexpr int kThreads = 256;

template <int DK, int DV, typename TQ, typename TD>
__global__ void __launch_bounds__(kThreads)
step_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k, const TQ *__restrict__ v,
            const TD *__restrict__ d, const float *__restrict__ beta,
            const float *__restrict__ alpha, float *__restrict__ S, TQ *__restrict__ o) {
    constexpr int TPR = DV / 4;          // threads per key row (one float4 each)
    constexpr int RG = kThreads / TPR;   // row groups
    constexpr int RPT = DK / RG;         // key rows per thread
    static_assert(RPT * RG == DK, "dk must be a multiple of the row-group count");

    __shared__ float sk[DK], sq[DK], skt[DK];
    __shared__ float4 sy[RG][TPR], sz[RG][TPR];
    __shared__ float s_ktq;

    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % TPR;  // column group: columns 4*cg .. 4*cg+3
    const int rg = tid / TPR;  // row group: rows rg, rg+RG, ...

    float4 *Mrow = reinterpret_cast<float4 *>(S + bh * DK * DV);
    float4 m[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) m[i] = load_stream(&Mrow[(rg + i * RG) * TPR + cg]);

    if (tid < DK) {
        const float kv = to_f32(k[bh * DK + tid]);
        const float qv = to_f32(q[bh * DK + tid]);
        sk[tid] = kv;
        sq[tid] = qv;
        skt[tid] = to_f32(d[bh * DK + tid]) * kv;
    }
    __syncthreads();

    if (tid < 64) {  // <k~, q>: wave 0 reduces over the key features
        float p = 0.f;
        for (int i = tid; i < DK; i += 64) p += skt[i] * sq[i];
        for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
        if (tid == 0) s_ktq = p;
    }

    float4 y = make_float4(0.f, 0.f, 0.f, 0.f), z = y;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kr = sk[rg + i * RG], qr = sq[rg + i * RG];
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
        const float4 a = sy[g][cg], b = sz[g][cg];
        y.x += a.x; y.y += a.y; y.z += a.z; y.w += a.w;
        z.x += b.x; z.y += b.y; z.z += b.z; z.w += b.w;
    }
    const float al = alpha ? alpha[bh] : 1.f;
    const float be = beta[bh];
    const TQ *vr = v + bh * DV + 4 * cg;
    float4 u;
    u.x = be * (to_f32(vr[0]) - al * y.x);
    u.y = be * (to_f32(vr[1]) - al * y.y);
    u.z = be * (to_f32(vr[2]) - al * y.z);
    u.w = be * (to_f32(vr[3]) - al * y.w);

    if (rg == 0) {
        const float c = s_ktq;
        TQ *orow = o + bh * DV + 4 * cg;
        orow[0] = from_f32<TQ>(al * z.x + c * u.x);
        orow[1] = from_f32<TQ>(al * z.y + c * u.y);
        orow[2] = from_f32<TQ>(al * z.z + c * u.z);
        orow[3] = from_f32<TQ>(al * z.w + c * u.w);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float w = skt[rg + i * RG];
        float4 mn;
        mn.x = al * m[i].x + w * u.x;
        mn.y = al * m[i].y + w * u.y;
        mn.z = al * m[i].z + w * u.z;
        mn.w = al * m[i].w + w * u.w;
        store_stream(&Mrow[(rg + i * RG) * TPR + cg], mn);
    }
}

template <int DK, int DV>
hipError_t launch_dims(const StepArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.BH));
#define OSDN_STEP_LAUNCH(TQ, TD)                                                              \
    hipLaunchKernelGGL((step_kernel<DK, DV, TQ, TD>), grid, dim3(kThreads), 0, stream,        \
                       static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),           \
                       static_cast<const TQ *>(a.v), static_cast<const TD *>(a.d), a.beta,   \
                       a.alpha, a.S, static_cast<TQ *>(a.o))
    if (a.qkv == OSDN_F32) {
        if (a.d_dtype == OSDN_F32) OSDN_STEP_LAUNCH(float, float);
        else OSDN_STEP_LAUNCH(float, bf16_t);
    } else {
        if (a.d_dtype == OSDN_F32) OSDN_STEP_LAUNCH(bf16_t, float);
        else OSDN_STEP_LAUNCH(bf16_t, bf16_t);
    }
#undef OSDN_STEP_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepArgs &a, hipStream_t stream) {
    if (a.dk == 64) return a.dv == 64 ? launch_dims<64, 64>(a, stream)
                                      : launch_dims<64, 128>(a, stream);
    return a.dv == 64 ? launch_dims<128, 64>(a, stream) : launch_dims<128, 128>(a, stream);
}

}  // namespace osdn
