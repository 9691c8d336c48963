// Chunkwise OSDN forward with fp32 arithmetic throughout (the OSDN_F32 path).
//
// One workgroup owns one (b,h) sequence and one BV-wide slice of the value columns: the
// state recurrence is separable over value columns (each column of M_t depends only on the
// same column of M_{t-1}), so slices never talk to each other.  The workgroup walks the
// chunks in order, keeping its dk x BV slice of the state in LDS, and per chunk of C rows
// (chunk algebra derived from the token step of the OSDN technical summary, section 2.1,
// with the gated-delta decay of Erase-then-Delta Attention, section 2.2, eq. 4):
//
//   a1  k~ = d (.) k;  g = running sum of ln(alpha) inside the chunk
//   a2  A[r][s] = beta_r e^{g_r - g_s} <k_r, k~_s>  for s < r          (chunk Gram matrix)
//   a3  T = (I + A)^{-1}, unit lower triangular                          (UT transform)
//   a4  R = diag(beta) (V - diag(e^g) K M);  U = T R                     (pseudo-values)
//   a5  P[r][s] = e^{g_r - g_s} <q_r, k~_s>  for s <= r                 (intra-chunk scores)
//   a6  O = diag(e^g) Q M + P U;  M <- e^{g_C} M + (diag(e^{g_C - g}) K~)^T U
//
// Rows past the end of the sequence are zero (beta = 0, alpha = 1), so they add nothing.
// For the backward the kernel can also record the state at every chunk start (and skip o).
// With the channel-wise gate the caller passes pre-scaled q, k, d and per-chunk factors G_C,
// and the state's rows are multiplied by G_C after each carry.
#include "osdn_internal.h"

namespace osdn {
namespace {

constexpr int kThreads = 256;

template <int DK, int BV, int CH, typename TQ, typename TD>
__global__ void __launch_bounds__(kThreads)
chunk_f32math_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k,
                     const TQ *__restrict__ v, const TD *__restrict__ d,
                     const float *__restrict__ beta, const float *__restrict__ alpha,
                     const float *S0, TQ *__restrict__ o, float *S_T, int64_t T, int dv,
                     const float *__restrict__ gcs, float *__restrict__ ckpt) {
    constexpr int PX = DK + 1;  // padded row pitches (bank-conflict relief)
    constexpr int PC = CH + 1;
    constexpr int PV = BV + 1;
    __shared__ float sX[CH * PX];   // K, later Q
    __shared__ float sKt[CH * PX];  // K~ = d (.) K
    __shared__ float sA[CH * PC];   // A, later P
    __shared__ float sT[CH * PC];   // T = (I + A)^{-1}
    __shared__ float sM[DK * PV];   // state slice M[:, j0:j0+BV]
    __shared__ float sR[CH * PV];   // V, then R
    __shared__ float sU[CH * PV];   // U
    __shared__ float sQM[CH * PV];  // Q M
    __shared__ float sg[CH];        // g (running log-decay)
    __shared__ float sb[CH];        // beta
    __shared__ float sgam[CH];      // e^{g_r}
    __shared__ float sdec[CH];      // e^{g_C - g_r}

    const int ntiles = dv / BV;
    const int64_t bh = blockIdx.x / ntiles;
    const int j0 = (blockIdx.x % ntiles) * BV;
    const int tid = threadIdx.x;

    for (int idx = tid; idx < DK * BV; idx += kThreads) {
        const int i = idx / BV, j = idx % BV;
        sM[i * PV + j] = S0 ? S0[(bh * DK + i) * dv + j0 + j] : 0.f;
    }

    for (int64_t c0 = 0; c0 < T; c0 += CH) {
        const int n = static_cast<int>(T - c0 < CH ? T - c0 : CH);
        const int64_t row0 = bh * T + c0;
        __syncthreads();  // the previous chunk is done with every buffer
        if (ckpt) {  // the state at this chunk's start, for the backward
            const int64_t cc = bh * ((T + CH - 1) / CH) + c0 / CH;
            for (int idx = tid; idx < DK * BV; idx += kThreads) {
                const int i = idx / BV, j = idx % BV;
                ckpt[(cc * DK + i) * dv + j0 + j] = sM[i * PV + j];
            }
        }

        // a1: keys, scaled keys, values, gates
        for (int idx = tid; idx < CH * DK; idx += kThreads) {
            const int r = idx / DK, i = idx % DK;
            float kv = 0.f, dd = 0.f;
            if (r < n) {
                kv = to_f32(k[(row0 + r) * DK + i]);
                dd = to_f32(d[(row0 + r) * DK + i]);
            }
            sX[r * PX + i] = kv;
            sKt[r * PX + i] = dd * kv;
        }
        for (int idx = tid; idx < CH * BV; idx += kThreads) {
            const int r = idx / BV, j = idx % BV;
            sR[r * PV + j] = r < n ? to_f32(v[(row0 + r) * dv + j0 + j]) : 0.f;
        }
        if (tid < CH) {
            sb[tid] = tid < n ? beta[row0 + tid] : 0.f;
            sg[tid] = (tid < n && alpha) ? logf(alpha[row0 + tid]) : 0.f;
        }
        __syncthreads();
        if (tid == 0) {
            float acc = 0.f;
            for (int r = 0; r < CH; ++r) {
                acc += sg[r];
                sg[r] = acc;
            }
        }
        __syncthreads();
        if (tid < CH) {
            sgam[tid] = __expf(sg[tid]);
            sdec[tid] = __expf(sg[CH - 1] - sg[tid]);
        }
        __syncthreads();

        // a2: strictly lower Gram matrix of (K, K~), gated and decayed
        for (int idx = tid; idx < CH * CH; idx += kThreads) {
            const int r = idx / CH, s = idx % CH;
            float val = 0.f;
            if (s < r) {
                float dot = 0.f;
                for (int i = 0; i < DK; ++i) dot += sX[r * PX + i] * sKt[s * PX + i];
                val = sb[r] * __expf(sg[r] - sg[s]) * dot;
            }
            sA[r * PC + s] = val;
        }
        __syncthreads();

        if (tid < CH) {
            // a3: column j of T by forward substitution, T[r][j] = delta_rj - sum A[r][s] T[s][j]
            const int j = tid;
            for (int r = 0; r < CH; ++r) {
                float val;
                if (r < j) {
                    val = 0.f;
                } else if (r == j) {
                    val = 1.f;
                } else {
                    float acc = 0.f;
                    for (int s = j; s < r; ++s) acc += sA[r * PC + s] * sT[s * PC + j];
                    val = -acc;
                }
                sT[r * PC + j] = val;
            }
        } else {
            // a4 (first half): R = diag(beta) (V - diag(e^g) K M)
            for (int idx = tid - CH; idx < CH * BV; idx += kThreads - CH) {
                const int r = idx / BV, j = idx % BV;
                float km = 0.f;
                for (int i = 0; i < DK; ++i) km += sX[r * PX + i] * sM[i * PV + j];
                sR[r * PV + j] = sb[r] * (sR[r * PV + j] - sgam[r] * km);
            }
        }
        __syncthreads();

        // a4 (second half): U = T R; meanwhile stage Q over K (K is no longer read)
        for (int idx = tid; idx < CH * BV; idx += kThreads) {
            const int r = idx / BV, j = idx % BV;
            float acc = 0.f;
            for (int s = 0; s <= r; ++s) acc += sT[r * PC + s] * sR[s * PV + j];
            sU[r * PV + j] = acc;
        }
        for (int idx = tid; idx < CH * DK; idx += kThreads) {
            const int r = idx / DK, i = idx % DK;
            sX[r * PX + i] = r < n ? to_f32(q[(row0 + r) * DK + i]) : 0.f;
        }
        __syncthreads();

        // a5: P = lower-inclusive (Q K~^T) with decay;  Q M for the inter-chunk read-out
        for (int idx = tid; idx < CH * CH; idx += kThreads) {
            const int r = idx / CH, s = idx % CH;
            float val = 0.f;
            if (s <= r) {
                float dot = 0.f;
                for (int i = 0; i < DK; ++i) dot += sX[r * PX + i] * sKt[s * PX + i];
                val = __expf(sg[r] - sg[s]) * dot;
            }
            sA[r * PC + s] = val;
        }
        for (int idx = tid; idx < CH * BV; idx += kThreads) {
            const int r = idx / BV, j = idx % BV;
            float qm = 0.f;
            for (int i = 0; i < DK; ++i) qm += sX[r * PX + i] * sM[i * PV + j];
            sQM[r * PV + j] = qm;
        }
        __syncthreads();

        // a6: outputs of this chunk and the state carried to the next one
        for (int idx = tid; idx < CH * BV; idx += kThreads) {
            const int r = idx / BV, j = idx % BV;
            if (o && r < n) {
                float acc = sgam[r] * sQM[r * PV + j];
                for (int s = 0; s <= r; ++s) acc += sA[r * PC + s] * sU[s * PV + j];
                o[(row0 + r) * dv + j0 + j] = from_f32<TQ>(acc);
            }
        }
        const float gam_last = sgam[CH - 1];
        for (int idx = tid; idx < DK * BV; idx += kThreads) {
            const int i = idx / BV, j = idx % BV;
            float acc = 0.f;
            for (int s = 0; s < CH; ++s)
                acc += sdec[s] * sKt[s * PX + i] * sU[s * PV + j];
            const float mv = gam_last * sM[i * PV + j] + acc;
            // channel-wise gate: the state's rows times the chunk's G_C
            sM[i * PV + j] = gcs ? gcs[(bh * ((T + CH - 1) / CH) + c0 / CH) * DK + i] * mv : mv;
        }
    }
    __syncthreads();
    if (S_T) {
        for (int idx = tid; idx < DK * BV; idx += kThreads) {
            const int i = idx / BV, j = idx % BV;
            S_T[(bh * DK + i) * dv + j0 + j] = sM[i * PV + j];
        }
    }
}

template <int DK, int CH, typename TQ, typename TD>
hipError_t launch_typed(const ChunkArgs &a, hipStream_t stream) {
    constexpr int BV = 32;
    const int ntiles = a.dv / BV;
    const dim3 grid(static_cast<unsigned>(a.BH * ntiles));
    hipLaunchKernelGGL((chunk_f32math_kernel<DK, BV, CH, TQ, TD>), grid, dim3(kThreads), 0,
                       stream, static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),
                       static_cast<const TQ *>(a.v), static_cast<const TD *>(a.d), a.beta,
                       a.alpha, a.S0, static_cast<TQ *>(a.o), a.S_T, a.T, a.dv, a.gcs,
                       static_cast<float *>(a.ckpt));
    return hipGetLastError();
}

template <int DK, int CH>
hipError_t launch_dtypes(const ChunkArgs &a, hipStream_t stream) {
    if (a.qkv == OSDN_F32)
        return a.d_dtype == OSDN_F32 ? launch_typed<DK, CH, float, float>(a, stream)
                                     : launch_typed<DK, CH, float, bf16_t>(a, stream);
    return a.d_dtype == OSDN_F32 ? launch_typed<DK, CH, bf16_t, float>(a, stream)
                                 : launch_typed<DK, CH, bf16_t, bf16_t>(a, stream);
}

template <int DK>
hipError_t launch_chunk(const ChunkArgs &a, hipStream_t stream) {
    switch (a.chunk) {
        case 16: return launch_dtypes<DK, 16>(a, stream);
        case 32: return launch_dtypes<DK, 32>(a, stream);
        default: return launch_dtypes<DK, 64>(a, stream);
    }
}

}  // namespace

hipError_t launch_chunk_fwd_f32math(const ChunkArgs &a, hipStream_t stream) {
    return a.dk == 64 ? launch_chunk<64>(a, stream) : launch_chunk<128>(a, stream);
}

}  // namespace osdn
