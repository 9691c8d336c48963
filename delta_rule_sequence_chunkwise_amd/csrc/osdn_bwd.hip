// Backward of the chunkwise OSDN forward, gfx950: the gradients of q, k, v, beta, d, alpha and
// the initial state for given gradients of o and of the final state.
//
// The pages give no backward pass.  The chunk form used here is derived by differentiating the
// chunk algebra of the forward (itself derived from the token step of the OSDN technical
// summary, section 2.1, with the gated-delta decay of Erase-then-Delta Attention, section 2.2,
// eq. 4).  Per chunk of C rows, with M0 the state at its start, dMC the gradient with respect
// to the state at its end, L its last row, and A, P, U, g, gam = e^g, w = e^{g_L - g} and
// G[r,s] = e^{g_r - g_s} as in the forward (A = b_r AS with AS the strictly lower, decayed
// K K~^T):
//
//   dU  = P^T dO + diag(w) K~ dMC               dR = (I + A)^{-T} dU
//   dM0 = gam_L dMC + Q^T diag(gam) dO - K^T diag(gam b) dR
//   dP  = lower-inclusive(dO U^T)               dA = -strictly-lower(dR U^T)
//   dQ  = diag(gam) dO M0^T + (dP o G) K~
//   dK  = -diag(gam b) dR M0^T + Gb K~          Gb = dA o G, row r scaled by b_r
//   dK~ = diag(w) U dMC^T + (dP o G)^T Q + Gb^T K
//   dV  = diag(b) dR
//   db_r = <dR_r, v_r - gam_r (K M0)_r> + sum_s dA[r,s] AS[r,s]
//   dg_r = gam_r <dO_r, (Q M0)_r> - b_r gam_r <dR_r, (K M0)_r> - w_r <(K~ dMC)_r, U_r>
//          + (row sum - column sum)_r of (dP o P + dA o A)
//          + [r = L] (gam_L <dMC, M0> + sum_s w_s <(K~ dMC)_s, U_s>)
//   d ln a_t = sum_{t <= r <= L} dg_r,   da = d ln a / a
//   dd  = dK~ o K,   dK += dK~ o D
//
// Launches on the caller's stream: (1) the forward (the bf16 matrix-core kernel for bf16
// inputs, the fp32 one for fp32 inputs) records M0 of every chunk into the workspace, and for
// bf16 inputs U of every row; (2) for bf16 inputs, bwd_tinv_kernel inverts every chunk's I + A
// in parallel into the workspace (T does not depend on the state), with P and K~; (3) the
// reverse pass walks the chunks backwards per (sequence, value slice) carrying dM, records dMC
// of every chunk (and for bf16 inputs dR and dV of every row) and writes the initial-state
// gradient; (4) the per-chunk pass computes every other gradient of a chunk's rows from M0,
// dMC and, for bf16 inputs, U and dR (for fp32 inputs it forms U and dR itself by triangular
// solves; one workgroup per chunk, or for bf16 inputs persistent workgroups taking every
// grid-th chunk).  For fp32 inputs (2) is skipped and (3), (4) are fp32 on the vector ALUs (bwd_state_kernel, bwd_chunk_kernel): tile products
// are register-blocked (each of the 256 threads owns one (M/16) x (N/16) block of every M x N
// product), the triangular solves run column-parallel with the partial sums of one column
// reduced across adjacent lanes.  For bf16 inputs they run on matrix cores
// (bwd_state_mfma_kernel, bwd_chunk_mfma_kernel).  Rows past the end of the sequence are zero
// (beta = 0, alpha = 1, dO = 0), so they add nothing.
#include <type_traits>

#include "osdn_internal.h"
#include "osdn_mfma.h"

namespace osdn {
namespace {

constexpr int NT = 256;  // threads per workgroup
// tiles per chunk in the channel-gate score workspace: AS, P and T = (I + diag(beta) AS)^{-1}
constexpr int kGateTiles = 3;

// fp32 16x16x4 on the matrix cores: lane (g, i) = (lane / 16, lane % 16) gives A[i][g] and
// B[g][i]; the result's lane (g, j) holds rows 4g .. 4g + 3 of column j, as in the bf16 forms.
// Its four products are added in k order, fused, so a product split 4 k at a time this way sums
// in the same order as a plain multiply-add loop over k.
__device__ __forceinline__ v4f mfma4f(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// acc[m][n] += sum_{kk < K} a(i0 + m, kk) * b(kk, j0 + n), unrolled deep: these kernels run one
// wave per SIMD, so only a wave's own independent reads hide the LDS latency
template <int TM, int TN, int K, typename FA, typename FB>
__device__ __forceinline__ void mm(float (&acc)[TM][TN], int i0, int j0, FA &&a, FB &&b) {
#pragma unroll 16
    for (int kk = 0; kk < K; ++kk) {
        float av[TM], bv[TN];
#pragma unroll
        for (int m = 0; m < TM; ++m) av[m] = a(i0 + m, kk);
#pragma unroll
        for (int n = 0; n < TN; ++n) bv[n] = b(kk, j0 + n);
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int n = 0; n < TN; ++n) acc[m][n] += av[m] * bv[n];
    }
}

template <int TM, int TN>
__device__ __forceinline__ void zero(float (&acc)[TM][TN]) {
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n) acc[m][n] = 0.f;
}

// X[r][j] -= b_r sum_{s<r} AS[r][s] X[s][j] for every row r in order, columns j < NC, in place
// (X = (I + A)^{-1} X with A = diag(b) AS).  Column j is owned by TPC adjacent lanes; lane sub
// keeps rows s = i TPC + sub of it in registers, and each row's sum is reduced across the TPC
// lanes on DPP (a shuffle through LDS per reduction step measured several times slower).
template <int C, int NC, int PX, int PA>
__device__ __forceinline__ void solve_lower(float *X, const float *AS, const float *b, int tid) {
    constexpr int TPC = NT / NC, RPT = C / TPC;
    static_assert(TPC * NC == NT && RPT * TPC == C && TPC <= 16, "solve layout");
    const int j = tid / TPC, sub = tid % TPC;
    float rhs[C], mine[RPT];
#pragma unroll
    for (int r = 0; r < C; ++r) rhs[r] = X[r * PX + j];
#pragma unroll
    for (int i = 0; i < RPT; ++i) mine[i] = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            if (i * TPC < r) {
                const int s = i * TPC + sub;
                if (s < r) part += AS[r * PA + s] * mine[i];
            }
        }
        part = group_sum<TPC>(part);
        const float val = rhs[r] - b[r] * part;
        if (r % TPC == sub) mine[r / TPC] = val;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) X[(i * TPC + sub) * PX + j] = mine[i];
}

// X[r][j] -= sum_{s>r} b_s AS[s][r] X[s][j] for rows r = C-1 .. 0, in place
// (X = (I + A)^{-T} X); the same layout
template <int C, int NC, int PX, int PA>
__device__ __forceinline__ void solve_upper(float *X, const float *AS, const float *b, int tid) {
    constexpr int TPC = NT / NC, RPT = C / TPC;
    static_assert(TPC * NC == NT && RPT * TPC == C && TPC <= 16, "solve layout");
    const int j = tid / TPC, sub = tid % TPC;
    float rhs[C], mine[RPT];
#pragma unroll
    for (int r = 0; r < C; ++r) rhs[r] = X[r * PX + j];
#pragma unroll
    for (int i = 0; i < RPT; ++i) mine[i] = 0.f;
#pragma unroll
    for (int r = C - 1; r >= 0; --r) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            if (i * TPC + TPC - 1 > r) {
                const int s = i * TPC + sub;
                if (s > r) part += b[s] * AS[s * PA + r] * mine[i];
            }
        }
        part = group_sum<TPC>(part);
        const float val = rhs[r] - part;
        if (r % TPC == sub) mine[r / TPC] = val;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) X[(i * TPC + sub) * PX + j] = mine[i];
}

// g = running sum of ln(alpha) over the chunk's rows (0 past the end), gam = e^g,
// w = e^{g_last - g}; beta (0 past the end).  One wave's work (several may write the same values).
template <int C>
__device__ __forceinline__ void decay_scan_of(float bv, float av, bool has_alpha, int n, float *sb,
                                              float *sg, float *sgam, float *sw, int lane) {
    const float x = wave_prefix((lane < n && has_alpha) ? logf(av) : 0.f);
    const float gl = lane_value(x, C - 1);
    if (lane < C) {
        sb[lane] = lane < n ? bv : 0.f;
        sg[lane] = x;
        sgam[lane] = __expf(x);
        sw[lane] = __expf(gl - x);
    }
}
// the same with the chunk's beta, alpha loaded here (rows past the end repeat the last one)
template <int C>
__device__ __forceinline__ void decay_scan(const float *beta, const float *alpha, int64_t row0,
                                           int n, float *sb, float *sg, float *sgam, float *sw,
                                           int lane) {
    const int r = lane < n ? lane : n - 1;
    decay_scan_of<C>(beta[row0 + r], alpha ? alpha[row0 + r] : 1.f, alpha != nullptr, n, sb, sg,
                     sgam, sw, lane);
}

// eight consecutive values of d as fp32 (32 bytes of fp32 or 16 bytes of bf16)
__device__ __forceinline__ void load8(const float *p, float (&out)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t *p, float (&out)[8]) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        out[2 * e] = __uint_as_float(w[e] << 16);
        out[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

// Q and K of the chunk in their input type, K~ = d (.) k in fp32 (zero rows past the end)
template <int C, int DK, int PQ, int PX, typename TQ, typename TD>
__device__ __forceinline__ void load_qk(const TQ *q, const TQ *k, const TD *d, int64_t row0, int n,
                                        TQ *sQ, TQ *sK, float *sKt, int tid) {
    for (int idx = tid; idx < C * DK; idx += NT) {
        const int r = idx / DK, f = idx % DK;
        TQ qv = from_f32<TQ>(0.f), kv = from_f32<TQ>(0.f);
        float dv = 0.f;
        if (r < n) {
            qv = q[(row0 + r) * DK + f];
            kv = k[(row0 + r) * DK + f];
            dv = to_f32(d[(row0 + r) * DK + f]);
        }
        sQ[r * PQ + f] = qv;
        sK[r * PQ + f] = kv;
        sKt[r * PX + f] = dv * to_f32(kv);
    }
}

// AS = strictly lower (K K~^T) o G and P = lower-inclusive (Q K~^T) o G
template <int C, int DK, int PQ, int PX, int PC, typename TQ>
__device__ __forceinline__ void scores(const TQ *sQ, const TQ *sK, const float *sKt,
                                       const float *sg, float *sAS, float *sP, int tid) {
    constexpr int TM = C / 16;
    const int i0 = (tid / 16) * TM, j0 = (tid % 16) * TM;
    float ak[TM][TM], aq[TM][TM];
    zero(ak);
    zero(aq);
    auto bkt = [&](int kk, int j) { return sKt[j * PX + kk]; };
    mm<TM, TM, DK>(ak, i0, j0, [&](int i, int kk) { return to_f32(sK[i * PQ + kk]); }, bkt);
    mm<TM, TM, DK>(aq, i0, j0, [&](int i, int kk) { return to_f32(sQ[i * PQ + kk]); }, bkt);
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int nn = 0; nn < TM; ++nn) {
            const int i = i0 + m, j = j0 + nn;
            const float G = j <= i ? __expf(sg[i] - sg[j]) : 0.f;
            sAS[i * PC + j] = j < i ? ak[m][nn] * G : 0.f;
            sP[i * PC + j] = aq[m][nn] * G;
        }
}

// T = (I + A)^{-1} for C = 64, A = diag(b) AS strictly lower, by 16-row blocks: the diagonal
// blocks D_i = (I + A_ii)^{-1} by forward substitution (four adjacent lanes per column), then
// the blocks below the diagonal level by level, T_ij = -D_i sum_{j<=k<i} A_ik T_kj, in fp32.
// tmp holds 3 x 16 x 17 floats.  Ends with a barrier.
template <int PC>
__device__ __forceinline__ void block_inverse64(float *sT, const float *sAS, const float *sb,
                                                float *tmp, int tid) {
    constexpr int C = 64;
    for (int idx = tid; idx < C * C; idx += NT) sT[(idx / C) * PC + idx % C] = 0.f;
    __syncthreads();
    {
        const int blk = tid >> 6, jj = (tid >> 2) & 15, sub = tid & 3, rb = 16 * blk;
        float mine[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (4 * i < r) {
                    const int s2 = 4 * i + sub;
                    if (s2 < r) part += sAS[(rb + r) * PC + rb + s2] * mine[i];
                }
            }
            part = group_sum<4>(part);  // the four lanes of the column, on DPP
            const float val = (r == jj ? 1.f : 0.f) - sb[rb + r] * part;
            if (r % 4 == sub) mine[r / 4] = val;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[(rb + 4 * i + sub) * PC + rb + jj] = mine[i];
    }
    __syncthreads();
    static_for<1, 4>([&](auto LV) __attribute__((always_inline)) {  // blocks (i, j = i - lv)
        constexpr int lv = decltype(LV)::value, np = 4 - lv;
        for (int idx = tid; idx < np * 256; idx += NT) {  // W = sum_k A_ik T_kj
            const int pr = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
            const int i = pr + lv, j = pr;
            const float *arow = sAS + (16 * i + r) * PC + 16 * j;
            const float *tcol = sT + 16 * j * PC + 16 * j + cc;
            float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 16 * lv; s2 += 4) {
                w0 += arow[s2] * tcol[s2 * PC];
                w1 += arow[s2 + 1] * tcol[(s2 + 1) * PC];
                w2 += arow[s2 + 2] * tcol[(s2 + 2) * PC];
                w3 += arow[s2 + 3] * tcol[(s2 + 3) * PC];
            }
            tmp[(pr * 16 + r) * 17 + cc] = sb[16 * i + r] * ((w0 + w1) + (w2 + w3));
        }
        __syncthreads();
        for (int idx = tid; idx < np * 256; idx += NT) {  // T_ij = -D_i W (D_i lower)
            const int pr = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
            const int i = pr + lv, j = pr;
            const float *drow = sT + (16 * i + r) * PC + 16 * i;
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int r2 = 0; r2 < 16; r2 += 2) {
                a0 += (r2 <= r ? drow[r2] : 0.f) * tmp[(pr * 16 + r2) * 17 + cc];
                a1 += (r2 + 1 <= r ? drow[r2 + 1] : 0.f) * tmp[(pr * 16 + r2 + 1) * 17 + cc];
            }
            sT[(16 * i + r) * PC + 16 * j + cc] = -(a0 + a1);
        }
        __syncthreads();
    });
}

// Fixed-order sum over the workgroup (every thread passes its part; every thread gets the sum)
__device__ __forceinline__ float block_sum(float x, float *scratch4, int tid) {
    x = sum_rows(group_sum<16>(x));  // over the wave, on DPP
    __syncthreads();
    if ((tid & 63) == 0) scratch4[tid >> 6] = x;
    __syncthreads();
    return scratch4[0] + scratch4[1] + scratch4[2] + scratch4[3];
}

// ---- reverse pass over chunks: the state gradient ------------------------------------------
// One workgroup per (sequence, BV-wide value slice); dM[:, slice] stays in LDS.  dMck[c] gets
// the gradient with respect to the state at the end of chunk c; dS0 the one at the start.
template <int C, int DK, int BV, typename TQ, typename TD>
__global__ void __launch_bounds__(NT)
bwd_state_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k, const TD *__restrict__ d,
                 const float *__restrict__ beta, const float *__restrict__ alpha,
                 const TQ *__restrict__ dO, const float *__restrict__ dS_T,
                 float *__restrict__ dMck, float *__restrict__ dS0, int64_t T, int dv) {
    constexpr int PQ = DK + (sizeof(TQ) == 2 ? 2 : 1);
    constexpr int PX = DK + 1, PC = C + 1, PS = BV + 1;
    __shared__ TQ sQ[C * PQ], sK[C * PQ];
    __shared__ float sKt[C * PX], sAS[C * PC], sP[C * PC];
    __shared__ float sdO[C * PS], sX[C * PS], sdM[DK * PS];
    __shared__ float sb[C], sg[C], sgam[C], sw[C];

    const int nvt = dv / BV;
    const int64_t bh = blockIdx.x / nvt;
    const int j0 = static_cast<int>(blockIdx.x % nvt) * BV;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t nch = (T + C - 1) / C;

    for (int idx = tid; idx < DK * BV; idx += NT) {
        const int f = idx / BV, j = idx % BV;
        sdM[f * PS + j] = dS_T ? dS_T[(bh * DK + f) * dv + j0 + j] : 0.f;
    }
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t c0 = c * C, row0 = bh * T + c0;
        const int n = static_cast<int>(T - c0 < C ? T - c0 : C);
        __syncthreads();  // the previous chunk is done with every buffer
        load_qk<C, DK, PQ, PX>(q, k, d, row0, n, sQ, sK, sKt, tid);
        for (int idx = tid; idx < C * BV; idx += NT) {
            const int r = idx / BV, j = idx % BV;
            sdO[r * PS + j] = r < n ? to_f32(dO[(row0 + r) * dv + j0 + j]) : 0.f;
        }
        if (tid < 64) decay_scan<C>(beta, alpha, row0, n, sb, sg, sgam, sw, lane);
        // the gradient with respect to the state at the end of this chunk
        for (int idx = tid; idx < DK * BV; idx += NT) {
            const int f = idx / BV, j = idx % BV;
            dMck[((bh * nch + c) * DK + f) * dv + j0 + j] = sdM[f * PS + j];
        }
        __syncthreads();
        scores<C, DK, PQ, PX, PC>(sQ, sK, sKt, sg, sAS, sP, tid);
        __syncthreads();
        {  // dU = P^T dO + diag(w) K~ dM
            constexpr int TM = C / 16, TN = BV / 16;
            const int i0 = (tid / 16) * TM, j0l = (tid % 16) * TN;
            float acc[TM][TN], acc2[TM][TN];
            zero(acc);
            zero(acc2);
            mm<TM, TN, DK>(acc, i0, j0l, [&](int i, int kk) { return sKt[i * PX + kk]; },
                           [&](int kk, int j) { return sdM[kk * PS + j]; });
            mm<TM, TN, C>(acc2, i0, j0l, [&](int i, int kk) { return sP[kk * PC + i]; },
                          [&](int kk, int j) { return sdO[kk * PS + j]; });
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int nn = 0; nn < TN; ++nn)
                    sX[(i0 + m) * PS + j0l + nn] = acc2[m][nn] + sw[i0 + m] * acc[m][nn];
        }
        __syncthreads();
        solve_upper<C, BV, PS, PC>(sX, sAS, sb, tid);  // dR
        __syncthreads();
        {  // dM <- gam_L dM + Q^T diag(gam) dO - K^T diag(gam b) dR
            constexpr int TM = DK / 16, TN = BV / 16;
            const int i0 = (tid / 16) * TM, j0l = (tid % 16) * TN;
            float acc[TM][TN];
            zero(acc);
            mm<TM, TN, C>(acc, i0, j0l, [&](int f, int r) { return to_f32(sQ[r * PQ + f]); },
                          [&](int r, int j) { return sgam[r] * sdO[r * PS + j]; });
            mm<TM, TN, C>(acc, i0, j0l, [&](int f, int r) { return to_f32(sK[r * PQ + f]); },
                          [&](int r, int j) { return -sgam[r] * sb[r] * sX[r * PS + j]; });
            const float gl = sgam[C - 1];
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int nn = 0; nn < TN; ++nn) {
                    float &x = sdM[(i0 + m) * PS + j0l + nn];
                    x = gl * x + acc[m][nn];
                }
        }
    }
    __syncthreads();
    if (dS0) {
        for (int idx = tid; idx < DK * BV; idx += NT) {
            const int f = idx / BV, j = idx % BV;
            dS0[(bh * DK + f) * dv + j0 + j] = sdM[f * PS + j];
        }
    }
}

// ---- per-chunk gradients ----------------------------------------------------------------------
// One workgroup per (sequence, chunk).  The value columns are taken BV at a time; dP, dA, dQ,
// dK and dK~ accumulate over them in registers.
template <int C, int DK, int DV, int BV, typename TQ, typename TD>
__global__ void __launch_bounds__(NT)
bwd_chunk_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k, const TQ *__restrict__ v,
                 const TD *__restrict__ d, const float *__restrict__ beta,
                 const float *__restrict__ alpha, const TQ *__restrict__ dO,
                 const float *__restrict__ Mck, const float *__restrict__ dMck,
                 TQ *__restrict__ gq, TQ *__restrict__ gk, TQ *__restrict__ gv,
                 float *__restrict__ gbeta, TD *__restrict__ gd, float *__restrict__ galpha,
                 int64_t T, int64_t nch) {
    constexpr int PQ = DK + (sizeof(TQ) == 2 ? 2 : 1);
    constexpr int PX = DK + 1, PC = C + 1, PS = BV + 1;
    constexpr int TC = C / 16, TK = DK / 16, TV = BV / 16;  // register blocks
    __shared__ TQ sQ[C * PQ], sK[C * PQ];
    __shared__ float sKt[C * PX], sAS[C * PC], sP[C * PC];
    // slice buffers; after the slices, sM0/sdM hold column partial sums
    __shared__ float sM0[DK * PS], sdM[DK * PS];
    __shared__ float sY[C * PS], sdO[C * PS], sU[C * PS], sdR[C * PS];
    __shared__ float sKM[C * PS], sQM[C * PS], sKdM[C * PS];
    __shared__ float sb[C], sg[C], sgam[C], sw[C], sdb[C], sdg[C], sew[C], sred[4];

    const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
    const int64_t c0 = c * C, row0 = bh * T + c0;
    const int n = static_cast<int>(T - c0 < C ? T - c0 : C);
    const int tid = threadIdx.x, lane = tid & 63;
    const int ti = tid / 16, tj = tid % 16;
    const float *M0 = Mck + (bh * nch + c) * DK * DV;
    const float *dMC = dMck + (bh * nch + c) * DK * DV;

    load_qk<C, DK, PQ, PX>(q, k, d, row0, n, sQ, sK, sKt, tid);
    if (tid < 64) decay_scan<C>(beta, alpha, row0, n, sb, sg, sgam, sw, lane);
    if (tid < C) sdb[tid] = sdg[tid] = sew[tid] = 0.f;
    __syncthreads();
    scores<C, DK, PQ, PX, PC>(sQ, sK, sKt, sg, sAS, sP, tid);

    float aQ[TC][TK], aK[TC][TK], aKt[TC][TK], adP[TC][TC], adA[TC][TC];
    zero(aQ);
    zero(aK);
    zero(aKt);
    zero(adP);
    zero(adA);
    float frob = 0.f;  // this thread's part of <dMC, M0>
    const int ic = ti * TC, jc = tj * TC;  // C x C block
    const int ik = ti * TC, jk = tj * TK;  // C x DK block
    const int is = ti * TC, js = tj * TV;  // C x BV block

    for (int s0 = 0; s0 < DV; s0 += BV) {
        __syncthreads();  // the previous slice (and the scores) are done
        for (int idx = tid; idx < DK * BV; idx += NT) {
            const int f = idx / BV, j = idx % BV;
            const float m0 = M0[f * DV + s0 + j], dm = dMC[f * DV + s0 + j];
            sM0[f * PS + j] = m0;
            sdM[f * PS + j] = dm;
            frob += m0 * dm;
        }
        for (int idx = tid; idx < C * BV; idx += NT) {
            const int r = idx / BV, j = idx % BV;
            sY[r * PS + j] = r < n ? to_f32(v[(row0 + r) * DV + s0 + j]) : 0.f;
            sdO[r * PS + j] = r < n ? to_f32(dO[(row0 + r) * DV + s0 + j]) : 0.f;
        }
        __syncthreads();
        {  // K M0, Q M0, K~ dMC on this slice; then Y = V - gam K M0 and R = b Y into U
            float a1[TC][TV], a2[TC][TV], a3[TC][TV];
            zero(a1);
            zero(a2);
            zero(a3);
            auto bm = [&](int kk, int j) { return sM0[kk * PS + j]; };
            mm<TC, TV, DK>(a1, is, js, [&](int i, int kk) { return to_f32(sK[i * PQ + kk]); }, bm);
            mm<TC, TV, DK>(a2, is, js, [&](int i, int kk) { return to_f32(sQ[i * PQ + kk]); }, bm);
            mm<TC, TV, DK>(a3, is, js, [&](int i, int kk) { return sKt[i * PX + kk]; },
                           [&](int kk, int j) { return sdM[kk * PS + j]; });
#pragma unroll
            for (int m = 0; m < TC; ++m)
#pragma unroll
                for (int nn = 0; nn < TV; ++nn) {
                    const int r = is + m, j = js + nn;
                    sKM[r * PS + j] = a1[m][nn];
                    sQM[r * PS + j] = a2[m][nn];
                    sKdM[r * PS + j] = a3[m][nn];
                    const float y = sY[r * PS + j] - sgam[r] * a1[m][nn];
                    sY[r * PS + j] = y;
                    sU[r * PS + j] = sb[r] * y;
                }
        }
        __syncthreads();
        solve_lower<C, BV, PS, PC>(sU, sAS, sb, tid);  // U = (I + A)^{-1} R
        __syncthreads();
        {  // dU = P^T dO + diag(w) K~ dMC
            float acc[TC][TV];
            zero(acc);
            mm<TC, TV, C>(acc, is, js, [&](int i, int kk) { return sP[kk * PC + i]; },
                          [&](int kk, int j) { return sdO[kk * PS + j]; });
#pragma unroll
            for (int m = 0; m < TC; ++m)
#pragma unroll
                for (int nn = 0; nn < TV; ++nn) {
                    const int r = is + m, j = js + nn;
                    sdR[r * PS + j] = acc[m][nn] + sw[r] * sKdM[r * PS + j];
                }
        }
        __syncthreads();
        solve_upper<C, BV, PS, PC>(sdR, sAS, sb, tid);  // dR = (I + A)^{-T} dU
        __syncthreads();
        for (int idx = tid; idx < C * BV; idx += NT) {
            const int r = idx / BV, j = idx % BV;
            if (r < n) gv[(row0 + r) * DV + s0 + j] = from_f32<TQ>(sb[r] * sdR[r * PS + j]);
        }
        if (tid < C) {  // row sums of this slice (each row owned by one thread)
            const int r = tid;
            float db = 0.f, go = 0.f, gr = 0.f, ew = 0.f;
            for (int j = 0; j < BV; ++j) {
                db += sdR[r * PS + j] * sY[r * PS + j];
                go += sdO[r * PS + j] * sQM[r * PS + j];
                gr += sdR[r * PS + j] * sKM[r * PS + j];
                ew += sKdM[r * PS + j] * sU[r * PS + j];
            }
            sdb[r] += db;
            sdg[r] += sgam[r] * go - sb[r] * sgam[r] * gr;
            sew[r] += sw[r] * ew;
        }
        // dP += dO U^T, dA += dR U^T (negated later), and the slice's part of dQ, dK, dK~
        auto bu = [&](int kk, int j) { return sU[j * PS + kk]; };
        mm<TC, TC, BV>(adP, ic, jc, [&](int i, int kk) { return sdO[i * PS + kk]; }, bu);
        mm<TC, TC, BV>(adA, ic, jc, [&](int i, int kk) { return sdR[i * PS + kk]; }, bu);
        auto bm0t = [&](int kk, int f) { return sM0[f * PS + kk]; };
        mm<TC, TK, BV>(aQ, ik, jk, [&](int i, int kk) { return sgam[i] * sdO[i * PS + kk]; }, bm0t);
        mm<TC, TK, BV>(aK, ik, jk,
                       [&](int i, int kk) { return -sgam[i] * sb[i] * sdR[i * PS + kk]; }, bm0t);
        mm<TC, TK, BV>(aKt, ik, jk, [&](int i, int kk) { return sw[i] * sU[i * PS + kk]; },
                       [&](int kk, int f) { return sdM[f * PS + kk]; });
    }
    frob = block_sum(frob, sred, tid);  // ends with a barrier: the slices are done

    // dP (lower-inclusive) and dA (strictly lower, negated); their products with P and A give
    // the decay terms: row sums here, column sums through LDS (sM0 as [16][C] partials)
    float *colpart = sM0;
    {
        float rowp[TC], colp[TC];
#pragma unroll
        for (int m = 0; m < TC; ++m) rowp[m] = colp[m] = 0.f;
        float rowb[TC];
#pragma unroll
        for (int m = 0; m < TC; ++m) rowb[m] = 0.f;
#pragma unroll
        for (int m = 0; m < TC; ++m)
#pragma unroll
            for (int nn = 0; nn < TC; ++nn) {
                const int i = ic + m, j = jc + nn;
                const float dp = j <= i ? adP[m][nn] : 0.f;
                const float da = j < i ? -adA[m][nn] : 0.f;
                adP[m][nn] = dp;
                adA[m][nn] = da;
                const float e = dp * sP[i * PC + j] + da * sb[i] * sAS[i * PC + j];
                rowp[m] += e;
                colp[nn] += e;
                rowb[m] += da * sAS[i * PC + j];
            }
#pragma unroll
        for (int m = 0; m < TC; ++m) {
#pragma unroll
            for (int w = 1; w < 16; w <<= 1) {
                rowp[m] += __shfl_xor(rowp[m], w);
                rowb[m] += __shfl_xor(rowb[m], w);
            }
        }
        if (tj == 0) {
#pragma unroll
            for (int m = 0; m < TC; ++m) {
                sdg[ic + m] += rowp[m];
                sdb[ic + m] += rowb[m];
            }
        }
#pragma unroll
        for (int nn = 0; nn < TC; ++nn) colpart[ti * C + jc + nn] = colp[nn];
    }
    __syncthreads();
    if (tid < C) {
        float s = 0.f;
        for (int t = 0; t < 16; ++t) s += colpart[t * C + tid];
        sdg[tid] -= s;
    }
    // dP o G and Gb = dA o G (row scaled by b) replace P and AS
#pragma unroll
    for (int m = 0; m < TC; ++m)
#pragma unroll
        for (int nn = 0; nn < TC; ++nn) {
            const int i = ic + m, j = jc + nn;
            const float G = j <= i ? __expf(sg[i] - sg[j]) : 0.f;
            sP[i * PC + j] = adP[m][nn] * G;
            sAS[i * PC + j] = adA[m][nn] * G * sb[i];
        }
    __syncthreads();
    {
        auto bkt = [&](int kk, int f) { return sKt[kk * PX + f]; };
        mm<TC, TK, C>(aQ, ik, jk, [&](int i, int kk) { return sP[i * PC + kk]; }, bkt);
        mm<TC, TK, C>(aK, ik, jk, [&](int i, int kk) { return sAS[i * PC + kk]; }, bkt);
        mm<TC, TK, C>(aKt, ik, jk, [&](int i, int kk) { return sP[kk * PC + i]; },
                      [&](int kk, int f) { return to_f32(sQ[kk * PQ + f]); });
        mm<TC, TK, C>(aKt, ik, jk, [&](int i, int kk) { return sAS[kk * PC + i]; },
                      [&](int kk, int f) { return to_f32(sK[kk * PQ + f]); });
    }
#pragma unroll
    for (int m = 0; m < TC; ++m) {
        const int r = ik + m;
        if (r < n) {
#pragma unroll
            for (int nn = 0; nn < TK; ++nn) {
                const int f = jk + nn;
                const int64_t e = (row0 + r) * DK + f;
                const float kv = to_f32(sK[r * PQ + f]);
                gq[e] = from_f32<TQ>(aQ[m][nn]);
                gk[e] = from_f32<TQ>(aK[m][nn] + aKt[m][nn] * to_f32(d[e]));
                gd[e] = from_f32<TD>(aKt[m][nn] * kv);
            }
        }
    }
    __syncthreads();
    if (tid == 0) {  // the last row's terms, then the reverse running sum of dg
        float ews = 0.f;
        for (int r = 0; r < n; ++r) ews += sew[r];
        float acc = 0.f;
        for (int r = n - 1; r >= 0; --r) {
            float g = sdg[r] - sew[r];
            if (r == n - 1) g += sgam[C - 1] * frob + ews;
            acc += g;
            sdg[r] = acc;  // d ln(alpha_r)
        }
    }
    __syncthreads();
    if (tid < n) {
        gbeta[row0 + tid] = sdb[tid];
        if (alpha && galpha) galpha[row0 + tid] = sdg[tid] / alpha[row0 + tid];
    }
}

// bf16 MFMA fragments from bf16 row-major LDS tiles (pitch a multiple of 8 elements):
// rows: lane (q, n) gets X[r0 + n][k0 + 8q .. +7] (one 16-byte read);
// cols: lane (q, n) gets X[k0 + 8q .. +7][c0 + n] (two transposing reads)
__device__ __forceinline__ v8s frag_rows(const uint16_t *X, int pitch, int r0, int k0, int lr, int lq) {
    return ld8(&X[(r0 + lr) * pitch + k0 + 8 * lq]);
}
__device__ __forceinline__ v8s frag_cols(const uint16_t *X, int pitch, int k0, int c0, int lr, int lq) {
    const int kb = k0 + 8 * lq, c = c0 + 4 * (lr & 3), r = lr >> 2;
    return cat8(ld_tr(&X[(kb + r) * pitch + c]), ld_tr(&X[(kb + 4 + r) * pitch + c]));
}
__device__ __forceinline__ uint16_t bf16_bits(float x) { return f32_to_bf16_bits(x); }

// ---- per-chunk gradients on bf16 matrix cores (bf16 inputs, C = 64) ---------------------------
// Same data flow as bwd_chunk_kernel, on eight waves (two per SIMD, so one wave's LDS and
// memory waits overlap the other's matrix work).  Wave (rw, hw) = (wave % 4, wave / 4) owns
// rows 16rw..16rw+15 of every product; of the 32-column value slice it takes columns
// 16hw..16hw+15, of the dk x C and C x C gradient tiles the feature tiles of half hw and the
// score tiles t = hw, hw + 2.  Products are 16x16 fp32 tiles in the MFMA C layout (lane (q, n)
// holds rows 4q..4q+3 of column n); operand fragments are 16-byte or transposing reads of bf16
// LDS tiles.  U = T R and dR = T^T dU take T from its hi/lo planes and R, dU split the same
// way (hi.hi + hi.lo + lo.hi: fp32 accuracy; the dropped lo.lo term is below 2^-16 of the
// product).  The row sums of the decay and beta gradients stay in registers as per-lane fp32
// partials across the slices and are reduced once at the end.
template <int DK, int DV, typename TD>
__global__ void __launch_bounds__(2 * NT)
bwd_chunk_mfma_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
                      const bf16_t *__restrict__ v, const TD *__restrict__ d,
                      const float *__restrict__ beta, const float *__restrict__ alpha,
                      const bf16_t *__restrict__ dO, const uint16_t *__restrict__ Mck,
                      const uint16_t *__restrict__ dMck, const uint16_t *__restrict__ Tck,
                      const uint16_t *__restrict__ Uck, const uint16_t *__restrict__ dRck,
                      bf16_t *__restrict__ gq, bf16_t *__restrict__ gk,
                      float *__restrict__ gbeta, TD *__restrict__ gd,
                      float *__restrict__ galpha, int64_t T, int64_t nch, int64_t total) {
    constexpr int C = 64, BV = 32, NW = 8, NTH = NW * 64;
    constexpr int PH = DK + 8, PCH = C + 8, PVH = BV + 8;  // bf16 pitches
    constexpr int NF = DK / 16, NFH = NF / 2;  // feature tiles; per half
    constexpr int MB = 2 * DK * PVH > C * PCH ? 2 * DK * PVH : C * PCH;
    constexpr int MU = DK * BV / 4 / NTH;      // 4-value units of an M0 (dMC) slice per thread
    static_assert(MU == 1 || MU == 2, "one or two M units per thread");
    static_assert(C * BV / 4 == NTH, "one 4-value unit of v, dO, U, dR per thread");
    __shared__ alignas(16) uint16_t sQ[C * PH], sK[C * PH], sKt[C * PH];
    __shared__ alignas(16) uint16_t sPb[C * PCH];  // dP o G (bf16) for the closing products
    __shared__ alignas(16) uint16_t sMb[MB];       // M0 and dMC slices, later Gb (bf16)
    __shared__ alignas(16) uint16_t sDOb[C * PVH], sUb[C * PVH], sDRb[C * PVH], sVb[C * PVH];
    __shared__ float sb[C], sg[C], sgam[C], sw[C];
    __shared__ float srow[2][6][C];  // per-half row sums of the dg and dbeta terms
    __shared__ float scol[4][C];     // column sums of the decay term, by row block
    __shared__ float sred[NW];
    uint16_t *const sM0b = sMb, *const sdMb = sMb + DK * PVH;

    // thread indices; re-derived at the top of every chunk from an opaque copy of the thread id,
    // so that the compiler does not hoist the many LDS addresses built from them out of the
    // chunk loop (held across it they would not fit in the registers)
    int tid, lane, wave, rw, hw, lr, lq, R0, jt, ro, fo;
    auto derive = [&]() __attribute__((always_inline)) {
        tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        lane = tid & 63;
        wave = tid >> 6;
        rw = wave & 3;   // this wave's rows: R0 = 16 rw ..
        hw = wave >> 2;  // this wave's half of the features and columns jt = 16 hw .. of a slice
        lr = lane & 15;
        lq = lane >> 4;
        R0 = 16 * rw;
        jt = 16 * hw;
        ro = R0 + 4 * lq + (lr & 3);  // an output 4-vector's row and first feature in its tile
        fo = 4 * (lr >> 2);
    };
    derive();
    // Persistent: the workgroup takes chunks ci = blockIdx.x, + gridDim.x, ... (ci = sequence *
    // nch + chunk), and issues the next chunk's prologue loads while it finishes the current one.
    // A chunk's rows are row0 .. row0 + n - 1 of the [B*H*T] token rows.
    auto rows_of_chunk = [&](int64_t cc, int64_t &r0, int &nn) __attribute__((always_inline)) {
        const int64_t cb = cc / nch, c0 = (cc % nch) * C;
        r0 = cb * T + c0;
        nn = static_cast<int>(T - c0 < C ? T - c0 : C);
    };
    constexpr int G = DK / 8, NU = C * G / NTH;  // units per row, units per thread
    static_assert(NU * NTH == C * G, "whole units");
    // the value slices' M0, dMC, v, dO, U and dR (bf16, four per 8-byte unit) pass through
    // named registers two slices ahead (two register sets; the slice loop is unrolled)
    struct SliceRegs {
        uint2 m0a, m0b, dma, dmb, vu, ou, uu, ru;
    };
    SliceRegs ra{}, rb{};
    auto load_slice = [&](SliceRegs &x, int S0, int64_t cc, int64_t r0, int nn)
        __attribute__((always_inline)) {
        const uint16_t *M0 = Mck + cc * DK * DV, *dMC = dMck + cc * DK * DV;  // bf16, by ckpt_at
        {
            const int f = tid / (BV / 4), j = 4 * (tid % (BV / 4));
            x.m0a = *reinterpret_cast<const uint2 *>(M0 + ckpt_at(f, S0 + j, DK));
            x.dma = *reinterpret_cast<const uint2 *>(dMC + ckpt_at(f, S0 + j, DK));
        }
        if constexpr (MU == 2) {
            const int u = tid + NTH, f = u / (BV / 4), j = 4 * (u % (BV / 4));
            x.m0b = *reinterpret_cast<const uint2 *>(M0 + ckpt_at(f, S0 + j, DK));
            x.dmb = *reinterpret_cast<const uint2 *>(dMC + ckpt_at(f, S0 + j, DK));
        }
        // the chunk's rows of every per-token array: uniform bases, 32-bit offsets
        const int r = tid / (BV / 4), j = 4 * (tid % (BV / 4));
        const int e = (r < nn ? r : nn - 1) * DV + S0 + j;
        x.vu = *reinterpret_cast<const uint2 *>(v + r0 * DV + e);
        x.ou = *reinterpret_cast<const uint2 *>(dO + r0 * DV + e);
        const int ue = rows_at(r < nn ? r : nn - 1, S0 + j);  // the chunk's column-tile block
        x.uu = *reinterpret_cast<const uint2 *>(Uck + cc * C * DV + ue);
        x.ru = *reinterpret_cast<const uint2 *>(dRck + cc * C * DV + ue);
    };
    constexpr int NS = DV / BV;  // value slices
    // a chunk's prologue loads, issued while the previous chunk finishes: beta, alpha (every
    // wave, for the scan), Q, K, K~ (bf16, 8 features per 16-byte unit; K~ from its plane) in
    // named registers (an array carried across the chunk loop would live in scratch or LDS)
    static_assert(NU == 1 || NU == 2, "one or two units per thread");
    float pbv, pav;
    uint4 q0r, q1r, k0r, k1r, w0r, w1r;
    auto qreg = [&](auto I) -> uint4 & { if constexpr (decltype(I)::value == 0) return q0r; else return q1r; };
    auto kreg = [&](auto I) -> uint4 & { if constexpr (decltype(I)::value == 0) return k0r; else return k1r; };
    auto wreg = [&](auto I) -> uint4 & { if constexpr (decltype(I)::value == 0) return w0r; else return w1r; };
    auto issue_prologue = [&](int64_t cc, int64_t r0, int nn) __attribute__((always_inline)) {
        pbv = beta[r0 + (lane < nn ? lane : nn - 1)];
        pav = (alpha ? alpha : beta)[r0 + (lane < nn ? lane : nn - 1)];  // unused without alpha
        __builtin_amdgcn_sched_barrier(0);  // the loads leave in this order (waits count them so)
        const uint16_t *pc = Tck + cc * (3 * C * C + C * DK);
        static_for<0, NU>([&](auto I) __attribute__((always_inline)) {
            const int u = tid + I * NTH, r = u / G, g = u % G;
            wreg(I) = *reinterpret_cast<const uint4 *>(pc + 3 * C * C + r * DK + 8 * g);
        });
        static_for<0, NU>([&](auto I) __attribute__((always_inline)) {
            const int u = tid + I * NTH, r = u / G, g = u % G;
            const int64_t e = (r0 + (r < nn ? r : nn - 1)) * DK + 8 * g;
            qreg(I) = *reinterpret_cast<const uint4 *>(q + e);
            kreg(I) = *reinterpret_cast<const uint4 *>(k + e);
        });
        __builtin_amdgcn_sched_barrier(0);
    };
    // score tile t of this wave's rows: AS = strictly lower (K K~^T) o G and P =
    // lower-inclusive (Q K~^T) o G in the C layout (zero for tiles above the diagonal)
    auto score_tiles = [&](int t, v4f &ak, v4f &aq) __attribute__((always_inline)) {
        ak = zero4();
        aq = zero4();
        if (t <= rw) {
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32) {
                const v8s kt = frag_rows(sKt, PH, 16 * t, k0, lr, lq);
                ak = mfma32(frag_rows(sK, PH, R0, k0, lr, lq), kt, ak);
                aq = mfma32(frag_rows(sQ, PH, R0, k0, lr, lq), kt, aq);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = R0 + 4 * lq + e, j = 16 * t + lr;
            const float G = j <= i ? __expf(sg[i] - sg[j]) : 0.f;
            ak[e] = j < i ? ak[e] * G : 0.f;
            aq[e] = aq[e] * G;
        }
    };

    int64_t ci = blockIdx.x, row0;
    int n;
    if (ci >= total) return;
    rows_of_chunk(ci, row0, n);
    issue_prologue(ci, row0, n);

#pragma unroll 1
    for (;;) {
    derive();
    v4f aQ[NFH], aK[NFH], aKt[NFH], adP[2], adA[2];
#pragma unroll
    for (int t = 0; t < NFH; ++t) aQ[t] = aK[t] = aKt[t] = zero4();
    adP[0] = adP[1] = adA[0] = adA[1] = zero4();
    float pdb[4] = {0.f, 0.f, 0.f, 0.f};  // <dR_r, V_r> over the value columns, per lane
    float frob = 0.f;
    const TD *dc = d + row0 * DK;

    // the first two value slices of this chunk, then its prologue tiles into LDS
    __builtin_amdgcn_sched_barrier(0);
    load_slice(ra, 0, ci, row0, n);
    if constexpr (NS > 1) load_slice(rb, BV, ci, row0, n);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NU>([&](auto I) __attribute__((always_inline)) {
        const int u = tid + I * NTH, r = u / G, g = u % G;
        const uint32_t m = r < n ? 0xffffffffu : 0u;  // rows past the end are zero
        const uint4 qq = qreg(I), kk = kreg(I);
        *reinterpret_cast<uint4 *>(&sQ[r * PH + 8 * g]) = make_uint4(qq.x & m, qq.y & m, qq.z & m, qq.w & m);
        *reinterpret_cast<uint4 *>(&sK[r * PH + 8 * g]) = make_uint4(kk.x & m, kk.y & m, kk.z & m, kk.w & m);
        *reinterpret_cast<uint4 *>(&sKt[r * PH + 8 * g]) = wreg(I);
    });
    // the decay scan: every wave computes it and writes the same values (no branch for its
    // loads to sink into: they stay first)
    decay_scan_of<C>(pbv, pav, alpha != nullptr, n, sb, sg, sgam, sw, lane);
    const float acur = pav;  // alpha of row lane of this chunk (wave 0's galpha)
    // d of this thread's output elements, loaded during the last slice (see below)
    float dfin[NFH][4];

    static_for<0, NS>([&](auto S) __attribute__((always_inline)) {
        constexpr int s0 = S * BV;
        SliceRegs &x = (S & 1) ? rb : ra;
        __syncthreads();  // the previous slice (and the prologue) are done
#pragma unroll
        for (int i = 0; i < MU; ++i) {
            const int u = tid + i * NTH, f = u / (BV / 4), j = 4 * (u % (BV / 4));
            const uint2 mm = i == 0 ? x.m0a : x.m0b, dd = i == 0 ? x.dma : x.dmb;
            *reinterpret_cast<uint2 *>(&sM0b[f * PVH + j]) = mm;
            *reinterpret_cast<uint2 *>(&sdMb[f * PVH + j]) = dd;
            frob += bf_lo(mm.x) * bf_lo(dd.x) + bf_hi(mm.x) * bf_hi(dd.x) +
                    bf_lo(mm.y) * bf_lo(dd.y) + bf_hi(mm.y) * bf_hi(dd.y);
        }
        {  // v, dO, U, dR; rows past the end are zero
            const int r = tid / (BV / 4), j = 4 * (tid % (BV / 4));
            const uint32_t m = r < n ? 0xffffffffu : 0u;
            *reinterpret_cast<uint2 *>(&sVb[r * PVH + j]) = make_uint2(x.vu.x & m, x.vu.y & m);
            *reinterpret_cast<uint2 *>(&sDOb[r * PVH + j]) = make_uint2(x.ou.x & m, x.ou.y & m);
            *reinterpret_cast<uint2 *>(&sUb[r * PVH + j]) = make_uint2(x.uu.x & m, x.uu.y & m);
            *reinterpret_cast<uint2 *>(&sDRb[r * PVH + j]) = make_uint2(x.ru.x & m, x.ru.y & m);
        }
        if constexpr (S + 2 < NS) load_slice(x, s0 + 2 * BV, ci, row0, n);  // two slices ahead
        if constexpr (S + 1 == NS) {
            // d where this thread's outputs go (after a quad transpose lane (lq, lr) holds row
            // R0 + 4 lq + lr % 4, features 16 tile + 4 (lr / 4) .. +3), ahead of the products
#pragma unroll
            for (int t = 0; t < NFH; ++t) {
                const int off = (ro < n ? ro : n - 1) * DK + 16 * (NFH * hw + t) + fo;
                if constexpr (sizeof(TD) == 4) {
                    const float4 y = *reinterpret_cast<const float4 *>(dc + off);
                    dfin[t][0] = y.x; dfin[t][1] = y.y; dfin[t][2] = y.z; dfin[t][3] = y.w;
                } else {
                    const uint2 y = *reinterpret_cast<const uint2 *>(dc + off);
                    dfin[t][0] = bf_lo(y.x); dfin[t][1] = bf_hi(y.x);
                    dfin[t][2] = bf_lo(y.y); dfin[t][3] = bf_hi(y.y);
                }
            }
        }
        __syncthreads();
        // dP += dO U^T, dA += dR U^T (negated later) on this wave's score tiles; the slice's
        // part of dO M0^T, dR M0^T, U dMC^T on this wave's feature tiles (K = the slice's 32
        // columns; the row factors gam, -gam b, w of dQ, dK, dK~ come at the end); <dR, V> on
        // this wave's tile
        static_for<0, 2>([&](auto I) __attribute__((always_inline)) {
            const int t = 2 * I + hw;
            if (t <= rw) {
                const v8s ub = frag_rows(sUb, PVH, 16 * t, 0, lr, lq);
                adP[I] = mfma32(frag_rows(sDOb, PVH, R0, 0, lr, lq), ub, adP[I]);
                adA[I] = mfma32(frag_rows(sDRb, PVH, R0, 0, lr, lq), ub, adA[I]);
            }
        });
        const v8s dob = frag_rows(sDOb, PVH, R0, 0, lr, lq), drb = frag_rows(sDRb, PVH, R0, 0, lr, lq);
        const v8s urb = frag_rows(sUb, PVH, R0, 0, lr, lq);
#pragma unroll
        for (int t = 0; t < NFH; ++t) {
            const int f0 = 16 * (NFH * hw + t);
            const v8s m0r = frag_rows(sM0b, PVH, f0, 0, lr, lq);
            aQ[t] = mfma32(dob, m0r, aQ[t]);
            aK[t] = mfma32(drb, m0r, aK[t]);
            aKt[t] = mfma32(urb, frag_rows(sdMb, PVH, f0, 0, lr, lq), aKt[t]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = R0 + 4 * lq + e, j = jt + lr;
            pdb[e] += __uint_as_float(uint32_t(sDRb[r * PVH + j]) << 16) *
                      __uint_as_float(uint32_t(sVb[r * PVH + j]) << 16);
        }
    });
    // the next chunk's prologue, in flight through this chunk's closing phase (past the last
    // chunk the loads repeat this one: every load is issued, so the wait counts stay exact)
    const int64_t cn = ci + gridDim.x;
    int64_t rn0 = row0;
    int nn = n;
    if (cn < total) rows_of_chunk(cn, rn0, nn);
    issue_prologue(cn < total ? cn : ci, rn0, nn);
    {  // <dMC, M0> over the workgroup (fixed order); ends with a barrier: the slices are done
        frob = sum_rows(group_sum<16>(frob));
        __syncthreads();
        if (lane == 0) sred[wave] = frob;
        __syncthreads();
        frob = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) frob += sred[w];
    }

    // masks of dP, dA; the decay terms dP o P + dA o A (row sums, and column sums by row
    // block) and the dbeta term of A, on this wave's score tiles
    float rowp[4] = {0.f, 0.f, 0.f, 0.f}, rowb[4] = {0.f, 0.f, 0.f, 0.f};
    static_for<0, 2>([&](auto I) __attribute__((always_inline)) {
        const int t = 2 * I + hw;
        v4f as, ps;  // AS and P of the tile, formed again
        score_tiles(t, as, ps);
        float colp = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = R0 + 4 * lq + e, j = 16 * t + lr;
            const float dp = j <= i ? adP[I][e] : 0.f;
            const float da = j < i ? -adA[I][e] : 0.f;
            adP[I][e] = dp;
            adA[I][e] = da;
            const float ex = dp * ps[e] + da * sb[i] * as[e];
            rowp[e] += ex;
            colp += ex;
            rowb[e] += da * as[e];
        }
        colp = sum_rows(colp);
        if (lq == 0) scol[rw][16 * t + lr] = colp;
    });
    // The slices' parts of dQ, dK, dK~ (dO M0^T, dR M0^T, U dMC^T) give the other row sums:
    //   <Q_r, (dO M0^T)_r> = <dO_r, (Q M0)_r>,  <K_r, (dR M0^T)_r> = <dR_r, (K M0)_r>,
    //   <K~_r, (U dMC^T)_r> = <U_r, (K~ dMC)_r>
    // (this wave's feature tiles; the other half's come through LDS); then they take their row
    // factors gam, -gam b, w for the closing products
    float pgo[4] = {0.f, 0.f, 0.f, 0.f}, pgr[4] = {0.f, 0.f, 0.f, 0.f}, pew[4] = {0.f, 0.f, 0.f, 0.f};
    // q, k, k~ at this lane's places of the feature tiles (rows R0 + 4 lq + e, column 16 T + lr),
    // four rows per transposing read
    v4s qt4[NFH], kt4[NFH], wt4[NFH];
#pragma unroll
    for (int t = 0; t < NFH; ++t) {
        const int off = (R0 + 4 * lq + (lr >> 2)) * PH + 16 * (NFH * hw + t) + 4 * (lr & 3);
        qt4[t] = ld_tr(&sQ[off]);
        kt4[t] = ld_tr(&sK[off]);
        wt4[t] = ld_tr(&sKt[off]);
    }
    auto bfe = [](short x) __attribute__((always_inline)) {
        return __uint_as_float(uint32_t(static_cast<uint16_t>(x)) << 16);
    };
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = R0 + 4 * lq + e;
        const float fq = sgam[r], fk = -sgam[r] * sb[r], fw = sw[r];
#pragma unroll
        for (int t = 0; t < NFH; ++t) {
            pgo[e] += bfe(qt4[t][e]) * aQ[t][e];
            pgr[e] += bfe(kt4[t][e]) * aK[t][e];
            pew[e] += bfe(wt4[t][e]) * aKt[t][e];
            aQ[t][e] *= fq;
            aK[t][e] *= fk;
            aKt[t][e] *= fw;
        }
        // dbeta: <dR_r, Y_r> with Y = V - gam K M0;  dg: gam go - gam b gr - w ew
        pdb[e] -= sgam[r] * pgr[e];
        pgo[e] *= fq;
        pgr[e] *= fk;
        pew[e] *= fw;
    }
    // row sums: across the 16 lanes of a row (total in its last lane), then (below) across the
    // two halves
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pgo[e] = row16_total(pgo[e]);
        pgr[e] = row16_total(pgr[e]);
        pew[e] = row16_total(pew[e]);
        pdb[e] = row16_total(pdb[e]);
        rowp[e] = row16_total(rowp[e]);
        rowb[e] = row16_total(rowb[e]);
    }
    if (lr == 15) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = R0 + 4 * lq + e;
            srow[hw][0][r] = pgo[e];
            srow[hw][1][r] = pgr[e];
            srow[hw][2][r] = pew[e];
            srow[hw][3][r] = pdb[e];
            srow[hw][4][r] = rowp[e];
            srow[hw][5][r] = rowb[e];
        }
    }
    // dP o G into sPb and Gb = dA o G (row scaled by b) into sMb, as bf16 (this wave's tiles)
    uint16_t *const sGb = sMb;
    static_for<0, 2>([&](auto I) __attribute__((always_inline)) {
        const int t = 2 * I + hw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = R0 + 4 * lq + e, j = 16 * t + lr;
            const float G = j <= i ? __expf(sg[i] - sg[j]) : 0.f;
            sPb[i * PCH + j] = bf16_bits(adP[I][e] * G);
            sGb[i * PCH + j] = bf16_bits(adA[I][e] * G * sb[i]);
        }
    });
    __syncthreads();
    if (tid < 64) {  // dbeta; dg of every row, then its reverse running sum d ln(alpha) (wave 0)
        const int r = lane;
        const float go = srow[0][0][r] + srow[1][0][r], gr = srow[0][1][r] + srow[1][1][r];
        const float ew = srow[0][2][r] + srow[1][2][r];
        const float db = srow[0][3][r] + srow[1][3][r] + srow[0][5][r] + srow[1][5][r];
        float g = go + gr + srow[0][4][r] + srow[1][4][r] -
                  (scol[0][r] + scol[1][r] + scol[2][r] + scol[3][r]);
        // the last row's terms: gam_L <dMC, M0> + sum_s w_s <(K~ dMC)_s, U_s>
        const float ews = sum_rows(group_sum<16>(r < n ? ew : 0.f));  // over the wave, on DPP
        g = r < n ? g - ew : 0.f;
        if (r == n - 1) g += sgam[C - 1] * frob + ews;
        g = wave_suffix(g, lane);  // x_r = sum_{r' >= r} g_r'
        if (r < n) {
            gbeta[row0 + r] = db;
            if (alpha && galpha) galpha[row0 + r] = g / acur;
        }
    }
    // dQ += (dP o G) K~, dK += Gb K~, dK~ += (dP o G)^T Q + Gb^T K on this wave's feature tiles
#pragma unroll
    for (int t = 0; t < NFH; ++t) {
        const int f0 = 16 * (NFH * hw + t);
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) {
            const v8s ktc = frag_cols(sKt, PH, k0, f0, lr, lq);
            aQ[t] = mfma32(frag_rows(sPb, PCH, R0, k0, lr, lq), ktc, aQ[t]);
            aK[t] = mfma32(frag_rows(sGb, PCH, R0, k0, lr, lq), ktc, aK[t]);
            aKt[t] = mfma32(frag_cols(sPb, PCH, k0, R0, lr, lq), frag_cols(sQ, PH, k0, f0, lr, lq), aKt[t]);
            aKt[t] = mfma32(frag_cols(sGb, PCH, k0, R0, lr, lq), frag_cols(sK, PH, k0, f0, lr, lq), aKt[t]);
        }
    }
    const __amdgpu_buffer_rsrc_t grs_q = __builtin_amdgcn_make_buffer_rsrc(gq + row0 * DK, 0, n * DK * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t grs_k = __builtin_amdgcn_make_buffer_rsrc(gk + row0 * DK, 0, n * DK * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t grs_d = __builtin_amdgcn_make_buffer_rsrc(
        gd + row0 * DK, 0, n * DK * static_cast<int>(sizeof(TD)), 0x00020000);
#pragma unroll
    for (int t = 0; t < NFH; ++t) {
        const v4f gqt = quad_transpose(aQ[t], lane), gkt = quad_transpose(aK[t], lane);
        const v4f gkw = quad_transpose(aKt[t], lane);  // dK~
        const int f = 16 * (NFH * hw + t) + fo;
        const uint2 kr = *reinterpret_cast<const uint2 *>(&sK[ro * PH + f]);
        const float kv[4] = {bf_lo(kr.x), bf_hi(kr.x), bf_lo(kr.y), bf_hi(kr.y)};
        v4f gk4, gd4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            gk4[e] = gkt[e] + gkw[e] * dfin[t][e];
            gd4[e] = gkw[e] * kv[e];
        }
        // rows past the end fall outside the buffers' ranges
        const int eo = ro * DK + f;
        const uint2 pq = pack4u(gqt), pk = pack4u(gk4);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pq.x, pq.y}, grs_q, eo * 2, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pk.x, pk.y}, grs_k, eo * 2, 0, 0);
        if constexpr (sizeof(TD) == 4) {
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(gd4[0]), __float_as_uint(gd4[1]), __float_as_uint(gd4[2]),
                      __float_as_uint(gd4[3])},
                grs_d, eo * 4, 0, 0);
        } else {
            const uint2 pd = pack4u(gd4);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pd.x, pd.y}, grs_d, eo * 2, 0, 0);
        }
    }
    if (cn >= total) break;
    ci = cn;
    row0 = rn0;
    n = nn;
    __syncthreads();  // the closing phase is done with the LDS tiles the next chunk overwrites
    }
}

// ---- (I + A)^{-1} and P of every chunk (bf16 inputs, C = 64) ---------------------------------
// One workgroup per (sequence, chunk).  AS = strictly lower (K K~^T) o G and P =
// lower-inclusive (Q K~^T) o G on matrix cores (the same tiles the per-chunk pass forms), then
// T = (I + diag(b) AS)^{-1} in fp32 by blocks.  Per chunk, bf16 and row-major: hi = bf16(T),
// lo = bf16(T - hi), P (zero above the diagonal), 64 x 64 each, then K~ = d (.) k (64 x dk).
// The reverse pass and the per-chunk pass take their products with T and T^T from the first
// two at fp32 accuracy (hi.hi + hi.lo + lo.hi), P^T dO from the third, and K~ as it is.  None
// depends on the state, so all chunks are done in parallel instead of inside the sequential
// reverse pass.
template <int DK, typename TD>
__global__ void __launch_bounds__(NT)
bwd_tinv_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
                const TD *__restrict__ d, const float *__restrict__ beta,
                const float *__restrict__ alpha, uint16_t *__restrict__ Tck, int64_t T,
                int64_t nch) {
    constexpr int C = 64, PH = DK + 8, PC = C + 1;
    // K~ (bf16) until AS and P are in registers; then AS, T and the block products' scratch
    // (fp32) in the same bytes, so four workgroups fit a CU.  The A operands (this wave's rows
    // of Q and K) come from memory straight into registers in the fragment layout.
    constexpr int KB = C * PH * 2, FB = (2 * C * PC + 3 * 16 * 17) * 4;
    __shared__ alignas(16) unsigned char smem[KB > FB ? KB : FB];
    __shared__ float sb[C], sg[C], sgam[C], sw[C];
    uint16_t *const sKt = reinterpret_cast<uint16_t *>(smem);
    float *const sAS = reinterpret_cast<float *>(smem), *const sT = sAS + C * PC;
    float *const sTmp = sT + C * PC;

    const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
    const int64_t c0 = c * C, row0 = bh * T + c0;
    const int n = static_cast<int>(T - c0 < C ? T - c0 : C);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const int R0 = 16 * wave;
    // this wave's rows of Q and K as A-operand fragments: lane (q, n) holds row R0 + n,
    // features k0 + 8q .. +7 of each 32-wide k-step (zero past the end)
    constexpr int NS = DK / 32;
    v8s qf[NS], kf[NS];
    {
        const int r = R0 + lr;
        const uint32_t m = r < n ? 0xffffffffu : 0u;
        const int64_t e = (row0 + (r < n ? r : n - 1)) * DK + 8 * lq;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint4 a = *reinterpret_cast<const uint4 *>(q + e + 32 * s);
            const uint4 b = *reinterpret_cast<const uint4 *>(k + e + 32 * s);
            qf[s] = __builtin_bit_cast(v8s, make_uint4(a.x & m, a.y & m, a.z & m, a.w & m));
            kf[s] = __builtin_bit_cast(v8s, make_uint4(b.x & m, b.y & m, b.z & m, b.w & m));
        }
    }
    uint16_t *dst = Tck + (bh * nch + c) * (3 * C * C + C * DK);
    {  // K~ = d (.) k as bf16, rows past the end zero, into LDS and its plane
        constexpr int G = DK / 8, NU = C * G / NT;
        static_assert(NU * NT == C * G, "whole units");
        uint4 ku[NU];
        float dd[NU][8];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = tid + i * NT, r = u / G, g = u % G;
            const int64_t e = (row0 + (r < n ? r : n - 1)) * DK + 8 * g;
            ku[i] = *reinterpret_cast<const uint4 *>(k + e);
            load8(d + e, dd[i]);
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = tid + i * NT, r = u / G, g = u % G;
            const uint32_t kw[4] = {ku[i].x, ku[i].y, ku[i].z, ku[i].w};
            uint32_t kt[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) kt[e] = pack2(dd[i][2 * e] * bf_lo(kw[e]), dd[i][2 * e + 1] * bf_hi(kw[e]));
            const uint32_t m = r < n ? 0xffffffffu : 0u;
            const uint4 x = make_uint4(kt[0] & m, kt[1] & m, kt[2] & m, kt[3] & m);
            *reinterpret_cast<uint4 *>(&sKt[r * PH + 8 * g]) = x;
            *reinterpret_cast<uint4 *>(dst + 3 * C * C + r * DK + 8 * g) = x;
        }
    }
    if (tid < 64) decay_scan<C>(beta, alpha, row0, n, sb, sg, sgam, sw, lane);
    __syncthreads();
    v4f ak[C / 16];  // this wave's rows of AS; P's go straight to its plane
#pragma unroll
    for (int t = 0; t < C / 16; ++t) {
        v4f aq = zero4();
        ak[t] = zero4();
        if (t <= wave) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const v8s kt = frag_rows(sKt, PH, 16 * t, 32 * s, lr, lq);
                ak[t] = mfma32(kf[s], kt, ak[t]);
                aq = mfma32(qf[s], kt, aq);
            }
        }
        v4f pt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = R0 + 4 * lq + e, j = 16 * t + lr;
            pt[e] = j <= i ? aq[e] * __expf(sg[i] - sg[j]) : 0.f;
        }
        // row R0 + 4 lq + lr % 4, columns 16 t + 4 (lr / 4) .. +3 after a quad transpose
        *reinterpret_cast<uint2 *>(dst + 2 * C * C + (R0 + 4 * lq + (lr & 3)) * C + 16 * t + 4 * (lr >> 2)) =
            pack4u(quad_transpose(pt, lane));
    }
    __syncthreads();  // K~ is dead: AS takes its bytes
#pragma unroll
    for (int t = 0; t < C / 16; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = R0 + 4 * lq + e, j = 16 * t + lr;
            sAS[i * PC + j] = j < i ? ak[t][e] * __expf(sg[i] - sg[j]) : 0.f;
        }
    block_inverse64<PC>(sT, sAS, sb, sTmp, tid);  // its first barrier orders the AS writes
    for (int u = tid; u < C * C / 4; u += NT) {  // four elements per thread and pass
        const int r = u / (C / 4), j = 4 * (u % (C / 4));
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float x0 = sT[r * PC + j + 2 * e], x1 = sT[r * PC + j + 2 * e + 1];
            hw[e] = pack2(x0, x1);
            lw[e] = pack2(x0 - bf_lo(hw[e]), x1 - bf_hi(hw[e]));
        }
        *reinterpret_cast<uint2 *>(dst + r * C + j) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2 *>(dst + C * C + r * C + j) = make_uint2(lw[0], lw[1]);
    }
}

// ---- reverse pass over chunks on bf16 matrix cores (bf16 inputs, C = 64) --------------------
// Same data flow as bwd_state_kernel, on eight waves (two per SIMD).  One workgroup per
// (sequence, 32-column value slice) walks the chunks backwards.  dM (fp32, dk x 32) lives in
// registers: wave w owns its 16x16 tiles in the MFMA C layout and stores them, rounded to bf16,
// straight to the checkpoint; LDS holds the same bf16 copy, the operand of K~ dM.  Per chunk c,
// with a barrier after each phase:
//   scores   q, k of chunk c into LDS; gam dO; one 16x16 tile of K~ dM per wave; one wave runs
//            the decay scan of chunk c-1 (double-buffered);
//   dU       dU = P^T dO + diag(w) K~ dM, one tile per wave, as hi/lo bf16; K~ of chunk c-1
//            into LDS;
//   dR       dR = T^T dU from the T planes (hi.hi + hi.lo + lo.hi), one tile per wave, stored
//            in bf16 for the per-chunk pass, with dV = diag(b) dR; P and dO of chunk c-1 into
//            LDS;
//   update   dM <- gam_L dM + Q^T diag(gam) dO - K^T diag(gam b) dR on the wave's own tiles;
//            the T planes of chunk c-1 into LDS.
// So each tile of the next chunk is written in a phase after the last read of its buffer,
// with no phase of its own; its loads go to registers two to four phases before.
template <int DK, int BV>
__global__ void __launch_bounds__(2 * NT)
bwd_state_mfma_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
                      const float *__restrict__ beta,
                      const float *__restrict__ alpha, const bf16_t *__restrict__ dO,
                      const float *__restrict__ dS_T, const uint16_t *__restrict__ Tck,
                      uint16_t *__restrict__ dMck, uint16_t *__restrict__ dRck,
                      bf16_t *__restrict__ gv, float *__restrict__ dS0, int64_t T, int dv) {
    constexpr int C = 64, NW = 8, NTH = NW * 64;
    constexpr int PH = DK + 8, PCH = C + 8, PVH = BV + 8;  // bf16 pitches
    constexpr int G = DK / 8, NU = C * G / NTH;  // 16-byte units of a Q/K row; units per thread
    constexpr int TU = 3 * C * C / 8 / NTH;      // 16-byte units of the T, P planes per thread
    constexpr int CHS = 3 * C * C + C * DK;      // per-chunk planes: T hi, T lo, P, K~
    constexpr int MT = DK / 64;                  // 16x16 tiles of dM per wave
    static_assert(BV == 32 && NU * NTH == C * G && NU <= 2 && TU == 3 && C * BV / 4 == NTH,
                  "unit layout");
    __shared__ alignas(16) uint16_t sQ[C * PH], sK[C * PH], sKt[C * PH];
    __shared__ alignas(16) uint16_t sPb[C * PCH], sTh[C * PCH], sTl[C * PCH];
    __shared__ alignas(16) uint16_t sDOb[C * PVH], sGDOb[C * PVH], sGDRb[C * PVH];
    __shared__ alignas(16) uint16_t sdUh[C * PVH], sdUl[C * PVH];
    __shared__ alignas(16) uint16_t sdMb[DK * PVH];  // bf16 copy of dM (operand of K~ dM)
    __shared__ float sb[2][C], sgam[2][C], sw[2][C];  // decay scan, by chunk parity

    // workgroup -> (sequence, value slice); the slices of one sequence share an XCD (and its
    // L2) when the sequence count allows it, so their re-reads of q, k, d and T hit L2
    const int nvt = dv / BV;
    const int64_t nseq = gridDim.x / nvt;
    int64_t bh;
    int vt;
    if ((nseq & 7) == 0) {
        const int64_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        vt = static_cast<int>(slot % nvt);
        bh = (slot / nvt) * 8 + xcd;
    } else {
        vt = static_cast<int>(blockIdx.x % nvt);
        bh = blockIdx.x / nvt;
    }
    const int j0 = vt * BV;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    const int rb = wave & 3, ct = wave >> 2;  // this wave's tile of the C x 32 products
    const int R0 = 16 * rb, jt = 16 * ct;
    const int64_t nch = (T + C - 1) / C;
    const int64_t seq0 = bh * T;
    auto rows_of = [&](int64_t cc) { return static_cast<int>(T - cc * C < C ? T - cc * C : C); };

    // q, k, K~, the T and P planes and dO of a coming chunk in named registers (an array
    // carried across the loop would live in scratch); unit i of this thread is u = tid + i NTH:
    // row u / G, features 8 (u % G) .. +7; plane unit u holds elements 8u .. 8u+7 of the three
    // 64 x 64 planes (plane u / 512, row (u / 8) % 64, columns 8 (u % 8) ..)
    uint4 q0, q1, k0r, k1r, w0, w1, t0, t1, t2;
    uint2 ou;
    auto qreg = [&](auto I) -> uint4 & { if constexpr (decltype(I)::value == 0) return q0; else return q1; };
    auto kreg = [&](auto I) -> uint4 & { if constexpr (decltype(I)::value == 0) return k0r; else return k1r; };
    auto wreg = [&](auto I) -> uint4 & { if constexpr (decltype(I)::value == 0) return w0; else return w1; };
    // loads and stores by part; the loads are spread over the phases (a wave stalls while the
    // CU's load queue is full, so one burst would hold up the barrier that follows it)
    auto load_qk = [&](int64_t cc) __attribute__((always_inline)) {
        const bf16_t *qc = q + (seq0 + cc * C) * DK, *kc = k + (seq0 + cc * C) * DK;
        const int nn = rows_of(cc);
        static_for<0, NU>([&](auto I) __attribute__((always_inline)) {
            const int u = tid + I * NTH, r = u / G, g = u % G;
            const int e = (r < nn ? r : nn - 1) * DK + 8 * g;
            qreg(I) = *reinterpret_cast<const uint4 *>(qc + e);
            kreg(I) = *reinterpret_cast<const uint4 *>(kc + e);
        });
    };
    auto store_qk = [&](int nn) __attribute__((always_inline)) {
        static_for<0, NU>([&](auto I) __attribute__((always_inline)) {
            const int u = tid + I * NTH, r = u / G, g = u % G;
            const uint32_t m = r < nn ? 0xffffffffu : 0u;  // rows past the end are zero
            const uint4 kq = kreg(I), qq = qreg(I);
            *reinterpret_cast<uint4 *>(&sQ[r * PH + 8 * g]) = make_uint4(qq.x & m, qq.y & m, qq.z & m, qq.w & m);
            *reinterpret_cast<uint4 *>(&sK[r * PH + 8 * g]) = make_uint4(kq.x & m, kq.y & m, kq.z & m, kq.w & m);
        });
    };
    auto load_kt = [&](int64_t cc) __attribute__((always_inline)) {  // K~, zero past the end
        const uint4 *wp = reinterpret_cast<const uint4 *>(Tck + (bh * nch + cc) * CHS + 3 * C * C);
        static_for<0, NU>([&](auto I) __attribute__((always_inline)) { wreg(I) = wp[tid + I * NTH]; });
    };
    auto store_kt = [&]() __attribute__((always_inline)) {
        static_for<0, NU>([&](auto I) __attribute__((always_inline)) {
            const int u = tid + I * NTH, r = u / G, g = u % G;
            *reinterpret_cast<uint4 *>(&sKt[r * PH + 8 * g]) = wreg(I);
        });
    };
    auto load_pdo = [&](int64_t cc) __attribute__((always_inline)) {  // P plane, dO slice
        t2 = reinterpret_cast<const uint4 *>(Tck + (bh * nch + cc) * CHS)[tid + 2 * NTH];
        const int nn = rows_of(cc), r = tid / (BV / 4), j = 4 * (tid % (BV / 4));
        ou = *reinterpret_cast<const uint2 *>(dO + (seq0 + cc * C + (r < nn ? r : nn - 1)) * dv + j0 + j);
    };
    auto store_pdo = [&](int nn) __attribute__((always_inline)) {
        *reinterpret_cast<uint4 *>(&sPb[((tid >> 3) & 63) * PCH + 8 * (tid & 7)]) = t2;
        const int r = tid / (BV / 4), j = 4 * (tid % (BV / 4));
        const uint32_t m = r < nn ? 0xffffffffu : 0u;
        *reinterpret_cast<uint2 *>(&sDOb[r * PVH + j]) = make_uint2(ou.x & m, ou.y & m);
    };
    auto load_t = [&](int64_t cc) __attribute__((always_inline)) {  // T hi, lo planes
        const uint4 *tp = reinterpret_cast<const uint4 *>(Tck + (bh * nch + cc) * CHS);
        t0 = tp[tid];
        t1 = tp[tid + NTH];
    };
    auto store_t = [&]() __attribute__((always_inline)) {
        const int r = (tid >> 3) & 63, g = tid & 7;  // unit tid of each plane
        *reinterpret_cast<uint4 *>(&sTh[r * PCH + 8 * g]) = t0;
        *reinterpret_cast<uint4 *>(&sTl[r * PCH + 8 * g]) = t1;
    };
    // decay scan of chunk cc into buffer cc & 1 (one wave; beta, alpha of the chunk in bv, av)
    float bv = 0.f, av = 1.f;
    auto load_ba = [&](int64_t cc) __attribute__((always_inline)) {
        const int r = min(lane, rows_of(cc) - 1);
        bv = beta[seq0 + cc * C + r];
        av = (alpha ? alpha : beta)[seq0 + cc * C + r];  // unused without alpha
    };
    auto scan = [&](int64_t cc) __attribute__((always_inline)) {
        const int nn = rows_of(cc), pb = static_cast<int>(cc & 1);
        const float x = wave_prefix((lane < nn && alpha) ? logf(av) : 0.f);
        const float gl = lane_value(x, C - 1);
        sb[pb][lane] = lane < nn ? bv : 0.f;
        sgam[pb][lane] = __expf(x);
        sw[pb][lane] = __expf(gl - x);
    };

    // dM tiles of this wave: tile index ti = MT wave + m, rows 16 (ti / 2) .., columns 16 (ti % 2) ..
    v4f dM[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int ti = MT * wave + m, f0 = 16 * (ti >> 1), c0 = 16 * (ti & 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int f = f0 + 4 * lq + e, j = c0 + lr;
            dM[m][e] = dS_T ? dS_T[(bh * DK + f) * dv + j0 + j] : 0.f;
            sdMb[f * PVH + j] = bf16_bits(dM[m][e]);
            if (nch > 0) dMck[(bh * nch + nch - 1) * DK * dv + ckpt_at(f, j0 + j, DK)] = bf16_bits(dM[m][e]);
        }
    }
    if (nch > 0) {  // the last chunk's tiles (q, k stay in registers for its first phase)
        load_qk(nch - 1);
        load_kt(nch - 1);
        load_pdo(nch - 1);
        load_t(nch - 1);
        store_kt();
        store_pdo(rows_of(nch - 1));
        store_t();
        // every global access of the loop below is issued unconditionally (past the first chunk
        // the loads repeat chunk 0, the stores fall outside their buffer's range), so that the
        // compiler's wait counts stay exact and a wait for one load does not also wait for the
        // stores and loads issued after it
        load_kt(nch > 1 ? nch - 2 : 0);
        load_pdo(nch > 1 ? nch - 2 : 0);
        load_ba(nch - 1);
        if (wave == NW - 1) scan(nch - 1);
    }

    for (int64_t c = nch - 1; c >= 0; --c) {
        const int n = rows_of(c), pb = static_cast<int>(c & 1);
        __syncthreads();  // the previous chunk is done with sQ, sK, sGDOb, sGDRb, sdMb
        store_qk(n);
        {  // gam-scaled dO for the dM update
            const int r = tid / (BV / 4), j = 4 * (tid % (BV / 4));
            const uint2 o = *reinterpret_cast<const uint2 *>(&sDOb[r * PVH + j]);
            const float gm = sgam[pb][r];
            *reinterpret_cast<uint2 *>(&sGDOb[r * PVH + j]) =
                make_uint2(pack2(gm * bf_lo(o.x), gm * bf_hi(o.x)), pack2(gm * bf_lo(o.y), gm * bf_hi(o.y)));
        }
        // this wave's tile of K~ dM
        v4f kdm = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32)
            kdm = mfma32(frag_rows(sKt, PH, R0, k0, lr, lq), frag_cols(sdMb, PVH, k0, jt, lr, lq), kdm);
        load_ba(c > 0 ? c - 1 : 0);  // the next chunk's beta, alpha (scanned in the dR phase)
        load_t(c > 0 ? c - 1 : 0);
        {  // dU = P^T dO + diag(w) K~ dM on this wave's tile (its own K~ dM: no barrier), as
           // hi/lo bf16
            v4f du = zero4();
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += 32)
                du = mfma32(frag_cols(sPb, PCH, k0, R0, lr, lq), frag_cols(sDOb, PVH, k0, jt, lr, lq), du);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = R0 + 4 * lq + e, j = jt + lr;
                const float x = du[e] + sw[pb][r] * kdm[e];
                const uint16_t h = bf16_bits(x);
                sdUh[r * PVH + j] = h;
                sdUl[r * PVH + j] = bf16_bits(x - __uint_as_float(uint32_t(h) << 16));
            }
        }
        load_qk(c > 0 ? c - 1 : 0);
        __syncthreads();
        {  // dR = T^T dU (T^T upper triangular: k-steps from the tile's first row on); -gam b dR
            v4f dr = zero4();
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += 32) {
                if (k0 + 32 <= R0) continue;
                const v8s th = frag_cols(sTh, PCH, k0, R0, lr, lq), tl = frag_cols(sTl, PCH, k0, R0, lr, lq);
                const v8s uh = frag_cols(sdUh, PVH, k0, jt, lr, lq), ul = frag_cols(sdUl, PVH, k0, jt, lr, lq);
                dr = mfma32(th, uh, dr);
                dr = mfma32(th, ul, dr);
                dr = mfma32(tl, uh, dr);
            }
            v4f gvt;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = R0 + 4 * lq + e, j = jt + lr;
                sGDRb[r * PVH + j] = bf16_bits(-sgam[pb][r] * sb[pb][r] * dr[e]);
                gvt[e] = sb[pb][r] * dr[e];
            }
            // dR and dV in bf16: row R0 + 4 lq + lr % 4, columns jt + 4 (lr / 4) .. +3; dR into
            // the chunk's block of column tiles (rows_at; padded, every row written), dV with
            // the rows past the end outside the buffer range
            const uint2 drp = pack4u(quad_transpose(dr, lane));
            const uint2 gvp = pack4u(quad_transpose(gvt, lane));
            const int64_t rowc = (seq0 + c * C) * dv;
            const int boff = ((R0 + 4 * lq + (lr & 3)) * dv + j0 + jt + 4 * (lr >> 2)) * 2;
            *reinterpret_cast<uint2 *>(dRck + (bh * nch + c) * C * dv +
                                       rows_at(R0 + 4 * lq + (lr & 3), j0 + jt + 4 * (lr >> 2))) = drp;
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{gvp.x, gvp.y}, __builtin_amdgcn_make_buffer_rsrc(gv + rowc, 0, n * dv * 2, 0x00020000),
                boff, 0, 0);
            // the next chunk's decay scan, into the other buffer (this chunk reads only its own)
            if (wave == NW - 1 && c > 0) scan(c - 1);
        }
        if (c > 0) store_kt();  // K~ of the next chunk (sKt was last read by this chunk's K~ dM)
        if (c > 0) store_pdo(rows_of(c - 1));  // P and dO of the next chunk (last read by dU)
        load_kt(c > 1 ? c - 2 : 0);
        load_pdo(c > 1 ? c - 2 : 0);
        __syncthreads();
        {  // dM <- gam_L dM + Q^T diag(gam) dO - K^T diag(gam b) dR on this wave's tiles; the
           // result is the gradient at the previous chunk's end
            const float gl = sgam[pb][C - 1];
            // slot c - 1 of the checkpoints: none (an empty range) for the first chunk
            const __amdgpu_buffer_rsrc_t mrsrc = __builtin_amdgcn_make_buffer_rsrc(
                dMck + ((bh * nch + (c > 0 ? c - 1 : 0)) * DK) * dv, 0, c > 0 ? DK * dv * 2 : 0,
                0x00020000);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int ti = MT * wave + m, f0 = 16 * (ti >> 1), c0 = 16 * (ti & 1);
                v4f acc = zero4();
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += 32) {
                    acc = mfma32(frag_cols(sQ, PH, k0, f0, lr, lq), frag_cols(sGDOb, PVH, k0, c0, lr, lq), acc);
                    acc = mfma32(frag_cols(sK, PH, k0, f0, lr, lq), frag_cols(sGDRb, PVH, k0, c0, lr, lq), acc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = f0 + 4 * lq + e, j = c0 + lr;
                    dM[m][e] = gl * dM[m][e] + acc[e];
                    sdMb[f * PVH + j] = bf16_bits(dM[m][e]);
                }
                // bf16, row f0 + 4 lq + lr % 4, columns c0 + 4 (lr / 4) .. +3
                const uint2 x = pack4u(quad_transpose(dM[m], lane));
                __builtin_amdgcn_raw_buffer_store_b64(
                    u32x2{x.x, x.y}, mrsrc, ckpt_at(f0 + 4 * lq + (lr & 3), j0 + c0 + 4 * (lr >> 2), DK) * 2, 0, 0);
            }
        }
        if (c > 0) store_t();  // T of the next chunk (last read by this chunk's dR)
    }
    if (dS0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int ti = MT * wave + m, f0 = 16 * (ti >> 1), c0 = 16 * (ti & 1);
            const v4f x = quad_transpose(dM[m], lane);
            store4(dS0 + (bh * DK + f0 + 4 * lq + (lr & 3)) * dv + j0 + c0 + 4 * (lr >> 2), x);
        }
    }
}

// compute units of the current device (cached per device; 256 if the query fails)
int64_t num_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (dev >= 0 && dev < 64) cache[dev] = cus;
    return cus;
}

template <int C, int DK, int DV, typename TQ, typename TD>
hipError_t bwd_typed(const BwdArgs &a, hipStream_t stream) {
    const int64_t nch = (a.T + C - 1) / C;
    // forward states at every chunk start (the matrix-core forward for bf16 inputs, the fp32
    // one for fp32 inputs), unless the caller passes those of its forward
    if (nch > 0 && !a.states_given) {
        ChunkArgs f{a.q, a.k, a.v, a.d, a.beta, a.alpha, a.S0, nullptr, nullptr, a.BH, a.T, DK,
                    DV, C, a.qkv, a.d_dtype};
        f.ckpt = a.Mck;
        f.uout = a.Uck;
        const hipError_t e = sizeof(TQ) == 2 ? launch_chunk_fwd_mfma(f, stream)
                                             : launch_chunk_fwd_f32math(f, stream);
        if (e != hipSuccess) return e;
    }
    constexpr int BVA = 32;  // value slice of the reverse pass
    if constexpr (sizeof(TQ) == 2) {
        if (nch > 0) {
            hipLaunchKernelGGL((bwd_tinv_kernel<DK, TD>), dim3(static_cast<unsigned>(a.BH * nch)),
                               dim3(NT), 0, stream, static_cast<const bf16_t *>(a.q),
                               static_cast<const bf16_t *>(a.k), static_cast<const TD *>(a.d),
                               a.beta, a.alpha, a.Tck, a.T, nch);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL((bwd_state_mfma_kernel<DK, BVA>),
                           dim3(static_cast<unsigned>(a.BH * (DV / BVA))), dim3(2 * NT), 0, stream,
                           static_cast<const bf16_t *>(a.q), static_cast<const bf16_t *>(a.k),
                           a.beta, a.alpha,
                           static_cast<const bf16_t *>(a.dO), a.dS_T, a.Tck,
                           static_cast<uint16_t *>(a.dMck), a.dRck, static_cast<bf16_t *>(a.gv),
                           a.dS0, a.T, DV);
    } else
    hipLaunchKernelGGL((bwd_state_kernel<C, DK, BVA, TQ, TD>),
                       dim3(static_cast<unsigned>(a.BH * (DV / BVA))), dim3(NT), 0, stream,
                       static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),
                       static_cast<const TD *>(a.d), a.beta, a.alpha,
                       static_cast<const TQ *>(a.dO), a.dS_T, static_cast<float *>(a.dMck), a.dS0,
                       a.T, DV);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nch == 0) return e;
    if constexpr (sizeof(TQ) == 2) {
        // persistent: one workgroup per CU (its LDS allows no more), each taking every
        // grid-th chunk
        const int64_t total = a.BH * nch;
        const int64_t grid = total < num_cus() ? total : num_cus();
        hipLaunchKernelGGL((bwd_chunk_mfma_kernel<DK, DV, TD>),
                           dim3(static_cast<unsigned>(grid)), dim3(2 * NT), 0, stream,
                           static_cast<const bf16_t *>(a.q), static_cast<const bf16_t *>(a.k),
                           static_cast<const bf16_t *>(a.v), static_cast<const TD *>(a.d),
                           a.beta, a.alpha, static_cast<const bf16_t *>(a.dO),
                           static_cast<const uint16_t *>(a.Mck), static_cast<const uint16_t *>(a.dMck),
                           a.Tck, a.Uck, a.dRck, static_cast<bf16_t *>(a.gq),
                           static_cast<bf16_t *>(a.gk), a.gbeta, static_cast<TD *>(a.gd),
                           a.galpha, a.T, nch, total);
    } else {
        constexpr int BVB = 32;  // value slice of the fp32 per-chunk pass
        hipLaunchKernelGGL((bwd_chunk_kernel<C, DK, DV, BVB, TQ, TD>),
                           dim3(static_cast<unsigned>(a.BH * nch)), dim3(NT), 0, stream,
                           static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),
                           static_cast<const TQ *>(a.v), static_cast<const TD *>(a.d), a.beta,
                           a.alpha, static_cast<const TQ *>(a.dO), static_cast<const float *>(a.Mck),
                           static_cast<const float *>(a.dMck),
                           static_cast<TQ *>(a.gq), static_cast<TQ *>(a.gk),
                           static_cast<TQ *>(a.gv), a.gbeta, static_cast<TD *>(a.gd), a.galpha,
                           a.T, nch);
    }
    return hipGetLastError();
}

// bf16 inputs use 64-row chunks, fp32 inputs 32-row chunks (their fp32 tiles take twice
// the LDS)
template <typename TQ, int DK, int DV>
hipError_t bwd_dtypes(const BwdArgs &a, hipStream_t stream) {
    constexpr int C = sizeof(TQ) == 2 ? 64 : 32;
    return a.d_dtype == OSDN_F32 ? bwd_typed<C, DK, DV, TQ, float>(a, stream)
                                 : bwd_typed<C, DK, DV, TQ, bf16_t>(a, stream);
}

template <typename TQ>
hipError_t bwd_dims(const BwdArgs &a, hipStream_t stream) {
    if (a.dk == 64) return a.dv == 64 ? bwd_dtypes<TQ, 64, 64>(a, stream) : bwd_dtypes<TQ, 64, 128>(a, stream);
    return a.dv == 64 ? bwd_dtypes<TQ, 128, 64>(a, stream) : bwd_dtypes<TQ, 128, 128>(a, stream);
}


// ---- the channel-wise gate: fp32 arithmetic for either input type, 32-row chunks ----------
// With a_t in [0,1]^dk scaling the key features of the state (Erase-then-Delta Attention,
// section 2.2, eq. 5), the forward's chunk algebra has per-feature decays: with Lg_r the
// running sum of ln a over the chunk's rows up to r (per feature, in double precision),
// G_r = e^{Lg_r}, rho_f(s -> r) = e^{Lg_rf - Lg_sf} and W_s = rho(s -> L) for the last row L,
//   AS[r,s] = sum_f k_rf k~_sf rho_f(s->r) (s < r),  P[r,s] = sum_f q_rf k~_sf rho_f(s->r) (s <= r),
//   U = (I + A)^{-1} diag(b) (V - (K o G) M0),  O = (Q o G) M0 + P U,
//   M_C = Diag(G_L) M0 + (K~ o W)^T U.
// Differentiating it gives, per chunk (dMC the gradient at its end):
//   dU = P^T dO + (K~ o W) dMC,   dR = (I + A)^{-T} dU,
//   dM0 = Diag(G_L) dMC + (Q o G)^T dO - (K o G)^T diag(b) dR,
//   dP = lower-inclusive(dO U^T),   dA = -strictly-lower(dR U^T),
//   dQ[r,f]  = G_rf (dO M0^T)[r,f] + sum_s dP[r,s] k~_sf rho_f(s->r),
//   dK'[r,f] = b_r (-G_rf (dR M0^T)[r,f] + sum_s dA[r,s] k~_sf rho_f(s->r)),
//   dK~[s,f] = W_sf (U dMC^T)[s,f] + sum_r (dP[r,s] q_rf + b_r dA[r,s] k_rf) rho_f(s->r),
//   db_r = <dR_r, v_r - ((K o G) M0)_r> + sum_s dA[r,s] AS[r,s],   dV = diag(b) dR,
//   dLg[r,f] = q_rf dQ + k_rf dK' - k~_rf dK~  (+ at r = L: G_Lf <dMC[f,:], M0[f,:]>
//              + sum_s k~_sf W_sf (U dMC^T)[s,f]),
//   d ln a_t = sum_{t <= r <= L} dLg[r],  da = d ln a / a,  dd = dK~ o K,  dK = dK' + dK~ o D.
// Every decay factor is e to a difference of running sums with the later row first, so at
// most 1.  Rows past the end are zero with gate 1 (ln a = 0) and beta = 0.

// Q, K, K~ = d (.) k in fp32 and ln a in double (zero rows, and ln a = 0, past the end), in two
// halves: the loads into registers (every one issued before any is used), then the LDS stores,
// so that a caller can keep the loads in flight across other work.  The registers hold the
// elements as loaded and are widened only when stored: a conversion at the load would make the
// wave wait for it there.
template <int C, int DK, typename TQ, typename TD>
struct QkGateRegs {
    static constexpr int IT = C * DK / NT;
    static_assert(IT * NT == C * DK, "tile layout");
    TQ q[IT], k[IT];
    TD d[IT];
    float a[IT];
};
template <int C, int DK, typename TQ, typename TD>
__device__ __forceinline__ void load_qk_regs(QkGateRegs<C, DK, TQ, TD> &x, const TQ *q, const TQ *k,
                                             const TD *d, const float *a, int64_t row0, int n,
                                             int tid) {
#pragma unroll
    for (int it = 0; it < QkGateRegs<C, DK, TQ, TD>::IT; ++it) {
        const int idx = tid + it * NT, r = idx / DK, f = idx % DK;
        const int64_t e = (row0 + (r < n ? r : 0)) * DK + f;
        x.q[it] = q[e];
        x.k[it] = k[e];
        x.d[it] = d[e];
        x.a[it] = a[e];
    }
}
template <int C, int DK, int PX, typename TQ, typename TD>
__device__ __forceinline__ void store_qk_lds(const QkGateRegs<C, DK, TQ, TD> &x, int n, float *sQ,
                                             float *sK, float *sKt, double *sLg, int tid) {
#pragma unroll
    for (int it = 0; it < QkGateRegs<C, DK, TQ, TD>::IT; ++it) {
        const int idx = tid + it * NT, r = idx / DK, f = idx % DK;
        const bool in = r < n;
        const float qv = to_f32(x.q[it]), kv = to_f32(x.k[it]);
        sQ[r * PX + f] = in ? qv : 0.f;
        sK[r * PX + f] = in ? kv : 0.f;
        sKt[r * PX + f] = in ? to_f32(x.d[it]) * kv : 0.f;
        sLg[r * PX + f] = in ? log(fmax(static_cast<double>(x.a[it]), 1e-300)) : 0.0;
    }
}
template <int C, int DK, int PX, typename TQ, typename TD>
__device__ __forceinline__ void load_qk_gate(const TQ *q, const TQ *k, const TD *d,
                                             const float *a, int64_t row0, int n, float *sQ,
                                             float *sK, float *sKt, double *sLg, int tid) {
    QkGateRegs<C, DK, TQ, TD> x;
    load_qk_regs<C, DK>(x, q, k, d, a, row0, n, tid);
    store_qk_lds<C, DK, PX>(x, n, sQ, sK, sKt, sLg, tid);
}

// ln a -> its running sum down each feature column (the threads of the first DK lanes); the
// column is read whole before the sums, so the reads do not wait on one another
template <int C, int DK, int PX>
__device__ __forceinline__ void gate_scan(double *sLg, int tid) {
    if (tid < DK) {
        double x[C];
#pragma unroll
        for (int r = 0; r < C; ++r) x[r] = sLg[r * PX + tid];
        double acc = 0.0;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            acc += x[r];
            sLg[r * PX + tid] = acc;
        }
    }
}

// AS (strictly lower) and P (lower-inclusive) with the per-feature decay inside the sum
template <int C, int DK, int PX, int PC>
__device__ __forceinline__ void scores_gate(const float *sQ, const float *sK, const float *sKt,
                                            const double *sLg, float *sAS, float *sP, int tid) {
    constexpr int TM = C / 16;
    const int i0 = (tid / 16) * TM, j0 = (tid % 16) * TM;
    float ak[TM][TM], aq[TM][TM];
    zero(ak);
    zero(aq);
    if (j0 <= i0 + TM - 1) {  // tiles wholly above the diagonal stay zero
#pragma unroll 4
        for (int f = 0; f < DK; ++f) {
            float qv[TM], kv[TM], tv[TM];
            double lr[TM], ls[TM];
#pragma unroll
            for (int m = 0; m < TM; ++m) {
                qv[m] = sQ[(i0 + m) * PX + f];
                kv[m] = sK[(i0 + m) * PX + f];
                lr[m] = sLg[(i0 + m) * PX + f];
                tv[m] = sKt[(j0 + m) * PX + f];
                ls[m] = sLg[(j0 + m) * PX + f];
            }
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int nn = 0; nn < TM; ++nn) {
                    if (j0 + nn <= i0 + m) {
                        const float e = __expf(static_cast<float>(lr[m] - ls[nn])) * tv[nn];
                        ak[m][nn] += kv[m] * e;
                        aq[m][nn] += qv[m] * e;
                    }
                }
        }
    }
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int nn = 0; nn < TM; ++nn) {
            const int i = i0 + m, j = j0 + nn;
            sAS[i * PC + j] = j < i ? ak[m][nn] : 0.f;
            sP[i * PC + j] = j <= i ? aq[m][nn] : 0.f;
        }
}

// The score tiles AS and P of every 32-row chunk with the channel-wise gate, and
// T = (I + diag(beta) AS)^{-1}, one workgroup per (sequence, chunk), into
// [BH, nchunks, kGateTiles, C, C] fp32: they depend on q, k, d, beta and the gate only, so the
// forward, the reverse pass (in each of its value slices) and the per-chunk pass load them.
template <int C, int DK, typename TQ, typename TD>
__global__ void __launch_bounds__(NT)
bwd_scores_gate_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k,
                       const TD *__restrict__ d, const float *__restrict__ beta,
                       const float *__restrict__ alpha_ch, float *__restrict__ scores,
                       int64_t T, int64_t nch) {
    constexpr int PX = DK + 1, PC = C + 1;
    __shared__ float sQ[C * PX], sK[C * PX], sKt[C * PX];
    __shared__ double sLg[C * PX];
    __shared__ float sAS[C * PC], sP[C * PC], sT[C * PC], sb[C];
    const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
    const int64_t c0 = c * C, row0 = bh * T + c0;
    const int n = static_cast<int>(T - c0 < C ? T - c0 : C);
    const int tid = threadIdx.x;
    load_qk_gate<C, DK, PX>(q, k, d, alpha_ch, row0, n, sQ, sK, sKt, sLg, tid);
    if (tid < C) sb[tid] = tid < n ? beta[row0 + tid] : 0.f;
    for (int idx = tid; idx < C * C; idx += NT) sT[(idx / C) * PC + idx % C] = idx / C == idx % C;
    __syncthreads();
    gate_scan<C, DK, PX>(sLg, tid);
    __syncthreads();
    scores_gate<C, DK, PX, PC>(sQ, sK, sKt, sLg, sAS, sP, tid);
    __syncthreads();
    // T: the forward substitution on the identity's columns
    solve_lower<C, C, PC, PC>(sT, sAS, sb, tid);
    __syncthreads();
    float *dst = scores + (bh * nch + c) * kGateTiles * C * C;
    for (int idx = tid; idx < C * C; idx += NT) {
        const int i = idx / C, j = idx % C;
        dst[idx] = sAS[i * PC + j];
        dst[C * C + idx] = sP[i * PC + j];
        dst[2 * C * C + idx] = sT[i * PC + j];
    }
}

// Reverse pass over chunks with the channel-wise gate: one workgroup per (sequence, BV-wide
// value slice), dM[:, slice] in LDS; dMck[c] gets the gradient at the end of chunk c.
template <int C, int DK, int BV, typename TQ, typename TD>
__global__ void __launch_bounds__(NT)
bwd_state_gate_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k,
                      const TD *__restrict__ d, const float *__restrict__ beta,
                      const float *__restrict__ alpha_ch, const TQ *__restrict__ dO,
                      const float *__restrict__ dS_T, const float *__restrict__ scores,
                      float *__restrict__ dMck, float *__restrict__ dS0, int64_t T, int dv) {
    constexpr int PX = DK + 1, PC = C + 1, PS = BV + 1;
    __shared__ float sQ[C * PX], sK[C * PX], sKt[C * PX];
    __shared__ double sLg[C * PX];
    __shared__ float sTi[C * PC], sP[C * PC];
    __shared__ float sdO[C * PS], sX[C * PS], sdM[DK * PS];
    __shared__ float sb[C], sGL[DK];

    const int nvt = dv / BV;
    const int64_t bh = blockIdx.x / nvt;
    const int j0 = static_cast<int>(blockIdx.x % nvt) * BV;
    const int tid = threadIdx.x;
    const int64_t nch = (T + C - 1) / C;
    // the products run on the fp32 matrix cores (16x16x4): wave wv, lane (lg, l16)
    static_assert(C == 32 && BV == 32 && DK % 64 == 0 && NT == 256, "matrix-core layout");
    const int lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

    for (int idx = tid; idx < DK * BV; idx += NT) {
        const int f = idx / BV, j = idx % BV;
        sdM[f * PS + j] = dS_T ? dS_T[(bh * DK + f) * dv + j0 + j] : 0.f;
    }
    // the next chunk's (c - 1's) inputs are loaded into registers while chunk c is processed; the
    // barriers wait for LDS only (the kernel reads back none of its global writes), so those
    // loads stay in flight across them
    constexpr int OIT = C * BV / NT;
    static_assert(OIT * NT == C * BV, "dO tile layout");
    constexpr int SIT = C * C / NT;  // score-tile elements per thread
    static_assert(SIT * NT == C * C, "score tile layout");
    QkGateRegs<C, DK, TQ, TD> nx;
    TQ ndo[OIT];
    float nti[SIT], np[SIT], nbt = 0.f;
    auto issue = [&](int64_t cc) __attribute__((always_inline)) {
        const int64_t r0 = bh * T + cc * C;
        const int nn = static_cast<int>(T - cc * C < C ? T - cc * C : C);
        const float *sc = scores + (bh * nch + cc) * kGateTiles * C * C;
#pragma unroll
        for (int it = 0; it < SIT; ++it) {
            nti[it] = sc[2 * C * C + tid + it * NT];  // T
            np[it] = sc[C * C + tid + it * NT];
        }
        load_qk_regs<C, DK>(nx, q, k, d, alpha_ch, r0, nn, tid);
#pragma unroll
        for (int it = 0; it < OIT; ++it) {
            const int idx = tid + it * NT, r = idx / BV, j = idx % BV;
            ndo[it] = dO[(r0 + (r < nn ? r : 0)) * dv + j0 + j];
        }
        nbt = tid < nn ? beta[r0 + tid] : 0.f;  // (beta past the end is 0)
    };
    if (nch > 0) issue(nch - 1);
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t c0 = c * C;
        const int n = static_cast<int>(T - c0 < C ? T - c0 : C);
        block_sync();  // the previous chunk is done with every buffer
        store_qk_lds<C, DK, PX>(nx, n, sQ, sK, sKt, sLg, tid);
#pragma unroll
        for (int it = 0; it < OIT; ++it) {
            const int idx = tid + it * NT, r = idx / BV, j = idx % BV;
            sdO[r * PS + j] = r < n ? to_f32(ndo[it]) : 0.f;
        }
#pragma unroll
        for (int it = 0; it < SIT; ++it) {
            const int idx = tid + it * NT, i = idx / C, j = idx % C;
            sTi[i * PC + j] = nti[it];
            sP[i * PC + j] = np[it];
        }
        if (tid < C) sb[tid] = nbt;
        if (c > 0) issue(c - 1);
#pragma unroll
        for (int it = 0; it < DK * BV / NT; ++it) {  // the gradient at this chunk's end
            const int idx = tid + it * NT, f = idx / BV, j = idx % BV;
            dMck[((bh * nch + c) * DK + f) * dv + j0 + j] = sdM[f * PS + j];
        }
        block_sync();
        gate_scan<C, DK, PX>(sLg, tid);
        block_sync();
        // in place: Q o G, K o G, K~ o W; and G_L
#pragma unroll
        for (int it = 0; it < C * DK / NT; ++it) {
            const int idx = tid + it * NT, r = idx / DK, f = idx % DK;
            const double lg = sLg[r * PX + f], lgL = sLg[(C - 1) * PX + f];
            const float g = __expf(static_cast<float>(lg));
            sQ[r * PX + f] *= g;
            sK[r * PX + f] *= g;
            sKt[r * PX + f] *= __expf(static_cast<float>(lgL - lg));
        }
        if (tid < DK) sGL[tid] = __expf(static_cast<float>(sLg[(C - 1) * PX + tid]));
        block_sync();
        {  // dU = (K~ o W) dM + P^T dO on the fp32 matrix cores: wave wv takes tile (wv / 2, wv % 2)
            const int ri = 16 * (wv >> 1) + l16, cj = 16 * (wv & 1) + l16;
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int t = 0; t < DK / 4; ++t)
                acc = mfma4f(sKt[ri * PX + 4 * t + lg], sdM[(4 * t + lg) * PS + cj], acc);
#pragma unroll
            for (int t = 0; t < C / 4; ++t)
                acc = mfma4f(sP[(4 * t + lg) * PC + ri], sdO[(4 * t + lg) * PS + cj], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) sX[(16 * (wv >> 1) + 4 * lg + e) * PS + cj] = acc[e];
        }
        block_sync();
        {  // dR = T^T dU on the fp32 matrix cores: wave wv takes tile (wv / 2, wv % 2)
            const int ri = 16 * (wv >> 1) + l16, cj = 16 * (wv & 1) + l16;
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < C / 4; ++t)
                acc = mfma4f(sTi[(4 * t + lg) * PC + ri], sX[(4 * t + lg) * PS + cj], acc);
            block_sync();  // every wave has read dU
#pragma unroll
            for (int e = 0; e < 4; ++e) sX[(16 * (wv >> 1) + 4 * lg + e) * PS + cj] = acc[e];
        }
        block_sync();
        {  // dM <- Diag(G_L) dM + (Q o G)^T dO - (K o G)^T diag(b) dR on the fp32 matrix cores:
           // wave wv takes feature tiles FW wv .. FW wv + FW - 1 and both column tiles
            constexpr int FW = DK / 64;
            v4f acc[FW][2];
#pragma unroll
            for (int ft = 0; ft < FW; ++ft) acc[ft][0] = acc[ft][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < C / 4; ++t) {
                const int r = 4 * t + lg;
                const float b0 = sdO[r * PS + l16], b1 = sdO[r * PS + 16 + l16];
#pragma unroll
                for (int ft = 0; ft < FW; ++ft) {
                    const float a = sQ[r * PX + 16 * (FW * wv + ft) + l16];
                    acc[ft][0] = mfma4f(a, b0, acc[ft][0]);
                    acc[ft][1] = mfma4f(a, b1, acc[ft][1]);
                }
            }
#pragma unroll
            for (int t = 0; t < C / 4; ++t) {
                const int r = 4 * t + lg;
                const float b0 = -sb[r] * sX[r * PS + l16], b1 = -sb[r] * sX[r * PS + 16 + l16];
#pragma unroll
                for (int ft = 0; ft < FW; ++ft) {
                    const float a = sK[r * PX + 16 * (FW * wv + ft) + l16];
                    acc[ft][0] = mfma4f(a, b0, acc[ft][0]);
                    acc[ft][1] = mfma4f(a, b1, acc[ft][1]);
                }
            }
#pragma unroll
            for (int ft = 0; ft < FW; ++ft)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = 16 * (FW * wv + ft) + 4 * lg + e;
                        float &x = sdM[f * PS + 16 * ct + l16];
                        x = sGL[f] * x + acc[ft][ct][e];
                    }
        }
    }
    block_sync();
    if (dS0) {
        for (int idx = tid; idx < DK * BV; idx += NT) {
            const int f = idx / BV, j = idx % BV;
            dS0[(bh * DK + f) * dv + j0 + j] = sdM[f * PS + j];
        }
    }
}

// Per-chunk gradients with the channel-wise gate: one workgroup per (sequence, chunk), the
// value columns taken BV at a time.
template <int C, int DK, int DV, int BV, typename TQ, typename TD>
__global__ void __launch_bounds__(NT)
bwd_chunk_gate_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k,
                      const TQ *__restrict__ v, const TD *__restrict__ d,
                      const float *__restrict__ beta, const float *__restrict__ alpha_ch,
                      const TQ *__restrict__ dO, const float *__restrict__ Mck,
                      const float *__restrict__ dMck, const float *__restrict__ scores,
                      TQ *__restrict__ gq, TQ *__restrict__ gk,
                      TQ *__restrict__ gv, float *__restrict__ gbeta, TD *__restrict__ gd,
                      float *__restrict__ galpha_ch, int64_t T, int64_t nch) {
    constexpr int PX = DK + 1, PC = C + 1, PS = BV + 1;
    constexpr int TC = C / 16, TK = DK / 16;  // register blocks
    constexpr int FPT = DK * BV / NT;                        // (f, j) pairs per thread
    static_assert(FPT * NT == DK * BV && NT % BV == 0, "slice layout");
    // raw Q, K, K~; K o G and K~ o W for the slice products (K o G is reused for dLg)
    __shared__ float sQ[C * PX], sK[C * PX], sKt[C * PX], sKg[C * PX], sKw[C * PX];
    __shared__ double sLg[C * PX];
    __shared__ float sAS[C * PC], sP[C * PC];  // AS, P; after the slices b dA and dP
    __shared__ float sM0[DK * PS], sdM[DK * PS];
    __shared__ float sY[C * PS], sdO[C * PS], sU[C * PS], sdR[C * PS];
    __shared__ float sb[C], sdb[C], sLast[DK];
    __shared__ float sT[C * PC];  // T = (I + A)^{-1} (from the score-tile kernel) for every slice

    const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
    const int64_t c0 = c * C, row0 = bh * T + c0;
    const int n = static_cast<int>(T - c0 < C ? T - c0 : C);
    const int tid = threadIdx.x;
    const int ti = tid / 16, tj = tid % 16;
    const float *M0 = Mck + (bh * nch + c) * DK * DV;
    const float *dMC = dMck + (bh * nch + c) * DK * DV;

    // the chunk's score tiles (from the score-tile kernel), loads issued first
    constexpr int SIT = C * C / NT;
    static_assert(SIT * NT == C * C, "score tile layout");
    float tas[SIT], tp[SIT], tt[SIT];
    {
        const float *sc = scores + (bh * nch + c) * kGateTiles * C * C;
#pragma unroll
        for (int it = 0; it < SIT; ++it) {
            tas[it] = sc[tid + it * NT];
            tp[it] = sc[C * C + tid + it * NT];
            tt[it] = sc[2 * C * C + tid + it * NT];
        }
    }
    load_qk_gate<C, DK, PX>(q, k, d, alpha_ch, row0, n, sQ, sK, sKt, sLg, tid);
#pragma unroll
    for (int it = 0; it < SIT; ++it) {
        const int idx = tid + it * NT, i = idx / C, j = idx % C;
        sAS[i * PC + j] = tas[it];
        sP[i * PC + j] = tp[it];
        sT[i * PC + j] = tt[it];
    }
    if (tid < C) {
        sb[tid] = tid < n ? beta[row0 + tid] : 0.f;
        sdb[tid] = 0.f;
    }
    block_sync();
    gate_scan<C, DK, PX>(sLg, tid);
    block_sync();
#pragma unroll
    for (int it = 0; it < C * DK / NT; ++it) {
        const int idx = tid + it * NT, r = idx / DK, f = idx % DK;
        const double lg = sLg[r * PX + f], lgL = sLg[(C - 1) * PX + f];
        sKg[r * PX + f] = sK[r * PX + f] * __expf(static_cast<float>(lg));
        sKw[r * PX + f] = sKt[r * PX + f] * __expf(static_cast<float>(lgL - lg));
    }

    // The slice products run on the fp32 matrix cores (16x16x4): wave wv, lane (lg, l16).
    static_assert(C == 32 && BV == 16 && DK % 64 == 0 && NT == 256, "matrix-core slice layout");
    constexpr int FT = DK / 64;  // feature tiles of dQ, dK', dK~ per wave
    const int lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // dQ, -dK' (before b), dK~ (before W): row tile x this wave's feature tiles 16 (FT wv + ft);
    // mS: this wave's tiles of dP, dA (the tile above the diagonal is masked off below, so it is
    // not formed: wave w takes slots 2w, 2w + 1 of dP(0,0), dP(1,0), dP(1,1), dA(0,0), dA(1,0),
    // dA(1,1))
    v4f mQ[2][FT], mK[2][FT], mKt[2][FT], mS[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        mS[rt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
            mQ[rt][ft] = v4f{0.f, 0.f, 0.f, 0.f};
            mK[rt][ft] = v4f{0.f, 0.f, 0.f, 0.f};
            mKt[rt][ft] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    }
    float frob[FPT];  // this thread's parts of <dMC[f,:], M0[f,:]>, f = tid / BV + i NT / BV
#pragma unroll
    for (int i = 0; i < FPT; ++i) frob[i] = 0.f;
    // the next slice's inputs are loaded into registers while the current one is processed (as
    // loaded: a conversion would wait for them); the barriers wait for LDS only, since the kernel
    // reads back none of its global writes
    constexpr int YIT = C * BV / NT;
    static_assert(YIT * NT == C * BV, "slice tile layout");
    float pm0[FPT], pdm[FPT];
    TQ pv[YIT], pdo[YIT];
    auto fetch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FPT; ++i) {
            const int idx = tid + i * NT, f = idx / BV, j = idx % BV;
            pm0[i] = M0[f * DV + s0 + j];
            pdm[i] = dMC[f * DV + s0 + j];
        }
#pragma unroll
        for (int i = 0; i < YIT; ++i) {
            const int idx = tid + i * NT, r = idx / BV, j = idx % BV;
            const int64_t e = (row0 + (r < n ? r : 0)) * DV + s0 + j;
            pv[i] = v[e];
            pdo[i] = dO[e];
        }
    };
    fetch(0);

    for (int s0 = 0; s0 < DV; s0 += BV) {
        block_sync();  // the previous slice (and the scaled copies) are done
#pragma unroll
        for (int i = 0; i < FPT; ++i) {
            const int idx = tid + i * NT, f = idx / BV, j = idx % BV;
            sM0[f * PS + j] = pm0[i];
            sdM[f * PS + j] = pdm[i];
            frob[i] += pm0[i] * pdm[i];
        }
#pragma unroll
        for (int i = 0; i < YIT; ++i) {
            const int idx = tid + i * NT, r = idx / BV, j = idx % BV;
            sY[r * PS + j] = r < n ? to_f32(pv[i]) : 0.f;
            sdO[r * PS + j] = r < n ? to_f32(pdo[i]) : 0.f;
        }
        if (s0 + BV < DV) fetch(s0 + BV);
        block_sync();
        {  // waves 0, 1: Y = V - (K o G) M0 on row tile wv, R = b Y into U;
           // waves 2, 3: dU = (K~ o W) dMC + P^T dO on row tile wv - 2, into dR
            const int rt = wv & 1, ri = 16 * rt + l16;
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            if (wv < 2) {
#pragma unroll 8
                for (int t = 0; t < DK / 4; ++t)
                    acc = mfma4f(sKg[ri * PX + 4 * t + lg], sM0[(4 * t + lg) * PS + l16], acc);
            } else {
#pragma unroll 8
                for (int t = 0; t < DK / 4; ++t)
                    acc = mfma4f(sKw[ri * PX + 4 * t + lg], sdM[(4 * t + lg) * PS + l16], acc);
#pragma unroll
                for (int t = 0; t < C / 4; ++t)
                    acc = mfma4f(sP[(4 * t + lg) * PC + ri], sdO[(4 * t + lg) * PS + l16], acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * lg + e;
                if (wv < 2) {
                    const float y = sY[r * PS + l16] - acc[e];
                    sY[r * PS + l16] = y;
                    sU[r * PS + l16] = sb[r] * y;
                } else {
                    sdR[r * PS + l16] = acc[e];
                }
            }
        }
        block_sync();
        {  // waves 0, 1: U = T R on row tile wv; waves 2, 3: dR = T^T dU on row tile wv - 2
            const int rt = wv & 1, ri = 16 * rt + l16;
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            if (wv < 2) {
#pragma unroll
                for (int t = 0; t < C / 4; ++t)
                    acc = mfma4f(sT[ri * PC + 4 * t + lg], sU[(4 * t + lg) * PS + l16], acc);
            } else {
#pragma unroll
                for (int t = 0; t < C / 4; ++t)
                    acc = mfma4f(sT[(4 * t + lg) * PC + ri], sdR[(4 * t + lg) * PS + l16], acc);
            }
            block_sync();  // every wave has read R and dU
            float *dst = wv < 2 ? sU : sdR;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(16 * rt + 4 * lg + e) * PS + l16] = acc[e];
        }
        block_sync();
        for (int idx = tid; idx < C * BV; idx += NT) {
            const int r = idx / BV, j = idx % BV;
            if (r < n) gv[(row0 + r) * DV + s0 + j] = from_f32<TQ>(sb[r] * sdR[r * PS + j]);
        }
        if (tid < C) {  // <dR_r, y_r> of this slice
            float db = 0.f;
            for (int j = 0; j < BV; ++j) db += sdR[tid * PS + j] * sY[tid * PS + j];
            sdb[tid] += db;
        }
        {  // dP += dO U^T, dA += dR U^T, dQ += dO M0^T, dK' -= dR M0^T, dK~ += U dMC^T
            float fO[2][4], fR[2][4], fU[2][4], fM[FT][4], fD[FT][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const int o = (16 * rt + l16) * PS + 4 * t + lg;
                    fO[rt][t] = sdO[o];
                    fR[rt][t] = sdR[o];
                    fU[rt][t] = sU[o];
                }
#pragma unroll
                for (int ft = 0; ft < FT; ++ft) {
                    const int o = (16 * (FT * wv + ft) + l16) * PS + 4 * t + lg;
                    fM[ft][t] = sM0[o];
                    fD[ft][t] = sdM[o];
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int ft = 0; ft < FT; ++ft) {
                        mQ[rt][ft] = mfma4f(fO[rt][t], fM[ft][t], mQ[rt][ft]);
                        mK[rt][ft] = mfma4f(fR[rt][t], fM[ft][t], mK[rt][ft]);
                        mKt[rt][ft] = mfma4f(fU[rt][t], fD[ft][t], mKt[rt][ft]);
                    }
#pragma unroll
            for (int slot = 0; slot < 2; ++slot) {
                const int sel = 2 * wv + slot;  // wave-uniform
                if (sel < 6) {
                    const bool isA = sel >= 3, r1 = sel % 3 != 0, c1 = sel % 3 == 2;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float a = isA ? (r1 ? fR[1][t] : fR[0][t])
                                            : (r1 ? fO[1][t] : fO[0][t]);
                        mS[slot] = mfma4f(a, c1 ? fU[1][t] : fU[0][t], mS[slot]);
                    }
                }
            }
        }
    }
    // the matrix-core tiles into the register blocks below, one C x DK (or C x C) product at a
    // time through the K~ o W rows, which are no longer read
    const int ic = ti * TC, jc = tj * TC;  // C x C block
    // C x DK block: rows ik.., features tj + 16 nn (the 16 lanes of a row pair read 16
    // consecutive features, so their LDS reads of a row are free of bank conflicts)
    const int ik = ti * TC;
    auto fk = [&](int nn) __attribute__((always_inline)) { return tj + 16 * nn; };
    float aQ[TC][TK], aK[TC][TK], aKt[TC][TK], adP[TC][TC], adA[TC][TC];
    auto spill_ck = [&](const v4f (&m)[2][FT], float sign, float (&out)[TC][TK])
        __attribute__((always_inline)) {
        block_sync();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sKw[(16 * rt + 4 * lg + e) * PX + 16 * (FT * wv + ft) + l16] =
                        sign * m[rt][ft][e];
        block_sync();
#pragma unroll
        for (int m_ = 0; m_ < TC; ++m_)
#pragma unroll
            for (int nn = 0; nn < TK; ++nn) out[m_][nn] = sKw[(ik + m_) * PX + fk(nn)];
    };
    spill_ck(mQ, 1.f, aQ);
    spill_ck(mK, -1.f, aK);
    spill_ck(mKt, 1.f, aKt);
    auto spill_cc = [&](bool isA, float (&out)[TC][TC]) __attribute__((always_inline)) {
        block_sync();
#pragma unroll
        for (int slot = 0; slot < 2; ++slot) {
            const int sel = 2 * wv + slot;
            if (sel < 6 && (sel >= 3) == isA) {
                const int r1 = sel % 3 != 0, c1 = sel % 3 == 2;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sKw[(16 * r1 + 4 * lg + e) * PC + 16 * c1 + l16] = mS[slot][e];
            }
        }
        block_sync();
#pragma unroll
        for (int m_ = 0; m_ < TC; ++m_)
#pragma unroll
            for (int nn = 0; nn < TC; ++nn) {
                // the tile above the diagonal is never written; it is masked off below
                out[m_][nn] = (ic + m_) / 16 >= (jc + nn) / 16 ? sKw[(ic + m_) * PC + jc + nn] : 0.f;
            }
    };
    spill_cc(false, adP);
    spill_cc(true, adA);
    // the gates for d ln a / a at the end, loaded now so that the loads are done by then
    float ra[C];
    if (tid < DK && galpha_ch) {
#pragma unroll
        for (int r = 0; r < C; ++r) ra[r] = alpha_ch[(row0 + (r < n ? r : 0)) * DK + tid];
    }
    // G_L <dMC[f,:], M0[f,:]> per feature: the BV threads of one f are adjacent lanes
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
#pragma unroll
        for (int m = 1; m < BV; m <<= 1) frob[i] += __shfl_xor(frob[i], m);
        const int f = tid / BV + i * (NT / BV);
        if (tid % BV == 0)
            sLast[f] = __expf(static_cast<float>(sLg[(C - 1) * PX + f])) * frob[i];
    }
    // dP (lower-inclusive), dA (strictly lower, negated); db_r += sum_s dA[r,s] AS[r,s]
    {
        float rowb[TC];
#pragma unroll
        for (int m = 0; m < TC; ++m) {
            rowb[m] = 0.f;
#pragma unroll
            for (int nn = 0; nn < TC; ++nn) {
                const int i = ic + m, j = jc + nn;
                adP[m][nn] = j <= i ? adP[m][nn] : 0.f;
                adA[m][nn] = j < i ? -adA[m][nn] : 0.f;
                rowb[m] += adA[m][nn] * sAS[i * PC + j];
            }
#pragma unroll
            for (int w = 1; w < 16; w <<= 1) rowb[m] += __shfl_xor(rowb[m], w);
        }
        block_sync();  // every slice product and every read of AS is done
        if (tj == 0) {
#pragma unroll
            for (int m = 0; m < TC; ++m) sdb[ic + m] += rowb[m];
        }
#pragma unroll
        for (int m = 0; m < TC; ++m)
#pragma unroll
            for (int nn = 0; nn < TC; ++nn) {
                const int i = ic + m, j = jc + nn;
                sP[i * PC + j] = adP[m][nn];
                sAS[i * PC + j] = adA[m][nn] * sb[i];
            }
    }
    // the slice terms' decay factors: dQ G, dK' b G, dK~ W; then the column sums
    // sum_s k~_sf (W o U dMC^T)[s,f] of the last row's term, through LDS (sM0 as [16][DK])
    float *colpart = sM0;
    {
        float colk[TK];
#pragma unroll
        for (int nn = 0; nn < TK; ++nn) colk[nn] = 0.f;
#pragma unroll
        for (int m = 0; m < TC; ++m)
#pragma unroll
            for (int nn = 0; nn < TK; ++nn) {
                const int r = ik + m, f = fk(nn);
                const double lg = sLg[r * PX + f], lgL = sLg[(C - 1) * PX + f];
                const float g = __expf(static_cast<float>(lg));
                aQ[m][nn] *= g;
                aK[m][nn] *= sb[r] * g;
                aKt[m][nn] *= __expf(static_cast<float>(lgL - lg));
                colk[nn] += sKt[r * PX + f] * aKt[m][nn];
            }
#pragma unroll
        for (int nn = 0; nn < TK; ++nn) colpart[ti * DK + fk(nn)] = colk[nn];
    }
    block_sync();
    if (tid < DK) {
        float s = 0.f;
        for (int t = 0; t < 16; ++t) s += colpart[t * DK + tid];
        sLast[tid] += s;
    }
    // the score terms, with the decay of every (row, column, feature) inside:
    // dQ[r,f] += sum_s dP[r,s] k~_sf rho,  dK'[r,f] += sum_s b_r dA[r,s] k~_sf rho
    {
        double lr[TC][TK];
#pragma unroll
        for (int m = 0; m < TC; ++m)
#pragma unroll
            for (int nn = 0; nn < TK; ++nn) lr[m][nn] = sLg[(ik + m) * PX + fk(nn)];
        for (int s = 0; s <= ik + TC - 1; ++s) {
            float kt[TK];
            double ls[TK];
#pragma unroll
            for (int nn = 0; nn < TK; ++nn) {
                kt[nn] = sKt[s * PX + fk(nn)];
                ls[nn] = sLg[s * PX + fk(nn)];
            }
#pragma unroll
            for (int m = 0; m < TC; ++m) {
                const int r = ik + m;
                if (s <= r) {
                    const float dp = sP[r * PC + s], da = sAS[r * PC + s];
#pragma unroll
                    for (int nn = 0; nn < TK; ++nn) {
                        const float e = __expf(static_cast<float>(lr[m][nn] - ls[nn])) * kt[nn];
                        aQ[m][nn] += dp * e;
                        aK[m][nn] += da * e;
                    }
                }
            }
        }
    }
    // dK~[s,f] += sum_{r >= s} (dP[r,s] q_rf + b_r dA[r,s] k_rf) rho_f(s -> r)
    {
        double ls[TC][TK];
#pragma unroll
        for (int m = 0; m < TC; ++m)
#pragma unroll
            for (int nn = 0; nn < TK; ++nn) ls[m][nn] = sLg[(ik + m) * PX + fk(nn)];
        for (int r = ik; r < C; ++r) {
            float qv[TK], kv[TK];
            double lr[TK];
#pragma unroll
            for (int nn = 0; nn < TK; ++nn) {
                qv[nn] = sQ[r * PX + fk(nn)];
                kv[nn] = sK[r * PX + fk(nn)];
                lr[nn] = sLg[r * PX + fk(nn)];
            }
#pragma unroll
            for (int m = 0; m < TC; ++m) {
                const int s = ik + m;
                if (s <= r) {
                    const float dp = sP[r * PC + s], da = sAS[r * PC + s];
#pragma unroll
                    for (int nn = 0; nn < TK; ++nn) {
                        const float e = __expf(static_cast<float>(lr[nn] - ls[m][nn]));
                        aKt[m][nn] += (dp * qv[nn] + da * kv[nn]) * e;
                    }
                }
            }
        }
    }
    // outputs, and dLg into sKg (K o G is no longer read)
#pragma unroll
    for (int m = 0; m < TC; ++m) {
        const int r = ik + m;
#pragma unroll
        for (int nn = 0; nn < TK; ++nn) {
            const int f = fk(nn);
            const float qv = sQ[r * PX + f], kv = sK[r * PX + f], tv = sKt[r * PX + f];
            sKg[r * PX + f] = qv * aQ[m][nn] + kv * aK[m][nn] - tv * aKt[m][nn];
            if (r < n) {
                const int64_t e = (row0 + r) * DK + f;
                gq[e] = from_f32<TQ>(aQ[m][nn]);
                gk[e] = from_f32<TQ>(aK[m][nn] + aKt[m][nn] * to_f32(d[e]));
                gd[e] = from_f32<TD>(aKt[m][nn] * kv);
            }
        }
    }
    block_sync();
    if (tid < DK && galpha_ch) {  // d ln a_t = sum_{r >= t} dLg[r]; the last row's term at n-1
        float acc = sLast[tid];
#pragma unroll
        for (int r = C - 1; r >= 0; --r) {
            if (r < n) {
                acc += sKg[r * PX + tid];
                galpha_ch[(row0 + r) * DK + tid] = acc / ra[r];
            }
        }
    }
    if (tid < n) gbeta[row0 + tid] = sdb[tid];
}

// The backward with the channel-wise gate: the fp32 forward (its GATE variant, 32-row chunks)
// records the state at every chunk start, then the reverse pass and the per-chunk gradients.
template <int DK, int DV, typename TQ, typename TD>
hipError_t bwd_gate_typed(const BwdArgs &a, hipStream_t stream) {
    constexpr int C = 32;
    const int64_t nch = (a.T + C - 1) / C;
    if (nch > 0) {  // the score tiles of every chunk, then the forward, which takes them
        hipLaunchKernelGGL((bwd_scores_gate_kernel<C, DK, TQ, TD>),
                           dim3(static_cast<unsigned>(a.BH * nch)), dim3(NT), 0, stream,
                           static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),
                           static_cast<const TD *>(a.d), a.beta, a.alpha_ch, a.scores, a.T, nch);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        ChunkArgs f{a.q, a.k, a.v, a.d, a.beta, nullptr, a.S0, nullptr, nullptr, a.BH, a.T, DK,
                    DV, C, a.qkv, a.d_dtype};
        f.alpha_ch = a.alpha_ch;
        f.ckpt = a.Mck;
        f.gate_scores = a.scores;
        e = launch_chunk_fwd_f32math(f, stream);
        if (e != hipSuccess) return e;
    }
    constexpr int BVA = 32, BVB = 16;
    hipLaunchKernelGGL((bwd_state_gate_kernel<C, DK, BVA, TQ, TD>),
                       dim3(static_cast<unsigned>(a.BH * (DV / BVA))), dim3(NT), 0, stream,
                       static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),
                       static_cast<const TD *>(a.d), a.beta, a.alpha_ch,
                       static_cast<const TQ *>(a.dO), a.dS_T, a.scores,
                       static_cast<float *>(a.dMck), a.dS0, a.T, DV);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nch == 0) return e;
    hipLaunchKernelGGL((bwd_chunk_gate_kernel<C, DK, DV, BVB, TQ, TD>),
                       dim3(static_cast<unsigned>(a.BH * nch)), dim3(NT), 0, stream,
                       static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),
                       static_cast<const TQ *>(a.v), static_cast<const TD *>(a.d), a.beta,
                       a.alpha_ch, static_cast<const TQ *>(a.dO),
                       static_cast<const float *>(a.Mck), static_cast<const float *>(a.dMck),
                       a.scores, static_cast<TQ *>(a.gq), static_cast<TQ *>(a.gk),
                       static_cast<TQ *>(a.gv), a.gbeta, static_cast<TD *>(a.gd), a.galpha_ch,
                       a.T, nch);
    return hipGetLastError();
}

template <typename TQ, int DK, int DV>
hipError_t bwd_gate_dtypes(const BwdArgs &a, hipStream_t stream) {
    return a.d_dtype == OSDN_F32 ? bwd_gate_typed<DK, DV, TQ, float>(a, stream)
                                 : bwd_gate_typed<DK, DV, TQ, bf16_t>(a, stream);
}

template <typename TQ>
hipError_t bwd_gate_dims(const BwdArgs &a, hipStream_t stream) {
    if (a.dk == 64)
        return a.dv == 64 ? bwd_gate_dtypes<TQ, 64, 64>(a, stream)
                          : bwd_gate_dtypes<TQ, 64, 128>(a, stream);
    return a.dv == 64 ? bwd_gate_dtypes<TQ, 128, 64>(a, stream)
                      : bwd_gate_dtypes<TQ, 128, 128>(a, stream);
}

}  // namespace

int32_t bwd_chunk_size(osdn_dtype qkv) { return qkv == OSDN_BF16 ? 64 : 32; }

hipError_t launch_chunk_bwd(const BwdArgs &a, hipStream_t stream) {
    return a.qkv == OSDN_BF16 ? bwd_dims<bf16_t>(a, stream) : bwd_dims<float>(a, stream);
}

hipError_t launch_chunk_bwd_gate(const BwdArgs &a, hipStream_t stream) {
    return a.qkv == OSDN_BF16 ? bwd_gate_dims<bf16_t>(a, stream) : bwd_gate_dims<float>(a, stream);
}

}  // namespace osdn
