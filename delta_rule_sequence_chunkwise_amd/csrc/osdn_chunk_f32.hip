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
//   a3  R = diag(beta) (V - diag(e^g) K M)
//   a4  U = (I + A)^{-1} R, by forward substitution down the rows       (UT transform)
//   a5  P[r][s] = e^{g_r - g_s} <q_r, k~_s>  for s <= r                 (intra-chunk scores)
//   a6  O = diag(e^g) Q M + P U;  M <- e^{g_C} M + (diag(e^{g_C - g}) K~)^T U
//
// Rows past the end of the sequence are zero (beta = 0, alpha = 1), so they add nothing.
// For the backward the kernel can also record the state at every chunk start (and skip o).
// With the channel-wise gate a_t in R^dk (GATE; Erase-then-Delta Attention, section 2.2,
// eq. 5) the decay is per key feature: Lg_r = sum_{t<=r} ln a_t per feature, kept in double
// precision, and every ratio the chunk needs is formed as e^{Lg_r - Lg_s} <= 1 (for A and P
// in one pass, each once):
//   A[r][s] = beta_r sum_i k_ri k~_si e^{Lg_ri - Lg_si},  P[r][s] = sum_i q_ri k~_si e^{...},
//   R = diag(beta) (V - (K o e^{Lg}) M),  O = (Q o e^{Lg}) M + P U,
//   M <- Diag(e^{Lg_C}) M + (K~ o e^{Lg_C - Lg})^T U.
// A gate of 0 is taken as e^{-690}, which rounds every ratio across it to 0 in fp32.
#include "osdn_internal.h"
#include "osdn_mfma.h"

namespace osdn {
namespace {

constexpr int kThreads = 512;  // eight waves: two per SIMD, so one hides the other's LDS waits

// X <- (I + A)^{-1} X in place for a strictly lower C x C A (C rows, NC columns): row r of the
// result is X_r - sum_{s<r} A[r][s] (result)_s, taken row by row.  Column j is owned by TPC
// adjacent lanes; lane sub keeps rows s = i TPC + sub of the column in registers, so each row
// costs one short dot product and a reduction over the TPC lanes.
template <int C, int NC, int PX, int PA>
__device__ __forceinline__ void solve_unit_lower(float *X, const float *A, int tid) {
    constexpr int TPC = kThreads / NC, RPT = C / TPC;
    static_assert(TPC * NC == kThreads && RPT * TPC == C && TPC <= 16, "solve layout");
    const int j = tid / TPC, sub = tid % TPC;
    float mine[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) mine[i] = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            if (i * TPC < r) {
                const int s = i * TPC + sub;
                if (s < r) part += A[r * PA + s] * mine[i];
            }
        }
        part = group_sum<TPC>(part);  // on DPP (an LDS shuffle per step measured far slower)
        const float val = X[r * PX + j] - part;
        if (r % TPC == sub) mine[r / TPC] = val;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) X[(i * TPC + sub) * PX + j] = mine[i];
}

// acc[m][n] += sum_{kk < K} a(i0 + m, kk) * b(kk, j0 + n): a register-blocked product tile,
// each operand value read from LDS once per TN (or TM) products
template <int TM, int TN, int K, typename FA, typename FB>
__device__ __forceinline__ void tile_mm(float (&acc)[TM][TN], int i0, int j0, FA &&a, FB &&b) {
#pragma unroll 4
    for (int kk = 0; kk < K; ++kk) {
        float av[TM], bv[TN];
#pragma unroll
        for (int m = 0; m < TM; ++m) av[m] = a(i0 + m, kk);
#pragma unroll
        for (int nn = 0; nn < TN; ++nn) bv[nn] = b(kk, j0 + nn);
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int nn = 0; nn < TN; ++nn) acc[m][nn] += av[m] * bv[nn];
    }
}

template <int DK, int BV, int CH, typename TQ, typename TD, bool GATE>
__global__ void __launch_bounds__(kThreads)
chunk_f32math_kernel(const TQ *__restrict__ q, const TQ *__restrict__ k,
                     const TQ *__restrict__ v, const TD *__restrict__ d,
                     const float *__restrict__ beta, const float *__restrict__ alpha,
                     const float *S0, TQ *__restrict__ o, float *S_T, int64_t T, int dv,
                     float *__restrict__ ckpt, const float *__restrict__ gscores) {
    constexpr int PX = DK + 1;  // padded row pitches (bank-conflict relief)
    constexpr int PC = CH + 1;
    constexpr int PV = BV + 1;
    __shared__ float sX[CH * PX];   // K, later Q
    __shared__ float sKt[CH * PX];  // K~ = d (.) K
    __shared__ float sA[CH * PC];   // A, later P
    __shared__ float sM[DK * PV];   // state slice M[:, j0:j0+BV]
    __shared__ float sR[CH * PV];   // V, then R, then U
    __shared__ float sQM[CH * PV];  // Q M
    __shared__ float sg[CH];        // g (running log-decay)
    __shared__ float sb[CH];        // beta
    __shared__ float sgam[CH];      // e^{g_r}
    __shared__ float sdec[CH];      // e^{g_C - g_r}
    __shared__ double sLg[GATE ? CH * PX : 1];  // channel-wise gate: Lg per row and feature
    __shared__ float sQ[GATE ? CH * PX : 1];    // channel-wise gate: Q (A and P in one pass)
    __shared__ float sP[GATE ? CH * PC : 1];    // channel-wise gate: P (A stays in sA)
    auto decay = [&](int r, int i) __attribute__((always_inline)) {  // e^{Lg_r}
        return expf(static_cast<float>(sLg[r * PX + i]));
    };

    const int ntiles = dv / BV;
    const int64_t bh = blockIdx.x / ntiles;
    const int j0 = (blockIdx.x % ntiles) * BV;
    const int tid = threadIdx.x;
    // product tiles: thread (ty, tx) of a 32 x 16 grid owns rows ty TM.., columns tx TN..
    static_assert(kThreads == 512 && BV == 32, "tile layout");
    constexpr int TR = CH < 32 ? 1 : CH / 32;  // rows per thread of a CH-row product
    constexpr int TS = CH / 16;                // columns per thread of a CH x CH product
    constexpr int TD_ = DK / 32;               // rows per thread of the DK-row state update
    const int ty = tid >> 4, tx = tid & 15;
    const int ir = ty * TR;                    // first row of a CH-row tile (< CH: active)
    const bool rows_ok = ir < CH;
    auto zero_tile = [](auto &acc) __attribute__((always_inline)) {
        for (auto &row : acc)
            for (auto &x : row) x = 0.f;
    };

    for (int idx = tid; idx < DK * BV; idx += kThreads) {
        const int i = idx / BV, j = idx % BV;
        sM[i * PV + j] = S0 ? S0[(bh * DK + i) * dv + j0 + j] : 0.f;
    }

    // The next chunk's k, d, v, beta (and q and the gate with GATE; the scalar decay without)
    // are loaded into registers while the current chunk is processed.  The barriers wait for
    // LDS only (the kernel reads back none of its global writes), so those loads stay in flight
    // across them.  Rows past the end re-read the chunk's last row and are zeroed on the way in.
    // Score tiles given (GATE): the next chunk's AS and P come with them.  The registers hold the
    // elements as loaded and are widened only when stored: a conversion at the load would make
    // the wave wait for it there.
    constexpr int LIT = CH * DK / kThreads, VIT = CH * BV / kThreads;
    constexpr int SIT = (CH * CH + kThreads - 1) / kThreads;
    static_assert(LIT * kThreads == CH * DK && VIT * kThreads == CH * BV, "prefetch layout");
    TQ nk[LIT], nq[GATE ? LIT : 1], nv[VIT];
    TD nd[LIT];
    float na[GATE ? LIT : 1], nb = 0.f, nal = 0.f;
    float nsa[GATE ? SIT : 1], nsp[GATE ? SIT : 1];
    const int64_t nchunks = (T + CH - 1) / CH;
    auto issue = [&](int64_t cn) __attribute__((always_inline)) {
        const int nn = static_cast<int>(T - cn < CH ? T - cn : CH);
        const int64_t r0 = bh * T + cn;
        if constexpr (GATE) {
            if (gscores) {
                // AS and P, the first two of the chunk's three score tiles (the third is T)
                const float *sc = gscores + (bh * nchunks + cn / CH) * 3 * CH * CH;
#pragma unroll
                for (int it = 0; it < SIT; ++it) {
                    const int idx = tid + it * kThreads;
                    if (idx < CH * CH) {
                        nsa[it] = sc[idx];
                        nsp[it] = sc[CH * CH + idx];
                    }
                }
            }
        }
#pragma unroll
        for (int it = 0; it < LIT; ++it) {
            const int idx = tid + it * kThreads, r = idx / DK, i = idx % DK;
            const int64_t e = (r0 + (r < nn ? r : nn - 1)) * DK + i;
            nk[it] = k[e];
            nd[it] = d[e];
            if constexpr (GATE) {
                nq[it] = q[e];
                na[it] = alpha[e];
            }
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int idx = tid + it * kThreads, r = idx / BV, j = idx % BV;
            nv[it] = v[(r0 + (r < nn ? r : nn - 1)) * dv + j0 + j];
        }
        if (tid < nn) {
            nb = beta[r0 + tid];
            if (!GATE && alpha) nal = alpha[r0 + tid];
        }
    };
    if (T > 0) issue(0);

    for (int64_t c0 = 0; c0 < T; c0 += CH) {
        const int n = static_cast<int>(T - c0 < CH ? T - c0 : CH);
        const int64_t row0 = bh * T + c0;
        block_sync();  // the previous chunk is done with every buffer
        if (ckpt) {  // the state at this chunk's start, for the backward
            const int64_t cc = bh * ((T + CH - 1) / CH) + c0 / CH;
#pragma unroll
            for (int it = 0; it < (DK * BV + kThreads - 1) / kThreads; ++it) {
                const int idx = tid + it * kThreads, i = idx / BV, j = idx % BV;
                if (idx < DK * BV) ckpt[(cc * DK + i) * dv + j0 + j] = sM[i * PV + j];
            }
        }

        // a1: keys, scaled keys, values, gates (from the registers loaded a step ago)
#pragma unroll
        for (int it = 0; it < LIT; ++it) {
            const int idx = tid + it * kThreads, r = idx / DK, i = idx % DK;
            const bool in = r < n;
            const float kv = to_f32(nk[it]);
            sX[r * PX + i] = in ? kv : 0.f;
            sKt[r * PX + i] = in ? to_f32(nd[it]) * kv : 0.f;
            if constexpr (GATE) {
                sQ[r * PX + i] = in ? to_f32(nq[it]) : 0.f;
                sLg[r * PX + i] = in ? log(fmax(static_cast<double>(na[it]), 1e-300)) : 0.0;
            }
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int idx = tid + it * kThreads, r = idx / BV, j = idx % BV;
            sR[r * PV + j] = r < n ? to_f32(nv[it]) : 0.f;
        }
        if (tid < CH) {
            sb[tid] = tid < n ? nb : 0.f;
            sg[tid] = (tid < n && alpha && !GATE) ? logf(nal) : 0.f;
        }
        if constexpr (GATE) {
            if (gscores) {  // AS into sA (scaled by beta below), P into sP
#pragma unroll
                for (int it = 0; it < SIT; ++it) {
                    const int idx = tid + it * kThreads, r = idx / CH, s_ = idx % CH;
                    if (idx < CH * CH) {
                        sA[r * PC + s_] = nsa[it];
                        sP[r * PC + s_] = nsp[it];
                    }
                }
            }
        }
        // without GATE, this chunk's q (staged over K in a4), issued before the next chunk's
        // loads so that the wait for it there covers these alone
        TQ cq[GATE ? 1 : LIT];
        if constexpr (!GATE) {
#pragma unroll
            for (int it = 0; it < LIT; ++it) {
                const int idx = tid + it * kThreads, r = idx / DK, i = idx % DK;
                cq[it] = q[(row0 + (r < n ? r : n - 1)) * DK + i];
            }
            asm volatile("" ::: "memory");  // keeps the next chunk's loads after these
        }
        // (on the last chunk it loads that chunk again, unused: with the issue unconditional, the
        // waits for q above count these loads as issued after it on every path)
        issue(c0 + CH < T ? c0 + CH : c0);
        if constexpr (GATE) {
            block_sync();
            if (tid < DK) {  // running sums down each feature column (read whole first)
                double x[CH];
#pragma unroll
                for (int r = 0; r < CH; ++r) x[r] = sLg[r * PX + tid];
                double acc = 0.0;
#pragma unroll
                for (int r = 0; r < CH; ++r) {
                    acc += x[r];
                    sLg[r * PX + tid] = acc;
                }
            }
        }
        block_sync();
        if (tid < 64) {  // running sum of ln(alpha) by a scan over wave 0's lanes
            const float acc = wave_prefix(tid < CH ? sg[tid] : 0.f);  // on DPP
            const float last = lane_value(acc, CH - 1);
            if (tid < CH) {
                sg[tid] = acc;
                sgam[tid] = __expf(acc);
                sdec[tid] = __expf(last - acc);
            }
        }
        block_sync();

        if constexpr (GATE) {
            // a2, a5 in one pass, the decay of each (row, column, feature) formed once and used
            // for both: thread (r, s0) owns columns s0, s0 + 1 of row r
            static_assert(CH * CH / 2 <= kThreads, "gate scores layout");
            if (gscores) {  // formed already (the backward's score tiles): A = diag(beta) AS
                for (int idx = tid; idx < CH * CH; idx += kThreads) {
                    const int r = idx / CH, s_ = idx % CH;
                    sA[r * PC + s_] *= sb[r];
                }
            } else if (tid < CH * CH / 2) {
                const int r = tid / (CH / 2), s0 = (tid % (CH / 2)) * 2;
                float ak0 = 0.f, ak1 = 0.f, aq0 = 0.f, aq1 = 0.f;
                if (s0 <= r) {
                    const bool two = s0 + 1 <= r;
                    for (int i = 0; i < DK; ++i) {
                        const double lr = sLg[r * PX + i];
                        const float e0 = __expf(static_cast<float>(lr - sLg[s0 * PX + i])) *
                                         sKt[s0 * PX + i];
                        const float e1 =
                            two ? __expf(static_cast<float>(lr - sLg[(s0 + 1) * PX + i])) *
                                      sKt[(s0 + 1) * PX + i]
                                : 0.f;
                        const float kx = sX[r * PX + i], qx = sQ[r * PX + i];
                        ak0 += kx * e0;
                        ak1 += kx * e1;
                        aq0 += qx * e0;
                        aq1 += qx * e1;
                    }
                }
                sA[r * PC + s0] = s0 < r ? sb[r] * ak0 : 0.f;
                sA[r * PC + s0 + 1] = s0 + 1 < r ? sb[r] * ak1 : 0.f;
                sP[r * PC + s0] = s0 <= r ? aq0 : 0.f;
                sP[r * PC + s0 + 1] = s0 + 1 <= r ? aq1 : 0.f;
            }
            block_sync();
            // in place, once per element: K o G, Q o G, K~ o e^{Lg_C - Lg}
#pragma unroll
            for (int it = 0; it < CH * DK / kThreads; ++it) {
                const int idx = tid + it * kThreads, r = idx / DK, i = idx % DK;
                const double lg = sLg[r * PX + i];
                const float g = __expf(static_cast<float>(lg));
                sX[r * PX + i] *= g;
                sQ[r * PX + i] *= g;
                sKt[r * PX + i] *= __expf(static_cast<float>(sLg[(CH - 1) * PX + i] - lg));
            }
            block_sync();
            // a3: R = diag(beta) (V - (K o G) M)
            if (rows_ok) {
                float km[TR][2];
                zero_tile(km);
                tile_mm<TR, 2, DK>(km, ir, 2 * tx, [&](int r, int i) { return sX[r * PX + i]; },
                                   [&](int i, int j) { return sM[i * PV + j]; });
#pragma unroll
                for (int m = 0; m < TR; ++m)
#pragma unroll
                    for (int nn = 0; nn < 2; ++nn) {
                        const int r = ir + m, j = 2 * tx + nn;
                        sR[r * PV + j] = sb[r] * (sR[r * PV + j] - km[m][nn]);
                    }
            }
            block_sync();
            // a4: U = (I + A)^{-1} R in place
            solve_unit_lower<CH, BV, PV, PC>(sR, sA, tid);
            block_sync();
            // (Q o G) M for the inter-chunk read-out
            if (rows_ok) {
                float qm[TR][2];
                zero_tile(qm);
                tile_mm<TR, 2, DK>(qm, ir, 2 * tx, [&](int r, int i) { return sQ[r * PX + i]; },
                                   [&](int i, int j) { return sM[i * PV + j]; });
#pragma unroll
                for (int m = 0; m < TR; ++m)
#pragma unroll
                    for (int nn = 0; nn < 2; ++nn) sQM[(ir + m) * PV + 2 * tx + nn] = qm[m][nn];
            }
            block_sync();
        } else {
            // a2: strictly lower Gram matrix of (K, K~), decayed (tiles above the diagonal
            // stay zero); a3: R = diag(beta) (V - diag(e^g) K M)
            if (rows_ok) {
                const int is = tx * TS;
                float ak[TR][TS];
                zero_tile(ak);
                if (is <= ir + TR - 1)
                    tile_mm<TR, TS, DK>(ak, ir, is, [&](int r, int i) { return sX[r * PX + i]; },
                                        [&](int i, int s_) { return sKt[s_ * PX + i]; });
#pragma unroll
                for (int m = 0; m < TR; ++m)
#pragma unroll
                    for (int nn = 0; nn < TS; ++nn) {
                        const int r = ir + m, s_ = is + nn;
                        sA[r * PC + s_] = s_ < r ? sb[r] * __expf(sg[r] - sg[s_]) * ak[m][nn] : 0.f;
                    }
                float km[TR][2];
                zero_tile(km);
                tile_mm<TR, 2, DK>(km, ir, 2 * tx, [&](int r, int i) { return sX[r * PX + i]; },
                                   [&](int i, int j) { return sM[i * PV + j]; });
#pragma unroll
                for (int m = 0; m < TR; ++m)
#pragma unroll
                    for (int nn = 0; nn < 2; ++nn) {
                        const int r = ir + m, j = 2 * tx + nn;
                        sR[r * PV + j] = sb[r] * (sR[r * PV + j] - sgam[r] * km[m][nn]);
                    }
            }
            block_sync();

            // a4: U = (I + A)^{-1} R in place; then stage Q over K (K is no longer read)
            solve_unit_lower<CH, BV, PV, PC>(sR, sA, tid);
#pragma unroll
            for (int it = 0; it < LIT; ++it) {
                const int idx = tid + it * kThreads, r = idx / DK, i = idx % DK;
                sX[r * PX + i] = r < n ? to_f32(cq[it]) : 0.f;
            }
            block_sync();

            // a5: P = lower-inclusive (Q K~^T) with decay;  Q M for the inter-chunk read-out
            if (rows_ok) {
                const int is = tx * TS;
                float aq[TR][TS];
                zero_tile(aq);
                if (is <= ir + TR - 1)
                    tile_mm<TR, TS, DK>(aq, ir, is, [&](int r, int i) { return sX[r * PX + i]; },
                                        [&](int i, int s_) { return sKt[s_ * PX + i]; });
#pragma unroll
                for (int m = 0; m < TR; ++m)
#pragma unroll
                    for (int nn = 0; nn < TS; ++nn) {
                        const int r = ir + m, s_ = is + nn;
                        sA[r * PC + s_] = s_ <= r ? __expf(sg[r] - sg[s_]) * aq[m][nn] : 0.f;
                    }
                float qm[TR][2];
                zero_tile(qm);
                tile_mm<TR, 2, DK>(qm, ir, 2 * tx, [&](int r, int i) { return sX[r * PX + i]; },
                                   [&](int i, int j) { return sM[i * PV + j]; });
#pragma unroll
                for (int m = 0; m < TR; ++m)
#pragma unroll
                    for (int nn = 0; nn < 2; ++nn) sQM[(ir + m) * PV + 2 * tx + nn] = qm[m][nn];
            }
            block_sync();
        }
        // a6: outputs of this chunk (P is zero above the diagonal) and the state carried to
        // the next one
        if (o && rows_ok) {
            const float *Pm = GATE ? sP : sA;  // the scores
            float pu[TR][2];
            zero_tile(pu);
            tile_mm<TR, 2, CH>(pu, ir, 2 * tx, [&](int r, int s_) { return Pm[r * PC + s_]; },
                               [&](int s_, int j) { return sR[s_ * PV + j]; });
#pragma unroll
            for (int m = 0; m < TR; ++m) {
                const int r = ir + m;
                if (r < n) {
#pragma unroll
                    for (int nn = 0; nn < 2; ++nn) {
                        const int j = 2 * tx + nn;
                        o[(row0 + r) * dv + j0 + j] =
                            from_f32<TQ>(sgam[r] * sQM[r * PV + j] + pu[m][nn]);
                    }
                }
            }
        }
        {
            const int id = ty * TD_;
            float mu[TD_][2];
            zero_tile(mu);
            if constexpr (GATE)  // sKt holds K~ o e^{Lg_C - Lg} here
                tile_mm<TD_, 2, CH>(mu, id, 2 * tx, [&](int i, int s_) { return sKt[s_ * PX + i]; },
                                    [&](int s_, int j) { return sR[s_ * PV + j]; });
            else
                tile_mm<TD_, 2, CH>(mu, id, 2 * tx,
                                    [&](int i, int s_) { return sdec[s_] * sKt[s_ * PX + i]; },
                                    [&](int s_, int j) { return sR[s_ * PV + j]; });
            const float gam_last = sgam[CH - 1];
#pragma unroll
            for (int m = 0; m < TD_; ++m)
#pragma unroll
                for (int nn = 0; nn < 2; ++nn) {
                    const int i = id + m, j = 2 * tx + nn;
                    const float keep = GATE ? decay(CH - 1, i) : gam_last;
                    sM[i * PV + j] = keep * sM[i * PV + j] + mu[m][nn];
                }
        }
    }
    block_sync();
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
    if (a.alpha_ch) {  // the per-feature log sums need LDS: at most 32 rows per chunk
        constexpr int CG = CH < 32 ? CH : 32;
        if (a.gate_scores && CG != 32) return hipErrorInvalidValue;  // tiles are 32 x 32
        hipLaunchKernelGGL((chunk_f32math_kernel<DK, BV, CG, TQ, TD, true>), grid, dim3(kThreads),
                           0, stream, static_cast<const TQ *>(a.q), static_cast<const TQ *>(a.k),
                           static_cast<const TQ *>(a.v), static_cast<const TD *>(a.d), a.beta,
                           a.alpha_ch, a.S0, static_cast<TQ *>(a.o), a.S_T, a.T, a.dv,
                           static_cast<float *>(a.ckpt), a.gate_scores);
    } else {
        hipLaunchKernelGGL((chunk_f32math_kernel<DK, BV, CH, TQ, TD, false>), grid,
                           dim3(kThreads), 0, stream, static_cast<const TQ *>(a.q),
                           static_cast<const TQ *>(a.k), static_cast<const TQ *>(a.v),
                           static_cast<const TD *>(a.d), a.beta, a.alpha, a.S0,
                           static_cast<TQ *>(a.o), a.S_T, a.T, a.dv, static_cast<float *>(a.ckpt),
                           nullptr);
    }
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
