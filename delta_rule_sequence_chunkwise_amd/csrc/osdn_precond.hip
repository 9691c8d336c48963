// Phase-1 preconditioner scan of OSDN, gfx950 (OSDN technical summary, section 2.2: online
// gradient descent on the hypergradient surrogate h_t, whose gradient depends on the key and
// the write gate only; section 2.3: the APF retention gate on the preconditioner state).
//
// For every (b,h) sequence, token by token, with x_t = k_t^2 and n_t = ||k_t||^2:
//
//   token t writes with d_t;   e_t = 1 - b_t <d_t, x_t>;   c_t = eta b_t / n_t  (0 if n_t = 0)
//   d_{t+1} = r_t d_t + c_t e_t x_t          (= r_t d_t - eta grad_d h_t(d_t))
//
// Two kernels compute it.
//
// * precond_serial_kernel: one wave per sequence walks the tokens; each lane holds dk/64
//   features of d, and each token costs two wave reductions (n_t and <d_t, x_t>).  Any key
//   type; it also serves the decode step (one token, state in place).
//
// * precond_chunk_kernel (bf16 keys, chunks of C = 64 tokens): the step is affine in d, so
//   over one chunk with start state d0, rho_j = prod_{i<j} r_i and R[j,i] = rho_j / rho_{i+1},
//     d_j = rho_j d0 + sum_{i<j} R[j,i] c_i e_i x_i ,
//   and substituting d_j into e_j gives a unit lower-triangular system for the chunk's e:
//     (I + L) e = 1 - b . rho . (X d0),      L[j,i] = b_j R[j,i] c_i <x_j, x_i>  (i < j),
//   after which the chunk's outputs are  D = rho d0^T + W X,  W[j,i] = R[j,i] c_i e_i (i < j),
//   and the next chunk starts from  rho_C d0 + X^T (R[C,.] . c . e).
//   The Gram matrix X X^T and the output product W X are bf16 matrix-core products (x = k^2 is
//   exact in fp32 for a bf16 key and rounded to bf16 only as an operand); everything the
//   carried state depends on besides L -- X d0, the solve and the carry -- runs in fp32 on
//   exact x.  R is formed from the running sum lr of ln r (clamped at -80 per token), as
//   e^{lr_j - lr_{i+1}}, which is at most 1 for a retention gate r <= 1.
//
//   One workgroup of eight waves owns one sequence and walks its chunks; step s handles the
//   chain of chunk s, the preparation of chunk s+1 and the output of chunk s-1, in three
//   phases separated by barriers:
//     A  all waves: partial sums of X d0 for chunk s (each wave one slice of the features),
//        and x = k^2 for chunk s+1: bf16 copy for the matrix cores, fp32 row norms -> c.
//     B  wave 0: the forward substitution for chunk s (row j of L in lane j's registers,
//        63 broadcast-and-update steps);  waves 1-4: output of chunk s-1 as D^T = X^T W^T on
//        16x16x32 products (W built in registers), stored as 16-byte rows of d;  waves 5-6:
//        keys of chunk s+3 into LDS (global_load_lds);  wave 7: the ln r scan of chunk s+2
//        and the gate loads of chunk s+3.
//     C  all waves: the carry d0 <- rho_C d0 + X^T (R[C,.] c e) for chunk s (each wave a slice
//        of the features), and the Gram tiles of chunk s+1 -> L.
#include "osdn_internal.h"
#include "osdn_mfma.h"

namespace osdn {
namespace {

// ---- serial scan ----------------------------------------------------------------------------

// sum over all 64 lanes, every lane receives it: xor 1 and 2 within quads, the two mirrors
// within 16-lane rows, then the two row swaps (v_permlane32_swap, v_permlane16_swap)
__device__ __forceinline__ float wave_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));
    return sum_rows(x);
}

template <int DK, typename TK, typename TD>
__global__ void __launch_bounds__(64)
precond_serial_kernel(const TK *__restrict__ k, const float *__restrict__ beta,
                      const float *__restrict__ r, const float *d1, float eta,
                      TD *__restrict__ d_out, float *d_next, int64_t T) {
    constexpr int FPL = DK / 64;  // features per lane
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    const int f0 = lane * FPL;
    float d[FPL];
#pragma unroll
    for (int i = 0; i < FPL; ++i) d[i] = d1 ? d1[bh * DK + f0 + i] : 1.f;
    const TK *kr = k + bh * T * DK + f0;
    const float *br = beta + bh * T;
    const float *rr = r ? r + bh * T : nullptr;
    TD *orow = d_out ? d_out + bh * T * DK + f0 : nullptr;

    float kn[FPL], bn = 0.f, rn = 1.f;
    if (T > 0) {
#pragma unroll
        for (int i = 0; i < FPL; ++i) kn[i] = to_f32(kr[i]);
        bn = br[0];
        rn = rr ? rr[0] : 1.f;
    }
    for (int64_t t = 0; t < T; ++t) {
        float x[FPL];
        const float bc = bn, rc = rn;
#pragma unroll
        for (int i = 0; i < FPL; ++i) x[i] = kn[i] * kn[i];
        if (t + 1 < T) {  // next token's loads are in flight while this one's reductions run
#pragma unroll
            for (int i = 0; i < FPL; ++i) kn[i] = to_f32(kr[(t + 1) * DK + i]);
            bn = br[t + 1];
            rn = rr ? rr[t + 1] : 1.f;
        }
        float sn = 0.f, sd = 0.f;
#pragma unroll
        for (int i = 0; i < FPL; ++i) {
            sn += x[i];
            sd += d[i] * x[i];
        }
        if (orow) {
#pragma unroll
            for (int i = 0; i < FPL; ++i) orow[t * DK + i] = from_f32<TD>(d[i]);
        }
        sn = wave_sum(sn);
        sd = wave_sum(sd);
        const float e = 1.f - bc * sd;
        const float coef = sn > 0.f ? eta * bc * e / sn : 0.f;
#pragma unroll
        for (int i = 0; i < FPL; ++i) d[i] = rc * d[i] + coef * x[i];
    }
    if (d_next) {
#pragma unroll
        for (int i = 0; i < FPL; ++i) d_next[bh * DK + f0 + i] = d[i];
    }
}

// ---- chunked scan -----------------------------------------------------------------------------

constexpr int CH = 64;       // tokens per chunk
constexpr int NW = 8;        // waves per workgroup
constexpr int NT = NW * 64;  // threads per workgroup
constexpr float kMinLogR = -80.f;

template <int DK>
struct alignas(16) PrecondLds {
    static constexpr int KU = DK / 8;   // 16-byte units per key row
    static constexpr int LP = CH + 4;   // fp32 row pitch of L (rows start 4 banks apart)
    // 16-byte unit u of key row j sits at unit u ^ sw(j): reads that take one unit from each
    // of 16 consecutive rows, and rows of 16 consecutive units, are bank-conflict free
    __device__ static constexpr int sw(int j) { return DK == 128 ? (j & 15) : ((j >> 1) & 7); }
    __device__ static constexpr int at(int j, int u) { return (j * KU + (u ^ sw(j))) * 8; }
    alignas(16) uint16_t kb[4][CH * DK];  // [chunk mod 4] keys (bf16), swizzled rows
    alignas(16) uint16_t xb[3][CH * DK];  // [chunk mod 3] bf16(k^2), same layout
    alignas(16) float L[2][CH * LP];      // [chunk parity] L, row-major (upper part zero)
    alignas(16) float beta[4][CH];        // [chunk mod 4] gate (0 past the end)
    alignas(16) float cc[4][CH];          // eta b / ||k||^2
    alignas(16) float lr[4][CH + 4];      // lr[0] = 0, lr[j+1] = sum_{i<=j} max(ln r_i, -80)
    alignas(16) float d0[2][DK];          // [chunk parity] start state of the chunk
    alignas(16) float ee[2][CH];          // [chunk parity] e of the chunk
    alignas(16) float wc[CH];             // R[C,j] c_j e_j of the chunk in its chain
    alignas(16) float up[NW][CH];         // per-wave partial sums of X d0
};

// inclusive prefix sum over the 64 lanes (shifts by 1, 2, 4, 8 inside each 16-lane row, then
// the last lane of rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3)
__device__ __forceinline__ float wave_prefix(float x) {
    x = dpp_add<0x111, 0xf>(x);
    x = dpp_add<0x112, 0xf>(x);
    x = dpp_add<0x114, 0xf>(x);
    x = dpp_add<0x118, 0xf>(x);
    x = dpp_add<0x142, 0xa>(x);
    x = dpp_add<0x143, 0xc>(x);
    return x;
}

template <int DK, typename TD>
__global__ void __launch_bounds__(NT)
precond_chunk_kernel(const uint16_t *__restrict__ k, const float *__restrict__ beta,
                     const float *__restrict__ r, const float *d1, float eta,
                     TD *__restrict__ d_out, float *d_next, int64_t T) {
    using L = PrecondLds<DK>;
    __shared__ L sm;
    const int64_t bh = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nc = static_cast<int>((T + CH - 1) / CH);
    const uint16_t *kq = k + bh * T * DK;
    const float *bq = beta + bh * T;
    const float *rq = r ? r + bh * T : nullptr;
    TD *oq = d_out + bh * T * DK;

    // keys of chunk cd into kb[cd & 3] (one wave: rows [R0, R0 + 32)); rows past the end
    // re-read the last row (their gate is zero)
    auto dma = [&](int cd, int R0) __attribute__((always_inline)) {
        constexpr int NLD = 32 * L::KU / 64;
        uint16_t *dst = sm.kb[cd & 3];
        const int64_t row0 = int64_t(cd) * CH;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int base = R0 * L::KU + i * 64;
            const int pu = base + lane, j = pu / L::KU, u = (pu % L::KU) ^ L::sw(j);
            const int64_t row = row0 + j < T ? row0 + j : T - 1;
            load_to_lds16(kq + row * DK + 8 * u, dst + 8 * base);
        }
    };
    // gate scan of chunk cs from this lane's b and r (one wave, row = lane)
    auto scan = [&](int cs, float bv, float rv) __attribute__((always_inline)) {
        const bool ok = int64_t(cs) * CH + lane < T;
        const float x = (ok && rq) ? fmaxf(__logf(rv), kMinLogR) : 0.f;
        const float incl = wave_prefix(x);
        sm.lr[cs & 3][lane + 1] = incl;
        if (lane == 0) sm.lr[cs & 3][0] = 0.f;
        sm.beta[cs & 3][lane] = ok ? bv : 0.f;
    };
    auto gates = [&](int cl, float &bv, float &rv) __attribute__((always_inline)) {
        const int64_t t = int64_t(cl) * CH + lane;
        bv = t < T ? bq[t] : 0.f;
        rv = (t < T && rq) ? rq[t] : 1.f;
    };

    // ---- prologue: zero L (its upper part is never written), d0 of chunk 0, keys of
    // chunks 0 and 1, gates of chunk 0 scanned and of chunk 1 in registers
    for (int i = threadIdx.x; i < 2 * CH * L::LP; i += NT) (&sm.L[0][0])[i] = 0.f;
    if (threadIdx.x < DK) sm.d0[0][threadIdx.x] = d1 ? d1[bh * DK + threadIdx.x] : 1.f;
    float bnext = 0.f, rnext = 1.f;
    if (nc > 0) {
        if (wave == 5 || wave == 6) {
            dma(0, 32 * (wave - 5));
            if (nc > 1) dma(1, 32 * (wave - 5));
            wait_global();
        } else if (wave == 7) {
            float b0, r0;
            gates(0, b0, r0);
            scan(0, b0, r0);
            if (nc > 1) gates(1, bnext, rnext);
        }
    }
    block_sync();

    const int q = lane >> 4, n = lane & 15;
    for (int s = -1; s <= nc; ++s) {
        const bool chain = s >= 0 && s < nc, prep = s + 1 < nc;
        // ---- phase A ----------------------------------------------------------------------
        if (chain) {  // partial X d0 over this wave's features; lane = row
            constexpr int UPW = L::KU / NW;
            const uint16_t *kt = sm.kb[s & 3];
            const float *d0 = sm.d0[s & 1];
            float acc = 0.f;
#pragma unroll
            for (int qq = 0; qq < UPW; ++qq) {
                const int u = wave * UPW + qq;
                const uint4 w = *reinterpret_cast<const uint4 *>(kt + L::at(lane, u));
                const v4f da = ld4(d0 + 8 * u), db = ld4(d0 + 8 * u + 4);
                const float k0 = bf_lo(w.x), k1 = bf_hi(w.x), k2 = bf_lo(w.y), k3 = bf_hi(w.y);
                const float k4 = bf_lo(w.z), k5 = bf_hi(w.z), k6 = bf_lo(w.w), k7 = bf_hi(w.w);
                acc += k0 * k0 * da[0] + k1 * k1 * da[1] + k2 * k2 * da[2] + k3 * k3 * da[3];
                acc += k4 * k4 * db[0] + k5 * k5 * db[1] + k6 * k6 * db[2] + k7 * k7 * db[3];
            }
            sm.up[wave][lane] = acc;
        }
        if (prep) {  // x = k^2 of chunk s+1: bf16 copy and fp32 row norms
            constexpr int LPR = L::KU;             // lanes per row
            constexpr int RPW = 64 / LPR;          // rows per wave and pass
            constexpr int NPASS = CH / (RPW * NW);
            const int cn = s + 1;
            const uint16_t *kt = sm.kb[cn & 3];
            uint16_t *xt = sm.xb[cn % 3];
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const int row = (p * NW + wave) * RPW + lane / LPR;
                const int e = (row * L::KU + lane % LPR) * 8;
                const uint4 w = *reinterpret_cast<const uint4 *>(kt + e);
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
                uint32_t o[4];
                float sn = 0.f;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float a = bf_lo(ws[h]), b = bf_hi(ws[h]);
                    const float xa = a * a, xb = b * b;
                    sn += xa + xb;
                    o[h] = pack2(xa, xb);
                }
                *reinterpret_cast<uint4 *>(xt + e) = make_uint4(o[0], o[1], o[2], o[3]);
                sn = dpp_add<0xb1, 0xf>(sn);
                sn = dpp_add<0x4e, 0xf>(sn);
                sn = dpp_add<0x141, 0xf>(sn);
                if (LPR == 16) sn = dpp_add<0x140, 0xf>(sn);
                if (lane % LPR == 0) {
                    const float bv = sm.beta[cn & 3][row];
                    sm.cc[cn & 3][row] = sn > 0.f ? eta * bv / sn : 0.f;
                }
            }
        }
        block_sync();

        // ---- phase B ----------------------------------------------------------------------
        if (wave == 0) {
            if (chain) {  // forward substitution (I + L) e = 1 - b rho (X d0); lane = row
                float Lrow[CH];
                const float *Lr = sm.L[s & 1] + lane * L::LP;
#pragma unroll
                for (int m = 0; m < CH / 4; ++m) {
                    const v4f t4 = ld4(Lr + 4 * m);
                    Lrow[4 * m] = t4[0];
                    Lrow[4 * m + 1] = t4[1];
                    Lrow[4 * m + 2] = t4[2];
                    Lrow[4 * m + 3] = t4[3];
                }
                float u = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) u += sm.up[w][lane];
                const float lrj = sm.lr[s & 3][lane];
                float e = 1.f - sm.beta[s & 3][lane] * __expf(lrj) * u;
#pragma unroll
                for (int i = 0; i < CH - 1; ++i) e = fmaf(-Lrow[i], lane_value(e, i), e);
                sm.ee[s & 1][lane] = e;
                sm.wc[lane] = __expf(sm.lr[s & 3][CH] - sm.lr[s & 3][lane + 1]) *
                              sm.cc[s & 3][lane] * e;
            }
        } else if (wave <= 4) {
            if (s >= 1) {  // output of chunk s-1: D^T = rho-scaled d0 + X^T W^T
                const int co = s - 1, sl = co & 3;
                const uint16_t *xt = sm.xb[co % 3];
                const float *ee = sm.ee[co & 1];
                const float *lr = sm.lr[sl], *cc = sm.cc[sl];
                constexpr int FPW = DK / 16 / 4;  // 16-feature tiles per output wave
                v8s wb[6];
#pragma unroll
                for (int J = 0, idx = 0; J < 4; ++J) {
#pragma unroll
                    for (int st = 0; st <= (J >> 1); ++st, ++idx) {
                        const int j = 16 * J + n;
                        const float lrj = lr[j];
                        float wv[8];
#pragma unroll
                        for (int m = 0; m < 8; ++m) {
                            const int i = 32 * st + 8 * q + m;
                            wv[m] = i < j ? __expf(lrj - lr[i + 1]) * cc[i] * ee[i] : 0.f;
                        }
                        wb[idx] = __builtin_bit_cast(
                            v8s, make_uint4(pack2(wv[0], wv[1]), pack2(wv[2], wv[3]),
                                            pack2(wv[4], wv[5]), pack2(wv[6], wv[7])));
                    }
                }
                const float *d0 = sm.d0[co & 1];
#pragma unroll
                for (int ft = 0; ft < FPW; ++ft) {
                    const int F = (wave - 1) * FPW + ft;
                    v8s xa[2];
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const int col = 16 * F + 4 * (n & 3);
                        const int r0 = 32 * st + 8 * q + (n >> 2);
                        const v4s lo = ld_tr(xt + L::at(r0, col >> 3) + (col & 7));
                        const v4s hi = ld_tr(xt + L::at(r0 + 4, col >> 3) + (col & 7));
                        xa[st] = cat8(lo, hi);
                    }
                    const v4f dv = ld4(d0 + 16 * F + 4 * q);
#pragma unroll
                    for (int J = 0, idx = 0; J < 4; ++J) {
                        const float rho = __expf(lr[16 * J + n]);
                        v4f acc = v4f{rho * dv[0], rho * dv[1], rho * dv[2], rho * dv[3]};
#pragma unroll
                        for (int st = 0; st <= (J >> 1); ++st, ++idx) acc = mfma32(xa[st], wb[idx], acc);
                        const int64_t tok = int64_t(co) * CH + 16 * J + n;
                        if (tok < T) store4(oq + tok * DK + 16 * F + 4 * q, acc);
                    }
                }
            }
        } else if (wave <= 6) {
            if (s + 3 < nc) dma(s + 3, 32 * (wave - 5));
        } else {
            if (s + 2 < nc) scan(s + 2, bnext, rnext);
            if (s + 3 < nc) gates(s + 3, bnext, rnext);
        }
        block_sync();

        // ---- phase C ----------------------------------------------------------------------
        if (chain) {  // carry: d0 <- rho_C d0 + X^T (R[C,.] c e) over this wave's features
            constexpr int FW = DK / NW;  // features per wave
            constexpr int G = 64 / FW;   // row groups
            const int f = wave * FW + lane % FW, g = lane / FW;
            const uint16_t *kt = sm.kb[s & 3];
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < CH / G; ++m) {
                const int j = g + G * m;
                const float kv = __uint_as_float(uint32_t(kt[L::at(j, f >> 3) + (f & 7)]) << 16);
                acc += sm.wc[j] * (kv * kv);
            }
            if (G == 8) acc = dpp_add<0x128, 0xf>(acc);  // row_ror:8
            acc = sum_rows(acc);                          // + lanes 16 and 32 away
            if (g == 0)
                sm.d0[(s + 1) & 1][f] = __expf(sm.lr[s & 3][CH]) * sm.d0[s & 1][f] + acc;
        }
        if (prep) {  // Gram tiles of chunk s+1 -> L
            const int cg = s + 1, sl = cg & 3;
            const uint16_t *xt = sm.xb[cg % 3];
            for (int tIdx = wave; tIdx < 10; tIdx += NW) {
                const int J = tIdx < 1 ? 0 : tIdx < 3 ? 1 : tIdx < 6 ? 2 : 3;
                const int I = tIdx - J * (J + 1) / 2;
                v4f acc = zero4();
#pragma unroll
                for (int st = 0; st < DK / 32; ++st) {
                    const int u = 4 * st + q;
                    acc = mfma32(ld8(xt + L::at(16 * J + n, u)), ld8(xt + L::at(16 * I + n, u)), acc);
                }
                const int i = 16 * I + n;
                const float ci = sm.cc[sl][i], lri = sm.lr[sl][i + 1];
                float *Lt = sm.L[cg & 1];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int j = 16 * J + 4 * q + m;
                    Lt[j * L::LP + i] =
                        i < j ? sm.beta[sl][j] * __expf(sm.lr[sl][j] - lri) * ci * acc[m] : 0.f;
                }
            }
        }
        if (wave == 5 || wave == 6) {  // keys of chunk s+2 have landed
            if (s + 3 < nc) wait_global_n<32 * L::KU / 64>();
            else wait_global();
        }
        block_sync();
    }
    if (d_next && threadIdx.x < DK) d_next[bh * DK + threadIdx.x] = sm.d0[nc & 1][threadIdx.x];
}

template <int DK>
hipError_t launch_dk(const PrecondArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.BH));
    if (a.chunk == 1) {
#define OSDN_SERIAL(TK, TD)                                                                   \
    hipLaunchKernelGGL((precond_serial_kernel<DK, TK, TD>), grid, dim3(64), 0, stream,        \
                       static_cast<const TK *>(a.k), a.beta, a.r, a.d1, a.eta,               \
                       static_cast<TD *>(a.d), a.d_next, a.T)
        if (a.k_dtype == OSDN_F32) {
            if (a.d_dtype == OSDN_F32) OSDN_SERIAL(float, float);
            else OSDN_SERIAL(float, bf16_t);
        } else {
            if (a.d_dtype == OSDN_F32) OSDN_SERIAL(bf16_t, float);
            else OSDN_SERIAL(bf16_t, bf16_t);
        }
#undef OSDN_SERIAL
    } else {
        if (a.d_dtype == OSDN_F32)
            hipLaunchKernelGGL((precond_chunk_kernel<DK, float>), grid, dim3(NT), 0, stream,
                               static_cast<const uint16_t *>(a.k), a.beta, a.r, a.d1, a.eta,
                               static_cast<float *>(a.d), a.d_next, a.T);
        else
            hipLaunchKernelGGL((precond_chunk_kernel<DK, bf16_t>), grid, dim3(NT), 0, stream,
                               static_cast<const uint16_t *>(a.k), a.beta, a.r, a.d1, a.eta,
                               static_cast<bf16_t *>(a.d), a.d_next, a.T);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_precond(const PrecondArgs &a, hipStream_t stream) {
    return a.dk == 64 ? launch_dk<64>(a, stream) : launch_dk<128>(a, stream);
}

}  // namespace osdn
