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
//   Every product runs on 16x16x32 bf16 matrix cores with fp32 accumulation.  x = k^2 of a
//   bf16 key is exact in fp32 and splits exactly into xh = bf16(x) plus xl = bf16(x - xh).
//   The products the carried state depends on -- X d0 and X^T w -- use both halves of x and
//   of the other operand (hi/lo bf16 pairs), so they are accurate to fp32; the Gram matrix
//   X X^T (which only enters through L) and the output product W X use xh alone, and the
//   forward substitution is fp32.  R is formed from the running sum lr of ln r (clamped at
//   -80 per token), as e^{lr_j - lr_{i+1}}, at most 1 for a retention gate r <= 1.
//
//   One workgroup of eight waves owns one sequence and walks its chunks with one barrier per
//   step; each role runs its own loop, so registers one role keeps do not add to another's:
//     wave 0      the chain of chunk s: X d0 (A = xh, xl rows; B = hi/lo of d0 in columns 0
//                 and 1), the forward substitution (row j of L in lane j's registers, 63
//                 broadcast-and-update steps), the carry d0 <- rho_C d0 + X^T w
//                 (A = hi/lo of w in rows 0 and 1; B = xh, xl by transposing LDS reads); d0
//                 and w are kept as bf16 hi/lo pairs too, ready as operands;
//     waves 1-3, 7  the output of chunk s-1 as D^T = X^T W^T (W built in registers from one
//                 exponential per fragment and per-token factors; each wave takes two token
//                 row blocks and half of the features), stored as 16-byte rows of d, and two
//                 Gram tiles of chunk s+1 each;
//     waves 5-6   keys of chunk s+2 squared from registers into xh, xl and the row norms,
//                 then the keys of chunk s+3 loaded into registers (a step of latency hidden);
//     wave 4      the gate scan of chunk s+2, the gate loads of chunk s+3 and two Gram tiles
//                 (it shares a SIMD with wave 0, so its load is kept light).
//   Keys go through registers rather than global_load_lds: an LDS read that may alias an
//   in-flight LDS DMA makes the compiler wait for every outstanding vector memory operation
//   of the wave, stores included.
#include <type_traits>

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

    TK kn[FPL];  // the next token's key as loaded (widened at its use, not at the load)
    float bn = 0.f, rn = 1.f;
    if (T > 0) {
#pragma unroll
        for (int i = 0; i < FPL; ++i) kn[i] = kr[i];
        bn = br[0];
        rn = rr ? rr[0] : 1.f;
    }
    for (int64_t t = 0; t < T; ++t) {
        float x[FPL];
        const float bc = bn, rc = rn;
#pragma unroll
        for (int i = 0; i < FPL; ++i) x[i] = to_f32(kn[i]) * to_f32(kn[i]);
        if (t + 1 < T) {  // next token's loads are in flight while this one's reductions run
#pragma unroll
            for (int i = 0; i < FPL; ++i) kn[i] = kr[(t + 1) * DK + i];
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

// f(integral_constant<I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int DK>
struct alignas(16) PrecondLds {
    static constexpr int KU = DK / 8;   // 16-byte units per row of x
    static constexpr int LP = CH + 4;   // fp32 row pitch of L (rows start 4 banks apart)
    // 16-byte unit u of row j sits at unit u ^ sw(j): reads that take one unit from each of 16
    // consecutive rows, and rows of consecutive units, are bank-conflict free
    __device__ static constexpr int sw(int j) { return DK == 128 ? (j & 15) : ((j >> 1) & 7); }
    __device__ static constexpr int at(int j, int u) { return (j * KU + (u ^ sw(j))) * 8; }
    alignas(16) uint16_t xh[4][CH * DK];  // [chunk mod 4] bf16(x), x = k^2 (fp32-exact)
    alignas(16) uint16_t xl[3][CH * DK];  // [chunk mod 3] bf16(x - xh): xh + xl = x exactly
    alignas(16) float L[2][CH * LP];      // [chunk parity] L, row-major (upper part zero)
    alignas(16) float nrm[4][CH];         // [chunk mod 4] ||k_j||^2
    alignas(16) float beta[4][CH];        // gate (0 past the end)
    alignas(16) float cc[4][CH];          // eta b / ||k||^2
    alignas(16) float lr[4][CH + 4];      // lr[0] = 0, lr[j+1] = sum_{i<=j} max(ln r_i, -80)
    alignas(16) float rho[4][CH];         // e^{lr_j}
    alignas(16) float d0[3][DK];          // [chunk mod 3] start state of the chunk
    alignas(16) float ew[2][CH];          // [chunk parity] e^{lr_{32(i/32)} - lr_{i+1}} c_i e_i
    alignas(16) uint16_t dsp[2][2][DK];   // [chunk parity][hi, lo] bf16 split of d0
    alignas(16) uint16_t wsp[2][CH];      // [hi, lo] bf16 split of w = R[C,.] c e
};

// an fp32 value -> (bf16(v), bf16(v - bf16(v))) as raw bits
__device__ __forceinline__ void split1(float v, uint16_t &hi, uint16_t &lo) {
    const uint32_t p = pack2(v, 0.f);
    hi = static_cast<uint16_t>(p);
    lo = static_cast<uint16_t>(pack2(v - bf_lo(p), 0.f));
}
// operand fragment whose lanes of column (or row) 0 hold eight hi values and of column 1 the
// matching lo values (from a [hi, lo] pair of bf16 arrays); other lanes hold zero
__device__ __forceinline__ v8s split_frag(const uint16_t *hi, const uint16_t *lo, int off, int n) {
    const v8s x = ld8((n == 1 ? lo : hi) + off);
    const v8s z = {0, 0, 0, 0, 0, 0, 0, 0};
    return n < 2 ? x : z;
}

template <int DK, typename TD>
__global__ void __launch_bounds__(NT)
precond_chunk_kernel(const uint16_t *__restrict__ k, const float *__restrict__ beta,
                     const float *__restrict__ r, const float *d1, float eta,
                     TD *__restrict__ d_out, float *d_next, int64_t T) {
    using L = PrecondLds<DK>;
    constexpr int NLD = 32 * L::KU / 64;  // 16-byte key loads per lane for half a key tile
    constexpr int KS = DK / 32;           // 32-feature slices of a row
    constexpr int NF = DK / 16;           // 16-feature tiles of a row
    __shared__ L sm;
    const int64_t bh = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane >> 4, n = lane & 15;
    const int nc = static_cast<int>((T + CH - 1) / CH);
    const uint16_t *kq = k + bh * T * DK;
    const float *bq = beta + bh * T;
    const float *rq = r ? r + bh * T : nullptr;
    TD *oq = d_out + bh * T * DK;

    // ---- key loading (waves 5 and 6, rows [R0, R0 + 32) of a chunk each): keys go to two sets
    // of eight named registers (a register array carried across the step loop would live in
    // scratch), so a chunk's loads are issued a whole step before it is squared; rows past the
    // end re-read the last row (their gate is zero)
    const int R0 = 32 * (wave - 5);
    uint4 kr0, kr1, kr2, kr3, kr4, kr5, kr6, kr7, kr8, kr9, kr10, kr11, kr12, kr13, kr14, kr15;
    auto kreg = [&](auto S, auto I) __attribute__((always_inline)) -> uint4 & {
        constexpr int R = 8 * decltype(S)::value + decltype(I)::value;
        if constexpr (R == 0) return kr0;
        else if constexpr (R == 1) return kr1;
        else if constexpr (R == 2) return kr2;
        else if constexpr (R == 3) return kr3;
        else if constexpr (R == 4) return kr4;
        else if constexpr (R == 5) return kr5;
        else if constexpr (R == 6) return kr6;
        else if constexpr (R == 7) return kr7;
        else if constexpr (R == 8) return kr8;
        else if constexpr (R == 9) return kr9;
        else if constexpr (R == 10) return kr10;
        else if constexpr (R == 11) return kr11;
        else if constexpr (R == 12) return kr12;
        else if constexpr (R == 13) return kr13;
        else if constexpr (R == 14) return kr14;
        else return kr15;
    };
    static_assert(NLD <= 8, "eight registers per key set");
    auto load_keys = [&](int cl, auto S) __attribute__((always_inline)) {
        const int64_t row0 = int64_t(cl) * CH;
        static_for<0, NLD>([&](auto I) __attribute__((always_inline)) {
            const int pu = R0 * L::KU + I * 64 + lane, j = pu / L::KU, u = pu % L::KU;
            const int64_t row = row0 + j < T ? row0 + j : T - 1;
            kreg(S, I) = *reinterpret_cast<const uint4 *>(kq + row * DK + 8 * u);
        });
    };
    // x = k^2 of the keys in registers -> xh, xl (xh + xl = x exactly for bf16 keys) and the
    // row norms (the KU units of a row sit in KU consecutive lanes)
    auto square_keys = [&](int cl, auto S) __attribute__((always_inline)) {
        uint16_t *xh = sm.xh[cl & 3], *xl = sm.xl[cl % 3];
        static_for<0, NLD>([&](auto I) __attribute__((always_inline)) {
            const int pu = R0 * L::KU + I * 64 + lane, j = pu / L::KU, u = pu % L::KU;
            const uint4 w = kreg(S, I);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
            uint32_t hi[4], lo[4];
            float sn = 0.f;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float a = bf_lo(ws[h]), b = bf_hi(ws[h]);
                const float xa = a * a, xb = b * b;
                sn += xa + xb;
                hi[h] = pack2(xa, xb);
                lo[h] = pack2(xa - bf_lo(hi[h]), xb - bf_hi(hi[h]));
            }
            *reinterpret_cast<uint4 *>(xh + L::at(j, u)) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(xl + L::at(j, u)) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            sn = dpp_add<0xb1, 0xf>(sn);
            sn = dpp_add<0x4e, 0xf>(sn);
            sn = dpp_add<0x141, 0xf>(sn);
            if (L::KU == 16) sn = dpp_add<0x140, 0xf>(sn);
            if (u == 0) sm.nrm[cl & 3][j] = sn;
        });
    };
    // gate scan of chunk cs from this lane's b and r (wave 4, row = lane)
    auto scan = [&](int cs, float bv, float rv) __attribute__((always_inline)) {
        const bool ok = int64_t(cs) * CH + lane < T;
        const float x = (ok && rq) ? fmaxf(__logf(rv), kMinLogR) : 0.f;
        const float incl = wave_prefix(x);
        sm.lr[cs & 3][lane + 1] = incl;
        sm.rho[cs & 3][lane] = __expf(incl - x);
        if (lane == 0) sm.lr[cs & 3][0] = 0.f;
        sm.beta[cs & 3][lane] = ok ? bv : 0.f;
    };
    auto gates = [&](int cl, float &bv, float &rv) __attribute__((always_inline)) {
        const int64_t t = int64_t(cl) * CH + lane;
        bv = t < T ? bq[t] : 0.f;
        rv = (t < T && rq) ? rq[t] : 1.f;
    };
    // Gram tiles t0 and t1 of chunk cg (tiles of the lower triangle in row order) -> L, and
    // c = eta b / ||k||^2 of the tile's columns (written by the diagonal tile)
    auto gram2 = [&](int cg, int t0, int t1) __attribute__((always_inline)) {
        const int sl = cg & 3;
        const uint16_t *xh = sm.xh[sl];
        int J[2], I[2];
        v4f acc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t = h == 0 ? t0 : t1;
            J[h] = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            I[h] = t - J[h] * (J[h] + 1) / 2;
            acc[h] = zero4();
        }
        // the epilogue's operands, read before the products: per column i its norm, beta and
        // running log-gate sum, per row j (four consecutive rows a lane) beta and the running sum
        float ni[2], bi[2], lri[2];
        v4f bj[2], lj[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = 16 * I[h] + n;
            ni[h] = sm.nrm[sl][i];
            bi[h] = sm.beta[sl][i];
            lri[h] = sm.lr[sl][i + 1];
            bj[h] = ld4(&sm.beta[sl][16 * J[h] + 4 * q]);
            lj[h] = ld4(&sm.lr[sl][16 * J[h] + 4 * q]);
        }
#pragma unroll
        for (int st = 0; st < KS; ++st) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int u = 4 * st + q;
                acc[h] = mfma32(ld8(xh + L::at(16 * J[h] + n, u)), ld8(xh + L::at(16 * I[h] + n, u)),
                                acc[h]);
            }
        }
        float *Lt = sm.L[cg & 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = 16 * I[h] + n;
            const float ci = ni[h] > 0.f ? eta * bi[h] / ni[h] : 0.f;
            if (J[h] == I[h] && q == 0) sm.cc[sl][i] = ci;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int j = 16 * J[h] + 4 * q + m;
                Lt[j * L::LP + i] = i < j ? bj[h][m] * __expf(lj[h][m] - lri[h]) * ci * acc[h][m] : 0.f;
            }
        }
    };

    // ---- prologue: zero L (its upper part is never written), d0 of chunk 0, x of chunk 0,
    // gates of chunk 0 scanned
    for (int i = threadIdx.x; i < 2 * CH * L::LP; i += NT) (&sm.L[0][0])[i] = 0.f;
    if (threadIdx.x < DK) {
        const float v = d1 ? d1[bh * DK + threadIdx.x] : 1.f;
        sm.d0[0][threadIdx.x] = v;
        split1(v, sm.dsp[0][0][threadIdx.x], sm.dsp[0][1][threadIdx.x]);
    }
    if (nc > 0) {
        if (wave == 5 || wave == 6) {
            load_keys(0, std::integral_constant<int, 0>{});
            square_keys(0, std::integral_constant<int, 0>{});
        } else if (wave == 4) {
            float b0, r0;
            gates(0, b0, r0);
            scan(0, b0, r0);
        }
    }
    block_sync();

    // Each role runs its own loop over steps s = -1 .. nc, one barrier per step: in step s
    // wave 0 chains chunk s, waves 1-3 and 7 write out chunk s-1, waves 1-4 and 7 build the
    // Gram tiles of chunk s+1, waves 5-6 square the keys of chunk s+2 and wave 4 scans its
    // gates.
    if (wave == 0) {
        // d0 stays in registers: lane (q, n) owns features 16 q + n and, for dk = 128,
        // 16 (q + 4) + n (the carry's column tiles q and q + 4)
        float d0a = sm.d0[0][16 * q + n], d0b = NF > 4 ? sm.d0[0][16 * (q + 4) + n] : 0.f;
        for (int s = -1; s <= nc; ++s) {
            if (s >= 0 && s < nc) {
                const int sl = s & 3;
                const uint16_t *xh = sm.xh[sl], *xl = sm.xl[s % 3];
                // u^T = d0^T X^T: A = [hi(d0) ; lo(d0) ; 0 ...] (rows 0, 1), B = xh then xl
                // (token columns 16J..), so the sum of output rows 0 and 1 is x . d0 to fp32
                // accuracy, in lane n of the first quarter for token 16J + n.  The fragments of
                // a feature slice are read together, one slice ahead of the products.
                v4f ua[4];
#pragma unroll
                for (int J = 0; J < 4; ++J) ua[J] = zero4();
                v8s fa[2][8];
                auto read_u = [&](int st, v8s *f) __attribute__((always_inline)) {
                    const int u = 4 * st + q;
#pragma unroll
                    for (int J = 0; J < 4; ++J) {
                        f[2 * J] = ld8(xh + L::at(16 * J + n, u));
                        f[2 * J + 1] = ld8(xl + L::at(16 * J + n, u));
                    }
                };
                read_u(0, fa[0]);
#pragma unroll
                for (int st = 0; st < KS; ++st) {
                    if (st + 1 < KS) read_u(st + 1, fa[(st + 1) & 1]);
                    const v8s b = split_frag(sm.dsp[s & 1][0], sm.dsp[s & 1][1], 32 * st + 8 * q, n);
                    __builtin_amdgcn_sched_barrier(0);  // the next slice's reads stay ahead
#pragma unroll
                    for (int J = 0; J < 4; ++J) {
                        ua[J] = mfma32(b, fa[st & 1][2 * J], ua[J]);
                        ua[J] = mfma32(b, fa[st & 1][2 * J + 1], ua[J]);
                    }
                }
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
                // row 0 + row 1 of tile J sits in lanes 0..15; the two row swaps bring tile J
                // to lanes 16J.., so lane j holds u_j
                uint32_t uj[4];
#pragma unroll
                for (int J = 0; J < 4; ++J) uj[J] = __float_as_uint(ua[J][0] + ua[J][1]);
                const u32x2 s01 = __builtin_amdgcn_permlane16_swap(uj[0], uj[1], false, false);
                const u32x2 s23 = __builtin_amdgcn_permlane16_swap(uj[2], uj[3], false, false);
                const u32x2 s03 = __builtin_amdgcn_permlane32_swap(s01[0], s23[0], false, false);
                const float u = __uint_as_float(s03[0]);
                // the carry's B fragments of X^T do not depend on e: the first two tiles' reads
                // are issued before the substitution, which uses no LDS
                v8s fb[3][4];
                auto read_c = [&](int F, v8s *f) __attribute__((always_inline)) {
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const int col = 16 * F + 4 * (n & 3), r0 = 32 * st + 8 * q + (n >> 2);
                        const int o0 = L::at(r0, col >> 3) + (col & 7);
                        const int o1 = L::at(r0 + 4, col >> 3) + (col & 7);
                        f[2 * st] = cat8(ld_tr(xh + o0), ld_tr(xh + o1));
                        f[2 * st + 1] = cat8(ld_tr(xl + o0), ld_tr(xl + o1));
                    }
                };
                read_c(0, fb[0]);
                read_c(1, fb[1]);
                // (I + L) e = 1 - b rho u by forward substitution; lane = row
                float e = 1.f - sm.beta[sl][lane] * sm.rho[sl][lane] * u;
#pragma unroll
                for (int i = 0; i < CH - 1; ++i) e = fmaf(-Lrow[i], lane_value(e, i), e);
                const float lr1 = sm.lr[sl][lane + 1], ce = sm.cc[sl][lane] * e;
                split1(__expf(sm.lr[sl][CH] - lr1) * ce, sm.wsp[0][lane], sm.wsp[1][lane]);
                sm.ew[s & 1][lane] = __expf(sm.lr[sl][lane & 32] - lr1) * ce;
                // carry d0 <- rho_C d0 + X^T w: A = [hi(w) ; lo(w) ; 0 ...], B = xh then xl
                v8s aw[2];
#pragma unroll
                for (int st = 0; st < 2; ++st) aw[st] = split_frag(sm.wsp[0], sm.wsp[1], 32 * st + 8 * q, n);
                v4f ca[NF];
#pragma unroll
                for (int F = 0; F < NF; ++F) {
                    if (F + 2 < NF) read_c(F + 2, fb[(F + 2) % 3]);
                    __builtin_amdgcn_sched_barrier(0);  // the reads stay two tiles ahead
                    ca[F] = zero4();
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        ca[F] = mfma32(aw[st], fb[F % 3][2 * st], ca[F]);
                        ca[F] = mfma32(aw[st], fb[F % 3][2 * st + 1], ca[F]);
                    }
                }
                // rows 0 (hi(w) . x) and 1 (lo(w) . x) of column tile F sit in lanes 0..15; the
                // row swaps bring tiles q and q + 4 to quarter q, so every lane writes two
                // features instead of lanes 0..15 writing all of them
                auto gather4 = [&](int F0) __attribute__((always_inline)) {
                    uint32_t x[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        x[i] = F0 + i < NF ? __float_as_uint(ca[F0 + i][0] + ca[F0 + i][1]) : 0u;
                    const u32x2 a = __builtin_amdgcn_permlane16_swap(x[0], x[1], false, false);
                    const u32x2 b = __builtin_amdgcn_permlane16_swap(x[2], x[3], false, false);
                    return __uint_as_float(__builtin_amdgcn_permlane32_swap(a[0], b[0], false, false)[0]);
                };
                const float rc = __expf(sm.lr[sl][CH]);
                float *dn = sm.d0[(s + 1) % 3];
                uint16_t *dh = sm.dsp[(s + 1) & 1][0], *dl = sm.dsp[(s + 1) & 1][1];
                d0a = rc * d0a + gather4(0);
                dn[16 * q + n] = d0a;
                split1(d0a, dh[16 * q + n], dl[16 * q + n]);
                if constexpr (NF > 4) {
                    d0b = rc * d0b + gather4(4);
                    dn[16 * (q + 4) + n] = d0b;
                    split1(d0b, dh[16 * (q + 4) + n], dl[16 * (q + 4) + n]);
                }
            }
            block_sync();
        }
    } else if (wave != 4 && wave != 5 && wave != 6) {
        // output waves 1, 2, 3, 7: wave ow takes the token row blocks {0, 3} or {1, 2} (the
        // same number of products) and one half of the feature tiles
        const int ow = wave == 7 ? 3 : wave - 1;
        const int Ja = (ow & 1) ? 1 : 0, Jb = 3 - Ja;  // Ja < 2 needs one token slice, Jb two
        for (int s = -1; s <= nc; ++s) {
            if (s + 1 < nc) gram2(s + 1, ow, ow + 4);
            if (s >= 1) {  // output of chunk s-1: D^T = d0 rho^T + X^T W^T, W[j,i] = R c_i e_i
                const int co = s - 1, sl = co & 3;
                const uint16_t *xt = sm.xh[sl];
                const float *ew = sm.ew[co & 1], *lr = sm.lr[sl];
                // W^T fragment for (row block J, token slice st): lane (q, n) holds
                // W[16J + n][32 st + 8q + m] = e^{lr_j - lr_{32 st}} ew[i]  (i < j)
                auto wfrag = [&](int J, int st) __attribute__((always_inline)) {
                    const int j = 16 * J + n, i0 = 32 * st + 8 * q;
                    const float ej = __expf(lr[j] - lr[32 * st]);
                    const v4f w0 = ld4(ew + i0), w1 = ld4(ew + i0 + 4);
                    float wv[8];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        wv[m] = i0 + m < j ? ej * w0[m] : 0.f;
                        wv[m + 4] = i0 + 4 + m < j ? ej * w1[m] : 0.f;
                    }
                    return __builtin_bit_cast(
                        v8s, make_uint4(pack2(wv[0], wv[1]), pack2(wv[2], wv[3]),
                                        pack2(wv[4], wv[5]), pack2(wv[6], wv[7])));
                };
                const v8s wa = wfrag(Ja, 0), wb0 = wfrag(Jb, 0), wb1 = wfrag(Jb, 1);
                const float *d0 = sm.d0[co % 3];
                const float rA = sm.rho[sl][16 * Ja + n], rB = sm.rho[sl][16 * Jb + n];
                const int64_t tA = int64_t(co) * CH + 16 * Ja + n, tB = int64_t(co) * CH + 16 * Jb + n;
#pragma unroll
                for (int ft = 0; ft < NF / 2; ++ft) {
                    const int F = (ow >> 1) * (NF / 2) + ft;
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
                    v4f accA = v4f{rA * dv[0], rA * dv[1], rA * dv[2], rA * dv[3]};
                    v4f accB = v4f{rB * dv[0], rB * dv[1], rB * dv[2], rB * dv[3]};
                    accA = mfma32(xa[0], wa, accA);
                    accB = mfma32(xa[0], wb0, accB);
                    accB = mfma32(xa[1], wb1, accB);
                    if (tA < T) store4(oq + tA * DK + 16 * F + 4 * q, accA);
                    if (tB < T) store4(oq + tB * DK + 16 * F + 4 * q, accB);
                }
            }
            block_sync();
        }
    } else if (wave != 4) {
        // keys of chunk c (waves 5 and 6): loaded into registers at the start of step c-3,
        // squared into LDS in step c-2; the two register sets alternate by step
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        if (nc > 1) load_keys(1, S0{});
        auto key_step = [&](int s, auto ld, auto sq) __attribute__((always_inline)) {
            if (s + 3 < nc) load_keys(s + 3, ld);
            if (s + 2 < nc) square_keys(s + 2, sq);
            block_sync();
        };
        for (int s = -1; s <= nc; s += 2) {
            key_step(s, S1{}, S0{});
            if (s + 1 <= nc) key_step(s + 1, S0{}, S1{});
        }
    } else {
        // gates of chunk c (wave 4, which shares a SIMD with the chain wave, so its load is
        // light): loaded in step c-3, scanned in step c-2
        float bv = 0.f, rv = 1.f;
        if (nc > 1) gates(1, bv, rv);
        for (int s = -1; s <= nc; ++s) {
            if (s + 2 < nc) scan(s + 2, bv, rv);
            if (s + 3 < nc) gates(s + 3, bv, rv);
            if (s + 1 < nc) gram2(s + 1, 8, 9);
            block_sync();
        }
    }
    if (d_next && threadIdx.x < DK) d_next[bh * DK + threadIdx.x] = sm.d0[nc % 3][threadIdx.x];
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
