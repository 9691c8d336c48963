// Chunkwise OSDN forward on bf16 matrix cores (the OSDN_BF16 path), gfx950.
//
// The chunk algebra is the same as the fp32 path (derived from the token step of the OSDN
// technical summary, section 2.1, with the gated-delta decay of Erase-then-Delta Attention,
// section 2.2, eq. 4); for one chunk of C = 64 rows starting from state M:
//
//   a1  k~ = d (.) k;  g = running sum of ln(alpha);  gam = e^g;  w = e^{g_C - g}
//   a2  A = strictly-lower( diag(beta) (K K~^T) (.) e^{g_r - g_s} )         chunk Gram matrix
//   a3  U = (I + A)^{-1} R, R = diag(beta) (V - diag(gam) K M)              UT transform
//   a5  P = lower-inclusive( (Q K~^T) (.) e^{g_r - g_s} )                    intra-chunk scores
//   a6  O = diag(gam) Q M + P U;   M <- gam_C M + K~^T diag(w) U            read-out, carry
//
// One workgroup owns one (b,h) sequence and a BV-wide slice of the value columns (value
// columns are independent given the chunk's A and P), holds its dk x BV fp32 slice of the
// state in VGPRs across all chunks, and walks the chunks in order.
//
// Products run on MFMA with bf16 operands and fp32 accumulation: 16x16x32 for the K=dk and
// K=64 contractions, 16x16x16 for the 16x16 blocks of the triangular solve (its output layout
// equals its B-operand layout, so results chain through registers).  Products whose result
// feeds another product as an A operand are computed transposed (X^T = B^T A^T), so each
// lane holds four consecutive columns of one row.  The unit-lower-triangular solve is
// blocked by 16: each diagonal block is inverted in registers as
// (I+N)^{-1} = (I-N)(I+N^2)(I+N^4)(I+N^8) (N strictly lower, N^16 = 0), and U comes from
// block forward substitution U_i = D_i (R_i - sum_{k<i} A_ik U_k).
//
// Software pipeline over chunks.  The state-independent work of chunk c+1 (staging k~, the
// decay scan, the Gram and score tiles, the block inverses) and the HBM loads of chunk c+2
// run beside the state-dependent work of chunk c, in three barrier-separated phases:
//   A  chunk c:   R, block substitution -> U          chunk c+1: k~, decay scan
//                 loads of chunk c+2: q, k (straight into LDS), d, beta, alpha (registers)
//   B  chunk c:   O = gam Q M + P U (to HBM), M <- gam_C M + K~^T (w U)
//      chunk c+1: Gram and score tiles, block inverses;   loads of chunk c+2: v (into LDS)
//   C  chunk c+1: K M and (Q M)^T;  wait for the chunk c+2 loads
// q, k and v are double-buffered in LDS (written by global_load_lds, 16 bytes per lane, with
// the 16-byte units of each q/k row XOR-swizzled by the row index so MFMA operand reads are
// bank-conflict free); k~, P and the block inverses are double-buffered by chunk parity.
// Each q/k/v buffer is its own __shared__ variable and the loop body is instantiated per
// chunk parity, so every buffer is known at compile time: the compiler can then tell that
// LDS reads of one buffer do not depend on the in-flight global_load_lds into another, and
// waits for those loads only where the kernel asks (before the phase-C barrier).
#include <type_traits>

#include "osdn_internal.h"

namespace osdn {
namespace {

typedef short v8s __attribute__((__vector_size__(8 * sizeof(short))));
typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
typedef float v4f __attribute__((__vector_size__(4 * sizeof(float))));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

constexpr int CH = 64;  // rows per chunk
constexpr int NBLK = CH / 16;
constexpr int NOFF = NBLK * (NBLK - 1) / 2;  // off-diagonal 16x16 blocks of the Gram matrix
constexpr int NGP = 16;  // off-diagonal Gram tiles (6) + score tiles (10)

// tile t of the Gram/score list: t < 6 is Gram (i,k), i > k; t >= 6 is score (i,k), i >= k
__device__ __forceinline__ void gp_tile(int t, int &i, int &kb) {
    constexpr int TI[NGP] = {1, 2, 2, 3, 3, 3, 0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int TK[NGP] = {0, 0, 1, 0, 1, 2, 0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    i = TI[t];
    kb = TK[t];
}

__device__ __forceinline__ v4f mfma32(v8s a, v8s b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma16(v4s a, v4s b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {  // one v_cvt_pk_bf16_f32
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint2 pack4u(v4f x) {
    return make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
}
__device__ __forceinline__ v4s pack4(v4f x) { return __builtin_bit_cast(v4s, pack4u(x)); }
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ v4f zero4() { return v4f{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ v4f ld4(const float *p) {  // 16-byte aligned LDS read
    return *reinterpret_cast<const v4f *>(p);
}
__device__ __forceinline__ v8s ld8(const uint16_t *p) {  // 16-byte aligned LDS read
    return *reinterpret_cast<const v8s *>(p);
}
__device__ __forceinline__ v4s ld4s(const uint16_t *p) {  // 8-byte aligned LDS read
    return *reinterpret_cast<const v4s *>(p);
}
// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane j addresses 8
// bytes (four bf16); lane i receives element i%4 of the four addressed by lane 4e + i/4, for
// e = 0..3.  With a row-major matrix X and lane j addressing X[k0 + j/4][n0 + 4(j%4)], lane i
// receives X[k0 + e][n0 + i], e = 0..3: the B-operand layout of the 16x16x16 product.
__device__ __forceinline__ v4s ld_tr(const uint16_t *p) {
    return __builtin_bit_cast(
        v4s, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p)));
}
__device__ __forceinline__ v8s cat8(v4s lo, v4s hi) {
    return v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// 16 bytes from global memory straight into LDS: lane l's bytes land at lds_base + 16 l
__device__ __forceinline__ void load_to_lds16(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds((glb_void_t *)(g), (lds_void_t *)(lds_base), 16, 0, 0);
}
// Workgroup barrier for LDS hand-offs: wait for this wave's LDS operations, then s_barrier.
// Unlike __syncthreads() it does not wait for outstanding global memory operations.  The
// waits are the s_waitcnt builtin (not inline asm) so the compiler's own wait insertion knows
// the counters they drain; the empty asm statements keep memory accesses on their side.
__device__ __forceinline__ void block_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_global() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    asm volatile("" ::: "memory");
}

template <int DK, int BV>
struct alignas(16) Smem {
    static constexpr int KU = DK / 8;   // 16-byte units per q/k row
    static constexpr int KP = DK + 8;   // row pitch (bf16) of k~ and the state copy
    static constexpr int CP = CH + 8;   // row pitch (bf16) of chunk-indexed rows
    static constexpr int DP = 16 + 4;   // row pitch (bf16) of 16x16 blocks
    // element offset of logical 16-byte unit u of row r in a swizzled q/k tile
    __device__ static constexpr int qk_at(int r, int u) { return (r * KU + (u ^ (r & 7))) * 8; }
    alignas(16) uint16_t kt[2][CH * KP];  // [chunk parity] k~, row-major
    alignas(16) uint16_t p[2][CH * CP];   // [chunk parity] P, row-major
    alignas(16) uint16_t dinv[2][NBLK * 16 * DP];  // D_i = (I + A_ii)^{-1}, row-major
    alignas(16) uint16_t aneg[2][NOFF * 16 * DP];  // -A_ik (i > k), row-major
    alignas(16) uint16_t mT[BV * KP];     // bf16 state slice, transposed: [value col][feature]
    alignas(16) uint16_t uT[BV * CP];     // U^T: [value col][row]
    alignas(16) uint16_t uwT[BV * CP];    // (diag(w) U)^T
    alignas(16) float beta[2][CH];
    alignas(16) float g[2][CH];
    alignas(16) float gam[2][CH];
    alignas(16) float w[2][CH];
};

// d, beta and alpha of one chunk, one chunk ahead, in registers (beta and alpha on the last
// wave, which runs the decay scan)
template <int DK, int NW, typename TD>
struct DPrefetch {
    static constexpr int SEGS = DK / 16;                  // 16-feature segments per row
    static constexpr int ITEMS = CH * SEGS / (NW * 64);   // (row, segment) items per thread
    static constexpr int DV4 = sizeof(TD) * 16 / 16;      // uint4 per 16 d values
    uint4 d[ITEMS][DV4];
    float beta, alpha;
};

template <int DK, int NW, typename TD>
__device__ __forceinline__ void load_d(DPrefetch<DK, NW, TD> &pf, const TD *d,
                                       const float *beta, const float *alpha, int64_t row0,
                                       int n, int tid) {
    using PF = DPrefetch<DK, NW, TD>;
#pragma unroll
    for (int j = 0; j < PF::ITEMS; ++j) {
        const int it = tid + j * NW * 64, r = min(it / PF::SEGS, n - 1), s = it % PF::SEGS;
        const uint4 *src = reinterpret_cast<const uint4 *>(d + (row0 + r) * DK + 16 * s);
#pragma unroll
        for (int e = 0; e < PF::DV4; ++e) pf.d[j][e] = src[e];
    }
    const int lane = tid - (NW - 1) * 64;
    if (lane >= 0) {
        const int r = min(lane, n - 1);
        pf.beta = beta[row0 + r];
        if (alpha) pf.alpha = alpha[row0 + r];
    }
}

// q and k rows of one chunk into LDS buffer b (rows past the end re-read the last row)
template <int DK, int BV, int NW>
__device__ __forceinline__ void load_qk(uint16_t *qb, uint16_t *kb, const uint16_t *q,
                                        const uint16_t *k, int64_t row0, int n, int wave,
                                        int lane) {
    using S = Smem<DK, BV>;
    constexpr int PER_WAVE = CH * S::KU / (NW * 64);
    static_assert(CH * S::KU % (NW * 64) == 0, "whole wave-loads");
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int base = (wave * PER_WAVE + i) * 64;  // physical unit of lane 0
        const int pu = base + lane, r = pu / S::KU, lu = (pu % S::KU) ^ (r & 7);
        const int64_t off = (row0 + min(r, n - 1)) * DK + 8 * lu;
        load_to_lds16(q + off, qb + 8 * base);
        load_to_lds16(k + off, kb + 8 * base);
    }
}

template <int DK, int BV, int NW>
__device__ __forceinline__ void load_v(uint16_t *vb, const uint16_t *v, int64_t row0, int n,
                                       int dv, int j0, int wave, int lane) {
    constexpr int VU = BV / 8;  // 16-byte units per value row
    constexpr int PER_WAVE = CH * VU / (NW * 64);
    static_assert(CH * VU % (NW * 64) == 0, "whole wave-loads");
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int base = (wave * PER_WAVE + i) * 64;
        const int pu = base + lane, r = pu / VU, u = pu % VU;
        load_to_lds16(v + (row0 + min(r, n - 1)) * dv + j0 + 8 * u, vb + 8 * base);
    }
}

__device__ __forceinline__ void d_values(const uint4 *src, float *out, float) {
    const float *f = reinterpret_cast<const float *>(src);
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = f[e];
}
__device__ __forceinline__ void d_values(const uint4 *src, float *out, bf16_t) {
    const uint32_t *u = reinterpret_cast<const uint32_t *>(src);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        out[2 * e] = bf_lo(u[e]);
        out[2 * e + 1] = bf_hi(u[e]);
    }
}

// k~ = d (.) k for chunk buffer b, from the k tile in LDS and d in registers
template <int DK, int BV, int NW, typename TD>
__device__ __forceinline__ void stage_kt(Smem<DK, BV> &sm, int b, const uint16_t *kb,
                                         const DPrefetch<DK, NW, TD> &pf, int tid) {
    using S = Smem<DK, BV>;
    using PF = DPrefetch<DK, NW, TD>;
    uint4 kr[PF::ITEMS][2];
#pragma unroll
    for (int j = 0; j < PF::ITEMS; ++j) {
        const int it = tid + j * NW * 64, r = it / PF::SEGS, s = it % PF::SEGS;
        kr[j][0] = *reinterpret_cast<const uint4 *>(&kb[S::qk_at(r, 2 * s)]);
        kr[j][1] = *reinterpret_cast<const uint4 *>(&kb[S::qk_at(r, 2 * s + 1)]);
    }
#pragma unroll
    for (int j = 0; j < PF::ITEMS; ++j) {
        const int it = tid + j * NW * 64, r = it / PF::SEGS, s = it % PF::SEGS;
        float dv[16];
        d_values(pf.d[j], dv, TD{});
        const uint32_t *ku = reinterpret_cast<const uint32_t *>(kr[j]);
        uint32_t pk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pk[e] = pack2(dv[2 * e] * bf_lo(ku[e]), dv[2 * e + 1] * bf_hi(ku[e]));
        uint4 *dst = reinterpret_cast<uint4 *>(&sm.kt[b][r * S::KP + 16 * s]);
        dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    }
}

// decay scan of one chunk (one wave, one row per lane): rows past the end get beta = 0 and
// alpha = 1, so they leave U, M and every kept output unchanged
template <int DK, int BV, int NW, typename TD>
__device__ __forceinline__ void scan_chunk(Smem<DK, BV> &sm, int b,
                                           const DPrefetch<DK, NW, TD> &pf, int n,
                                           bool has_alpha, int lane) {
    const bool ok = lane < n;
    float x = (ok && has_alpha) ? __logf(pf.alpha) : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    const float glast = __shfl(x, 63);
    sm.beta[b][lane] = ok ? pf.beta : 0.f;
    sm.g[b][lane] = x;
    sm.gam[b][lane] = __expf(x);
    sm.w[b][lane] = __expf(glast - x);
}

// (I + N)^{-1} of diagonal block `wave` from its Gram tile G (C layout) and G^T (C layout,
// the A layout of G): N is the strictly-lower part of beta_r e^{g_r - g_s} G
template <int DK, int BV>
__device__ __forceinline__ void diag_inverse(Smem<DK, BV> &sm, int b, int wave, int lr, int lq,
                                             v4f Gd, v4f Gdt) {
    using S = Smem<DK, BV>;
    const int b0 = 16 * wave;
    const v4f g4 = ld4(&sm.g[b][b0 + 4 * lq]);
    const v4f bt4 = ld4(&sm.beta[b][b0 + 4 * lq]);
    const float g1 = sm.g[b][b0 + lr], bt1 = sm.beta[b][b0 + lr];
    v4f Nc, Na_f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // C layout: row 4lq+e, column lr;  A layout: row lr, column 4lq+e
        Nc[e] = (lr < 4 * lq + e) ? bt4[e] * __expf(g4[e] - g1) * Gd[e] : 0.f;
        Na_f[e] = (4 * lq + e < lr) ? bt1 * __expf(g1 - g4[e]) * Gdt[e] : 0.f;
    }
    const v4s Na = pack4(Na_f), Nb = pack4(Nc);
    // squares in both layouts: X^2 (C = B layout) = X X;  (X^2)^T (C = A layout) = X^T X^T
    const v4f N2 = mfma16(Na, Nb, zero4());
    const v4f N2t = mfma16(Nb, Na, zero4());
    const v4s N2a = pack4(N2t), N2b = pack4(N2);
    const v4f N4 = mfma16(N2a, N2b, zero4());
    const v4f N4t = mfma16(N2b, N2a, zero4());
    const v4s N4a = pack4(N4t), N4b = pack4(N4);
    // D^T = (I - N^T)(I + N^2T)(I + N^4T)(I + N^8T), built in C layout = A layout of D
    v4f Y = mfma16(N4b, N4a, zero4());  // (N^8)^T
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (4 * lq + e == lr) Y[e] += 1.f;
    Y = mfma16(N4b, pack4(Y), Y);
    Y = mfma16(N2b, pack4(Y), Y);
    Y = mfma16(pack4(-Nc), pack4(Y), Y);
    *reinterpret_cast<uint2 *>(&sm.dinv[b][wave * 16 * S::DP + lr * S::DP + 4 * lq]) = pack4u(Y);
}

// Gram and score tiles of chunk parity b, scaled and masked; the block inverses
template <int DK, int BV, int NW>
__device__ __forceinline__ void prep_tiles(Smem<DK, BV> &sm, int b, const uint16_t *qb,
                                           const uint16_t *kb, int wave, int lr, int lq) {
    using S = Smem<DK, BV>;
    constexpr int KS = DK / 32;
    constexpr int GPW = (NGP + NW - 1) / NW;
    // operand fragments of a batch first, then its products (two tiles per batch)
    v8s dk_[KS], dt_[KS];
    if (wave < NBLK) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            dk_[kk] = ld8(&kb[S::qk_at(16 * wave + lr, 4 * kk + lq)]);
            dt_[kk] = ld8(&sm.kt[b][(16 * wave + lr) * S::KP + 32 * kk + 8 * lq]);
        }
    }
    v4f GP[GPW];
#pragma unroll
    for (int j0 = 0; j0 < GPW; j0 += 2) {
        v8s fa[2][KS], fb[2][KS];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int t = wave + (j0 + jj) * NW;
            if (j0 + jj < GPW && t < NGP) {
                int i, kc;
                gp_tile(t, i, kc);
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    fa[jj][kk] = ld8(&sm.kt[b][(16 * kc + lr) * S::KP + 32 * kk + 8 * lq]);
                if (t < 6) {
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk)
                        fb[jj][kk] = ld8(&kb[S::qk_at(16 * i + lr, 4 * kk + lq)]);
                } else {
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk)
                        fb[jj][kk] = ld8(&qb[S::qk_at(16 * i + lr, 4 * kk + lq)]);
                }
            }
        }
        if (j0 == 0) {
            // diagonal block: G in C layout and G^T in C layout (= A layout of G)
            if (wave < NBLK) {
                v4f Gd = zero4(), Gdt = zero4();
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    Gd = mfma32(dk_[kk], dt_[kk], Gd);
                    Gdt = mfma32(dt_[kk], dk_[kk], Gdt);
                }
                diag_inverse<DK, BV>(sm, b, wave, lr, lq, Gd, Gdt);
            }
        }
        // off-diagonal Gram and score tiles, transposed: tile (i,k) = K~_k X_i^T with X = K
        // or Q, so the lane holds row 16i+lr, columns 16k+4lq..+3 of block (i,k)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            if (j0 + jj < GPW) {
                GP[j0 + jj] = zero4();
                if (wave + (j0 + jj) * NW < NGP) {
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk)
                        GP[j0 + jj] = mfma32(fa[jj][kk], fb[jj][kk], GP[j0 + jj]);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int t = wave + j * NW;
        if (t < NGP) {
            int i, kb;
            gp_tile(t, i, kb);
            const int r = 16 * i + lr;
            const float gr = sm.g[b][r];
            const v4f gs = ld4(&sm.g[b][16 * kb + 4 * lq]);
            v4f val;
            if (t < 6) {
                const float nb = -sm.beta[b][r];
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = nb * __expf(gr - gs[e]) * GP[j][e];
                *reinterpret_cast<uint2 *>(&sm.aneg[b][t * 16 * S::DP + lr * S::DP + 4 * lq]) =
                    pack4u(val);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * kb + 4 * lq + e;
                    val[e] = s <= r ? __expf(gr - gs[e]) * GP[j][e] : 0.f;
                }
                *reinterpret_cast<uint2 *>(&sm.p[b][r * S::CP + 16 * kb + 4 * lq]) =
                    pack4u(val);
            }
        }
    }
}

// K M (C layout) on the substitution waves, (Q M)^T on the read-out waves, for chunk buffer b
template <int DK, int BV, int NW>
__device__ __forceinline__ void state_products(const Smem<DK, BV> &sm, const uint16_t *qb,
                                               const uint16_t *kb, int wave, int lr, int lq,
                                               v4f (&XM)[NBLK]) {
    using S = Smem<DK, BV>;
    constexpr int NCT = BV / 16;
    constexpr int KS = DK / 32;
    const bool km_wave = wave < NCT;
    const int ct = km_wave ? wave : wave - NCT;
    v8s fx[KS], fr[NBLK][KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) fx[kk] = ld8(&sm.mT[(16 * ct + lr) * S::KP + 32 * kk + 8 * lq]);
    if (km_wave) {
#pragma unroll
        for (int rt = 0; rt < NBLK; ++rt)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                fr[rt][kk] = ld8(&kb[S::qk_at(16 * rt + lr, 4 * kk + lq)]);
    } else {
#pragma unroll
        for (int rt = 0; rt < NBLK; ++rt)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                fr[rt][kk] = ld8(&qb[S::qk_at(16 * rt + lr, 4 * kk + lq)]);
    }
    if (km_wave) {
#pragma unroll
        for (int rt = 0; rt < NBLK; ++rt) {
            v4f acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) acc = mfma32(fr[rt][kk], fx[kk], acc);
            XM[rt] = acc;
        }
    } else {
#pragma unroll
        for (int rt = 0; rt < NBLK; ++rt) {
            v4f acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) acc = mfma32(fx[kk], fr[rt][kk], acc);
            XM[rt] = acc;
        }
    }
}

template <int DK, int BV, int NW, typename TD>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
chunk_mfma_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const uint16_t *__restrict__ v, const TD *__restrict__ d,
                  const float *__restrict__ beta, const float *__restrict__ alpha,
                  const float *S0, uint16_t *__restrict__ o, float *S_T, int64_t BH,
                  int64_t T, int dv) {
    using S = Smem<DK, BV>;
    constexpr int NCT = BV / 16;                 // 16-wide value-column tiles
    constexpr int NRT = DK / 16;                 // 16-row key-feature tiles of the state
    constexpr int MT = NRT * NCT / NW;           // state tiles per wave
    constexpr int KC = CH / 32;                  // k-steps over the chunk rows
    static_assert(NW == 2 * NCT, "one substitution wave and one read-out wave per 16 columns");
    static_assert(NW >= NBLK, "one wave per diagonal block");
    static_assert((NRT * NCT) % NW == 0, "state tiles split evenly");

    __shared__ S sm;
    // q, k, v buffers: one __shared__ variable each (see the file comment)
    __shared__ alignas(16) uint16_t q_buf0[CH * DK], q_buf1[CH * DK];
    __shared__ alignas(16) uint16_t k_buf0[CH * DK], k_buf1[CH * DK];
    __shared__ alignas(16) uint16_t v_buf0[CH * BV], v_buf1[CH * BV];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15;        // row (A) / column (B, C) index inside a 16-tile
    const int lq = lane >> 4;        // quarter: k-offset (A, B) / row group (C)
    const bool km_wave = wave < NCT; // K M, R, substitution for value tile `wave`
    const int scan_wave = NW - 1;

    // workgroup -> (sequence, value slice); slices of one sequence share an XCD (and its L2)
    const int nvt = dv / BV;
    int64_t bh;
    int vt;
    if ((BH & 7) == 0) {
        const int64_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        vt = static_cast<int>(slot % nvt);
        bh = (slot / nvt) * 8 + xcd;
    } else {
        vt = static_cast<int>(blockIdx.x % nvt);
        bh = blockIdx.x / nvt;
    }
    const int j0 = vt * BV;
    const int64_t seq0 = bh * T;  // first token row of the sequence
    const bool has_alpha = alpha != nullptr;

    // score tiles above the diagonal are read as zeros by the read-out and never written
    for (int i = tid; i < 2 * CH * S::CP; i += NW * 64) (&sm.p[0][0])[i] = 0;

    // ---- state slice in registers (C layout of 16x16 tiles) --------------------------------
    v4f M[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int tt = wave + t * NW, rt = tt / NCT, ct = tt % NCT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * lq + i, col = j0 + 16 * ct + lr;
            M[t][i] = S0 ? S0[(bh * DK + row) * dv + col] : 0.f;
        }
        *reinterpret_cast<uint2 *>(&sm.mT[(16 * ct + lr) * S::KP + 16 * rt + 4 * lq]) =
            pack4u(M[t]);
    }

    const int64_t nchunks = (T + CH - 1) / CH;
    auto rows_of = [&](int64_t cc) {
        return static_cast<int>(T - cc * CH < CH ? T - cc * CH : CH);
    };

    DPrefetch<DK, NW, TD> pf;
    v4f XM[NBLK];
    if (nchunks > 0) {
        // prologue: chunk 0 loaded and prepared, chunk 1 loading
        const int n0 = rows_of(0);
        load_qk<DK, BV, NW>(q_buf0, k_buf0, q, k, seq0, n0, wave, lane);
        load_v<DK, BV, NW>(v_buf0, v, seq0, n0, dv, j0, wave, lane);
        load_d<DK, NW, TD>(pf, d, beta, alpha, seq0, n0, tid);
        wait_global();
        block_sync();
        stage_kt<DK, BV, NW, TD>(sm, 0, k_buf0, pf, tid);
        if (wave == scan_wave) scan_chunk<DK, BV, NW, TD>(sm, 0, pf, n0, has_alpha, lane);
        if (nchunks > 1) {
            const int n1 = rows_of(1);
            load_qk<DK, BV, NW>(q_buf1, k_buf1, q, k, seq0 + CH, n1, wave, lane);
            load_v<DK, BV, NW>(v_buf1, v, seq0 + CH, n1, dv, j0, wave, lane);
            load_d<DK, NW, TD>(pf, d, beta, alpha, seq0 + CH, n1, tid);
        }
        block_sync();
        prep_tiles<DK, BV, NW>(sm, 0, q_buf0, k_buf0, wave, lr, lq);
        state_products<DK, BV, NW>(sm, q_buf0, k_buf0, wave, lr, lq, XM);
        wait_global();
        block_sync();
    }

    // One pipelined iteration for chunk c; the chunk parity P is a compile-time constant so
    // every q/k/v buffer reference is static.
    auto iteration = [&](auto parity, int64_t c) {
        constexpr int P = decltype(parity)::value;
        uint16_t *q_cur = P ? q_buf1 : q_buf0, *q_nxt = P ? q_buf0 : q_buf1;
        uint16_t *k_cur = P ? k_buf1 : k_buf0, *k_nxt = P ? k_buf0 : k_buf1;
        uint16_t *v_cur = P ? v_buf1 : v_buf0;
        const int b0 = P, b1 = P ^ 1;
        const bool has1 = c + 1 < nchunks, has2 = c + 2 < nchunks;
        const int n = rows_of(c);
        const int64_t row0 = seq0 + c * CH;

        // ---- phase A ------------------------------------------------------------------------
        if (km_wave) {
            // R = beta (V - gam (K M)) for value tile `wave`, then U by block substitution
            const int ct = wave;
            v4s vt4[NBLK], dA[NBLK], aN[NOFF];
            v4f bt4[NBLK], gm4[NBLK];
#pragma unroll
            for (int rt = 0; rt < NBLK; ++rt) {
                // transposing read: lane gets V[16rt + 4lq + e][16ct + lr]
                vt4[rt] = ld_tr(&v_cur[(16 * rt + 4 * lq + (lr >> 2)) * BV + 16 * ct +
                                       4 * (lr & 3)]);
                bt4[rt] = ld4(&sm.beta[b0][16 * rt + 4 * lq]);
                gm4[rt] = ld4(&sm.gam[b0][16 * rt + 4 * lq]);
                dA[rt] = ld4s(&sm.dinv[b0][rt * 16 * S::DP + lr * S::DP + 4 * lq]);
            }
#pragma unroll
            for (int u = 0; u < NOFF; ++u)
                aN[u] = ld4s(&sm.aneg[b0][u * 16 * S::DP + lr * S::DP + 4 * lq]);
            v4f U[NBLK];
#pragma unroll
            for (int i = 0; i < NBLK; ++i) {
                v4f Y;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Y[e] = bt4[i][e] * (__uint_as_float(static_cast<uint32_t>(
                                            static_cast<uint16_t>(vt4[i][e])) << 16) -
                                        gm4[i][e] * XM[i][e]);
#pragma unroll
                for (int kb = 0; kb < i; ++kb)
                    Y = mfma16(aN[(i * (i - 1)) / 2 + kb], pack4(U[kb]), Y);
                U[i] = mfma16(dA[i], pack4(Y), zero4());
            }
#pragma unroll
            for (int i = 0; i < NBLK; ++i) {
                const int r0 = 16 * i + 4 * lq;
                const v4f w4 = ld4(&sm.w[b0][r0]);
                const int row = 16 * ct + lr;
                *reinterpret_cast<uint2 *>(&sm.uT[row * S::CP + r0]) = pack4u(U[i]);
                *reinterpret_cast<uint2 *>(&sm.uwT[row * S::CP + r0]) = pack4u(w4 * U[i]);
            }
        }
        if (has1) {
            stage_kt<DK, BV, NW, TD>(sm, b1, k_nxt, pf, tid);
            if (wave == scan_wave)
                scan_chunk<DK, BV, NW, TD>(sm, b1, pf, rows_of(c + 1), has_alpha, lane);
        }
        if (has2) {
            const int n2 = rows_of(c + 2);
            load_d<DK, NW, TD>(pf, d, beta, alpha, row0 + 2 * CH, n2, tid);
            load_qk<DK, BV, NW>(q_cur, k_cur, q, k, row0 + 2 * CH, n2, wave, lane);
        }
        block_sync();

        // ---- phase B ------------------------------------------------------------------------
        {
            // read-out of chunk c (read-out waves) and state carry (all waves); fragments first
            v8s au[KC], pb[NBLK][KC];
            float gr[NBLK];
            if (!km_wave) {
                const int ct = wave - NCT;
#pragma unroll
                for (int kk = 0; kk < KC; ++kk)
                    au[kk] = ld8(&sm.uT[(16 * ct + lr) * S::CP + 32 * kk + 8 * lq]);
#pragma unroll
                for (int rt = 0; rt < NBLK; ++rt) {
                    const int r = 16 * rt + lr;
                    gr[rt] = sm.gam[b0][r];
#pragma unroll
                    for (int kk = 0; kk <= rt / 2; ++kk)
                        pb[rt][kk] = ld8(&sm.p[b0][r * S::CP + 32 * kk + 8 * lq]);
                }
            }
            v8s ma[MT][KC], mb[MT][KC];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int tt = wave + t * NW, rt = tt / NCT, ct = tt % NCT;
#pragma unroll
                for (int kk = 0; kk < KC; ++kk) {
                    // A = K~^T by transposing reads of row-major K~: rows 32kk + 8lq + e
                    const uint16_t *base = &sm.kt[b0][(32 * kk + 8 * lq + (lr >> 2)) * S::KP +
                                                      16 * rt + 4 * (lr & 3)];
                    ma[t][kk] = cat8(ld_tr(base), ld_tr(base + 4 * S::KP));
                    mb[t][kk] = ld8(&sm.uwT[(16 * ct + lr) * S::CP + 32 * kk + 8 * lq]);
                }
            }
            const float gC = sm.gam[b0][CH - 1];
            if (!km_wave) {
                // O^T tile = (gam Q M)^T + U^T P^T: lane holds O[row 16rt+lr][4 value columns]
                const int ct = wave - NCT;
#pragma unroll
                for (int rt = 0; rt < NBLK; ++rt) {
                    const int r = 16 * rt + lr;
                    v4f acc = gr[rt] * XM[rt];
#pragma unroll
                    for (int kk = 0; kk <= rt / 2; ++kk) acc = mfma32(au[kk], pb[rt][kk], acc);
                    if (r < n)
                        *reinterpret_cast<uint2 *>(o + (row0 + r) * dv + j0 + 16 * ct + 4 * lq) =
                            pack4u(acc);
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int tt = wave + t * NW, rt = tt / NCT, ct = tt % NCT;
                v4f acc = gC * M[t];
#pragma unroll
                for (int kk = 0; kk < KC; ++kk) acc = mfma32(ma[t][kk], mb[t][kk], acc);
                M[t] = acc;
                *reinterpret_cast<uint2 *>(&sm.mT[(16 * ct + lr) * S::KP + 16 * rt + 4 * lq]) =
                    pack4u(acc);
            }
        }
        if (has1) prep_tiles<DK, BV, NW>(sm, b1, q_nxt, k_nxt, wave, lr, lq);
        if (has2) load_v<DK, BV, NW>(v_cur, v, row0 + 2 * CH, rows_of(c + 2), dv, j0, wave, lane);
        block_sync();

        // ---- phase C ------------------------------------------------------------------------
        if (has1) state_products<DK, BV, NW>(sm, q_nxt, k_nxt, wave, lr, lq, XM);
        wait_global();
        block_sync();
    };

    for (int64_t c = 0; c < nchunks; c += 2) {
        iteration(std::integral_constant<int, 0>{}, c);
        if (c + 1 < nchunks) iteration(std::integral_constant<int, 1>{}, c + 1);
    }

    if (S_T) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int tt = wave + t * NW, rt = tt / NCT, ct = tt % NCT;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rt + 4 * lq + i, col = j0 + 16 * ct + lr;
                S_T[(bh * DK + row) * dv + col] = M[t][i];
            }
        }
    }
}

template <int DK, typename TD>
hipError_t launch_typed(const ChunkArgs &a, hipStream_t stream) {
    constexpr int BV = 32, NW = 4;
    const int nvt = a.dv / BV;
    const dim3 grid(static_cast<unsigned>(a.BH * nvt));
    hipLaunchKernelGGL((chunk_mfma_kernel<DK, BV, NW, TD>), grid, dim3(NW * 64), 0, stream,
                       static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
                       static_cast<const uint16_t *>(a.v), static_cast<const TD *>(a.d),
                       a.beta, a.alpha, a.S0, static_cast<uint16_t *>(a.o), a.S_T, a.BH, a.T,
                       a.dv);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_fwd_mfma(const ChunkArgs &a, hipStream_t stream) {
    if (a.dk == 64)
        return a.d_dtype == OSDN_F32 ? launch_typed<64, float>(a, stream)
                                     : launch_typed<64, bf16_t>(a, stream);
    return a.d_dtype == OSDN_F32 ? launch_typed<128, float>(a, stream)
                                 : launch_typed<128, bf16_t>(a, stream);
}

}  // namespace osdn
