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
// One workgroup of five waves owns one (b,h) sequence and a 32-wide slice of the value
// columns (value columns are independent given the chunk's A and P) and walks the chunks in
// order, with one barrier per chunk step.  The waves have three roles, each running its own
// loop with the same barriers:
//
// * State waves (0, 1), one per 16 value columns.  A state wave holds its dk x 16 slice of M
//   in VGPRs (fp32, the C layout of 16x16 MFMA tiles) for the whole sequence and runs the
//   state-dependent chain of chunk c without touching LDS for M or U: R, the block forward
//   substitution U_i = D_i (R_i - sum_{k<i} A_ik U_k) (16x16x16 products; their output layout
//   equals their B-operand layout), the read-out O^T = (M^T Q^T) diag(gam) + U^T P^T, the
//   carry M <- gam_C M + K~^T (w U), and then K M and M^T Q^T of chunk c+1.
//   A pair of 16x16 C-layout tiles becomes one 16x16x32 operand fragment with two packs and
//   four lane swaps (v_permlane32_swap, v_permlane16_swap): lane (quarter q, column n) then
//   holds rows 8q..8q+7 of the 32-row pair, which is both the B layout of the pair and the
//   A layout of its transpose.  So every K-slot runs in natural order and each q, k and P
//   operand fragment is a single 16-byte LDS read.
// * Prep waves (2, 3) work one chunk ahead: k~ of chunk c+1 (from the k tile and d prefetched
//   into registers a chunk earlier), its Gram and score tiles, and the inverses
//   D_i = (I + A_ii)^{-1} of the diagonal blocks, computed in registers as
//   (I-N)(I+N^2)(I+N^4)(I+N^8) (N strictly lower, N^16 = 0).  The tiles are split by column
//   block: wave 2 takes blocks {0,3}, wave 3 blocks {1,2}, ten tiles each, so each wave builds
//   only its own k~ blocks and needs no other wave's k~.
// * The loader wave (4) issues the q, k, v loads of chunk c+2 straight into LDS and runs the
//   decay scan of chunk c+2.  Issuing loads stalls while HBM drains them; here that stall
//   falls on a wave with little else to do.
//
// q, k and v reach LDS by global_load_lds (16 bytes per lane; the 16-byte units of each q/k
// row are XOR-swizzled by the row index so fragment reads are bank-conflict free), double-
// buffered by chunk parity; the state waves read the v tile of chunk c+1 into registers at
// the end of step c.  k~, P and the block inverses are double-buffered by chunk parity, the
// scan outputs by chunk mod 3.  Every wave drains its global memory operations before the
// end-of-step barrier.
#include <type_traits>

#include "osdn_internal.h"

namespace osdn {
namespace {

typedef short v8s __attribute__((__vector_size__(8 * sizeof(short))));
typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
typedef float v4f __attribute__((__vector_size__(4 * sizeof(float))));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

constexpr int CH = 64;                       // rows per chunk
constexpr int NBLK = CH / 16;                // 16-row blocks per chunk
constexpr int NOFF = NBLK * (NBLK - 1) / 2;  // off-diagonal 16x16 blocks of the Gram matrix
constexpr int BV = 32;                       // value columns per workgroup
constexpr int NW = 5;                        // waves per workgroup: 2 state, 2 prep, 1 loader
constexpr int VW = 16;                       // value columns per state wave

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
// receives X[k0 + e][n0 + i], e = 0..3.
__device__ __forceinline__ v4s ld_tr(const uint16_t *p) {
    return __builtin_bit_cast(
        v4s, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p)));
}
__device__ __forceinline__ v8s cat8(v4s lo, v4s hi) {
    return v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Two 16x16 fp32 tiles in C layout (lane (q, n) holds rows 4q..4q+3 of column n; x0 is rows
// 0..15 of a 32-row pair, x1 rows 16..31) -> one bf16 fragment in which lane (q, n) holds
// rows 8q..8q+7 of column n.  permlane32_swap(a, b) returns (a.r0 a.r1 b.r0 b.r1) and
// (a.r2 a.r3 b.r2 b.r3), permlane16_swap(a, b) returns (a.r0 b.r0 a.r2 b.r2) and
// (a.r1 b.r1 a.r3 b.r3), with r0..r3 the four 16-lane rows.
__device__ __forceinline__ v8s c_to_frag(v4f x0, v4f x1) {
    const uint32_t a0 = pack2(x0[0], x0[1]), a1 = pack2(x0[2], x0[3]);
    const uint32_t b0 = pack2(x1[0], x1[1]), b1 = pack2(x1[2], x1[3]);
    const u32x2 s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
    const u32x2 s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
    const u32x2 t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
    const u32x2 t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
    return __builtin_bit_cast(v8s, make_uint4(t0[0], t1[0], t0[1], t1[1]));
}
// 16 bytes from global memory straight into LDS: lane l's bytes land at lds_base + 16 l
__device__ __forceinline__ void load_to_lds16(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds((glb_void_t *)(g), (lds_void_t *)(lds_base), 16, 0, 0);
}
// Workgroup barrier for LDS hand-offs: wait for this wave's LDS operations, then s_barrier.
// The waits are the s_waitcnt builtin (not inline asm) so the compiler's own wait insertion
// knows the counters they drain; the empty asm statements keep memory accesses on their side.
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

template <int DK>
struct alignas(16) Lds {
    static constexpr int KU = DK / 8;   // 16-byte units per q/k row
    static constexpr int KP = DK + 8;   // row pitch (bf16) of k~
    static constexpr int CP = CH + 8;   // row pitch (bf16) of P
    static constexpr int DP = 16 + 4;   // row pitch (bf16) of 16x16 blocks
    // element offset of logical 16-byte unit u of row r in a swizzled q/k tile
    __device__ static constexpr int qk_at(int r, int u) { return (r * KU + (u ^ (r & 7))) * 8; }
    alignas(16) uint16_t kt[2][CH * KP];            // [chunk parity] k~, row-major
    alignas(16) uint16_t p[2][CH * CP];             // [chunk parity] P, row-major
    alignas(16) uint16_t dinv[2][NBLK * 16 * DP];   // D_i = (I + A_ii)^{-1}, row-major
    alignas(16) uint16_t aneg[2][NOFF * 16 * DP];   // -A_ik (i > k), row-major
    alignas(16) float beta[3][CH];                  // [chunk mod 3] scan outputs
    alignas(16) float g[3][CH];
    alignas(16) float gam[3][CH];
    alignas(16) float w[3][CH];
    // decay factors of off-diagonal 16x16 tiles (i > k), all <= 1:
    // e^{g_r - g_s} = ea[r] * cik[t(i,k)] * eb[s] with ea[r] = e^{g_r - g_{16i}},
    // cik = e^{g_{16i} - g_{16k+15}}, eb[s] = e^{g_{16k+15} - g_s}
    alignas(16) float ea[3][CH];
    alignas(16) float eb[3][CH];
    alignas(16) float cik[3][8];
    alignas(16) uint16_t ntile[NBLK][16 * 16];  // N of diagonal block kb, row-major (prep)
};

// Prep wave pw owns the Gram/score column blocks kblk(pw, 0), kblk(pw, 1)
__host__ __device__ constexpr int kblk(int pw, int j) { return pw == 0 ? (j == 0 ? 0 : 3) : (j == 0 ? 1 : 2); }

// d of a prep wave's two blocks, one chunk ahead (fragment layout: lane (q, n) holds row
// 16 kb + n, features 32 s + 8 q .. +7)
template <int DK, typename TD>
struct PrepRegs {
    static constexpr int NS = DK / 32;
    static constexpr int DU = sizeof(TD) * 8 / 16;  // uint4 per 8 values of d
    uint4 d[2][NS][DU];
};

template <int DK, typename TD, int PW>
__device__ __forceinline__ void load_d_frag(PrepRegs<DK, TD> &pr, const TD *d, int64_t row0,
                                            int n, int lr, int lq) {
    using PR = PrepRegs<DK, TD>;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = min(16 * kblk(PW, j) + lr, n - 1);
#pragma unroll
        for (int s = 0; s < PR::NS; ++s) {
            const uint4 *src = reinterpret_cast<const uint4 *>(d + (row0 + r) * DK + 32 * s + 8 * lq);
#pragma unroll
            for (int e = 0; e < PR::DU; ++e) pr.d[j][s][e] = src[e];
        }
    }
}

__device__ __forceinline__ void d_values(const uint4 *src, float *out, float) {
    const float *f = reinterpret_cast<const float *>(src);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = f[e];
}
__device__ __forceinline__ void d_values(const uint4 *src, float *out, bf16_t) {
    const uint32_t *u = reinterpret_cast<const uint32_t *>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        out[2 * e] = bf_lo(u[e]);
        out[2 * e + 1] = bf_hi(u[e]);
    }
}

// q and k rows of one chunk into LDS (loader wave; rows past the end re-read the last row)
template <int DK>
__device__ __forceinline__ void load_qk(uint16_t *qb, uint16_t *kb, const uint16_t *q,
                                        const uint16_t *k, int64_t row0, int n, int lane) {
    using L = Lds<DK>;
    constexpr int NLOAD = CH * L::KU / 64;
    static_assert(CH * L::KU % 64 == 0, "whole wave-loads");
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
        const int base = i * 64;  // physical unit of lane 0
        const int pu = base + lane, r = pu / L::KU, lu = (pu % L::KU) ^ (r & 7);
        const int64_t off = (row0 + min(r, n - 1)) * DK + 8 * lu;
        load_to_lds16(q + off, qb + 8 * base);
        load_to_lds16(k + off, kb + 8 * base);
    }
}

// the workgroup's 64 x 32 slice of v into LDS as [value tile][row][16] (loader wave)
__device__ __forceinline__ void load_v(uint16_t *vb, const uint16_t *v, int64_t row0, int n,
                                       int dv, int j0, int lane) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const int vt = ii >> 1, h = ii & 1;
        const int r = 32 * h + (lane >> 1);
        load_to_lds16(v + (row0 + min(r, n - 1)) * dv + j0 + VW * vt + 8 * (lane & 1),
                      vb + (vt * CH + 32 * h) * VW);
    }
}

// x + (x of the lane selected by the DPP control), 0 where the control selects no lane
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false);
    return x + __int_as_float(y);
}
__device__ __forceinline__ float lane_value(float x, int l) {  // x of lane l (wave-uniform)
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// one of four wave-uniform values, chosen by the lane's 16-lane block
__device__ __forceinline__ float per_block(float v0, float v1, float v2, float v3, int lane) {
    const int b = lane >> 4;
    return b == 0 ? v0 : (b == 1 ? v1 : (b == 2 ? v2 : v3));
}

// decay scan of one chunk (one wave, one row per lane): rows past the end get beta = 0 and
// alpha = 1, so they leave U, M and every kept output unchanged.  The inclusive prefix sum of
// ln(alpha) runs on DPP: shifts by 1, 2, 4, 8 inside each 16-lane row, then the last lane of
// rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3.
template <int DK>
__device__ __forceinline__ void scan_chunk(Lds<DK> &sm, int slot, float beta, float alpha, int n,
                                           bool has_alpha, int lane) {
    const bool ok = lane < n;
    float x = (ok && has_alpha) ? __logf(alpha) : 0.f;
    x = dpp_add<0x111, 0xf>(x);  // row_shr:1
    x = dpp_add<0x112, 0xf>(x);  // row_shr:2
    x = dpp_add<0x114, 0xf>(x);  // row_shr:4
    x = dpp_add<0x118, 0xf>(x);  // row_shr:8
    x = dpp_add<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
    x = dpp_add<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
    const float s0 = lane_value(x, 0), e0 = lane_value(x, 15);
    const float s1 = lane_value(x, 16), e1 = lane_value(x, 31);
    const float s2 = lane_value(x, 32), e2 = lane_value(x, 47);
    const float s3 = lane_value(x, 48), e3 = lane_value(x, 63);
    const float gbs = per_block(s0, s1, s2, s3, lane);  // g at the first row of the block
    const float gbe = per_block(e0, e1, e2, e3, lane);  // g at the last row of the block
    sm.beta[slot][lane] = ok ? beta : 0.f;
    sm.g[slot][lane] = x;
    sm.gam[slot][lane] = __expf(x);
    sm.w[slot][lane] = __expf(e3 - x);
    sm.ea[slot][lane] = __expf(x - gbs);
    sm.eb[slot][lane] = __expf(gbe - x);
    // lane t < 6: off-diagonal tile t = i(i-1)/2 + k of the Gram list, (i,k) = (1,0) (2,0)
    // (2,1) (3,0) (3,1) (3,2): e^{g_{16i} - g_{16k+15}}
    const int t = lane & 7;
    const float gi = t >= 3 ? s3 : (t >= 1 ? s2 : s1);
    const float gk = (t == 0 || t == 1 || t == 3) ? e0 : ((t == 2 || t == 4) ? e1 : e2);
    if (lane < 6) sm.cik[slot][lane] = __expf(gi - gk);
}

// D_kb = (I + N)^{-1} of diagonal block kb from N in the A layout (lane holds N[lr][4lq+e]);
// the B layout (lane holds N[4lq+e][lr]) comes back through LDS with a transposing read
template <int DK>
__device__ __forceinline__ void diag_inverse(Lds<DK> &sm, int b, int kb, int lr, int lq,
                                             v4f Na_f) {
    using L = Lds<DK>;
    const uint2 na = pack4u(Na_f);
    *reinterpret_cast<uint2 *>(&sm.ntile[kb][lr * 16 + 4 * lq]) = na;
    const v4s Na = __builtin_bit_cast(v4s, na);
    const v4s Nb = ld_tr(&sm.ntile[kb][(4 * lq + (lr >> 2)) * 16 + 4 * (lr & 3)]);
    // squares in both layouts: X^2 (C = B layout) = X X;  (X^2)^T (C = A layout) = X^T X^T
    const v4f N2 = mfma16(Na, Nb, zero4());
    const v4f N2t = mfma16(Nb, Na, zero4());
    const v4s N2a = pack4(N2t), N2b = pack4(N2);
    const v4f N4 = mfma16(N2a, N2b, zero4());
    const v4f N4t = mfma16(N2b, N2a, zero4());
    const v4s N4a = pack4(N4t), N4b = pack4(N4);
    // D^T = (I - N^T)(I + N^2T)(I + N^4T)(I + N^8T), built in C layout = A layout of D;
    // the A operand N^T (A layout) is N in the B layout
    v4f Y = mfma16(N4b, N4a, zero4());  // (N^8)^T
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (4 * lq + e == lr) Y[e] += 1.f;
    Y = mfma16(N4b, pack4(Y), Y);
    Y = mfma16(N2b, pack4(Y), Y);
    const uint2 nb = __builtin_bit_cast(uint2, Nb);
    const v4s mNb = __builtin_bit_cast(v4s, make_uint2(nb.x ^ 0x80008000u, nb.y ^ 0x80008000u));
    Y = mfma16(mNb, pack4(Y), Y);
    *reinterpret_cast<uint2 *>(&sm.dinv[b][kb * 16 * L::DP + lr * L::DP + 4 * lq]) = pack4u(Y);
}

template <int DK, typename TD>
__global__ void __launch_bounds__(NW * 64)
chunk_mfma_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const uint16_t *__restrict__ v, const TD *__restrict__ d,
                  const float *__restrict__ beta, const float *__restrict__ alpha,
                  const float *S0, uint16_t *__restrict__ o, float *S_T, int64_t BH,
                  int64_t T, int dv) {
    using L = Lds<DK>;
    constexpr int NS = DK / 32;   // 32-wide k-steps over the key features
    constexpr int NFT = DK / 16;  // 16-row feature tiles of the state

    __shared__ L sm;
    // q and k buffers: one __shared__ variable each (see the file comment)
    __shared__ alignas(16) uint16_t q_buf0[CH * DK], q_buf1[CH * DK];
    __shared__ alignas(16) uint16_t k_buf0[CH * DK], k_buf1[CH * DK];
    __shared__ alignas(16) uint16_t v_buf0[BV * CH], v_buf1[BV * CH];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15;  // row (A) / column (B, C) index inside a 16-tile
    const int lq = lane >> 4;  // quarter: k-offset (A, B) / row group (C)
    const bool state_wave = wave < 2;
    const int ct = wave & 1;   // value tile of a state wave

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
    const int64_t nchunks = (T + CH - 1) / CH;
    auto rows_of = [&](int64_t cc) __attribute__((always_inline)) {
        return static_cast<int>(T - cc * CH < CH ? T - cc * CH : CH);
    };

    // score tiles above the diagonal are read as zeros by the read-out and never written
    for (int i = tid; i < 2 * CH * L::CP; i += NW * 64) (&sm.p[0][0])[i] = 0;

    // The two roles run separate loops with the same barriers: two in the prologue (chunk 0
    // loaded; chunk 0 scanned), then one per step c = -1 .. nchunks-1, where step -1 prepares
    // chunk 0 and forms K M, M^T Q^T of chunk 0.
    if (state_wave) {
        // ---- state slice: C layout of 16x16 tiles, feature tile ft ----------------------------
        v4f M[NFT], KM[NBLK], Z[NBLK];
        v4s VT[NBLK];  // v tile of the next chunk (C layout of this wave's 16 columns)
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ft + 4 * lq + i, col = j0 + VW * ct + lr;
                M[ft][i] = S0 ? S0[(bh * DK + row) * dv + col] : 0.f;
            }
        if (nchunks > 0) block_sync();

        // K M and M^T Q^T of the next chunk from the current state, and its v tile, from the
        // q/k/v buffers qn/kn/vn
        auto products = [&](const uint16_t *qn, const uint16_t *kn, const uint16_t *vn)
            __attribute__((always_inline)) {
#pragma unroll
            for (int rt = 0; rt < NBLK; ++rt)  // transposing read: V[16rt + 4lq + e][lr]
                VT[rt] = ld_tr(&vn[ct * CH * VW + (16 * rt + 4 * lq + (lr >> 2)) * VW + 4 * (lr & 3)]);
            v8s mb[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) mb[s] = c_to_frag(M[2 * s], M[2 * s + 1]);
#pragma unroll
            for (int rt = 0; rt < NBLK; ++rt) {
                v8s kf[NS], qf[NS];
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    kf[s] = ld8(&kn[L::qk_at(16 * rt + lr, 4 * s + lq)]);
                    qf[s] = ld8(&qn[L::qk_at(16 * rt + lr, 4 * s + lq)]);
                }
                v4f a = zero4(), z = zero4();
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    a = mfma32(kf[s], mb[s], a);  // K M: rows 16rt+4lq+e, column lr
                    z = mfma32(mb[s], qf[s], z);  // M^T Q^T: value column 4lq+e, row 16rt+lr
                }
                KM[rt] = a;
                Z[rt] = z;
            }
        };

        int sl = 2;  // c mod 3
        for (int64_t c = -1; c < nchunks; ++c) {
            if (c >= 0) {
                // ---- chunk c: R, U, read-out, carry --------------------------------------------
                const int b = static_cast<int>(c & 1);
                const int n = rows_of(c);
                const int64_t row0 = seq0 + c * CH;
                // R = beta (V - gam (K M)), then U by block forward substitution
                v4s dA[NBLK], aN[NOFF];
#pragma unroll
                for (int rt = 0; rt < NBLK; ++rt)
                    dA[rt] = ld4s(&sm.dinv[b][rt * 16 * L::DP + lr * L::DP + 4 * lq]);
#pragma unroll
                for (int u = 0; u < NOFF; ++u)
                    aN[u] = ld4s(&sm.aneg[b][u * 16 * L::DP + lr * L::DP + 4 * lq]);
                v4f U[NBLK];
#pragma unroll
                for (int i = 0; i < NBLK; ++i) {
                    const v4f bt4 = ld4(&sm.beta[sl][16 * i + 4 * lq]);
                    const v4f gm4 = ld4(&sm.gam[sl][16 * i + 4 * lq]);
                    v4f Y;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Y[e] = bt4[e] * (__uint_as_float(static_cast<uint32_t>(
                                             static_cast<uint16_t>(VT[i][e])) << 16) -
                                         gm4[e] * KM[i][e]);
#pragma unroll
                    for (int kb = 0; kb < i; ++kb)
                        Y = mfma16(aN[(i * (i - 1)) / 2 + kb], pack4(U[kb]), Y);
                    U[i] = mfma16(dA[i], pack4(Y), zero4());
                }
                // U and w U as fragments over the chunk rows
                v8s ub[2], uwb[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const v4f w0 = ld4(&sm.w[sl][32 * s + 4 * lq]);
                    const v4f w1 = ld4(&sm.w[sl][32 * s + 16 + 4 * lq]);
                    ub[s] = c_to_frag(U[2 * s], U[2 * s + 1]);
                    uwb[s] = c_to_frag(w0 * U[2 * s], w1 * U[2 * s + 1]);
                }
                // read-out O^T = (M^T Q^T) diag(gam) + U^T P^T: lane holds O[16rt+lr][4 columns]
#pragma unroll
                for (int rt = 0; rt < NBLK; ++rt) {
                    const int r = 16 * rt + lr;
                    v4f acc = sm.gam[sl][r] * Z[rt];
#pragma unroll
                    for (int s = 0; s <= rt / 2; ++s)
                        acc = mfma32(ub[s], ld8(&sm.p[b][r * L::CP + 32 * s + 8 * lq]), acc);
                    if (r < n)
                        *reinterpret_cast<uint2 *>(o + (row0 + r) * dv + j0 + VW * ct + 4 * lq) =
                            pack4u(acc);
                }
                // carry: M <- gam_C M + K~^T (w U); A = K~^T by transposing reads of row-major K~
                const float gC = sm.gam[sl][CH - 1];
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) {
                    v4f acc = gC * M[ft];
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const uint16_t *base =
                            &sm.kt[b][(32 * s + 8 * lq + (lr >> 2)) * L::KP + 16 * ft + 4 * (lr & 3)];
                        acc = mfma32(cat8(ld_tr(base), ld_tr(base + 4 * L::KP)), uwb[s], acc);
                    }
                    M[ft] = acc;
                }
            }
            // K M, M^T Q^T and v of chunk c+1 (a branch per buffer parity)
            if (c + 1 < nchunks) {
                if ((c + 1) & 1) products(q_buf1, k_buf1, v_buf1);
                else products(q_buf0, k_buf0, v_buf0);
            }
            wait_global();
            block_sync();
            sl = sl == 2 ? 0 : sl + 1;
        }

        if (S_T) {
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * ft + 4 * lq + i, col = j0 + VW * ct + lr;
                    S_T[(bh * DK + row) * dv + col] = M[ft][i];
                }
        }
        return;
    }

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // ---- loader wave: q, k, v of chunk c+2 into LDS, and the decay scan of chunk c+2 --------
    // Issuing the loads stalls while HBM drains them, so a wave with little other work issues
    // them; the parity of the target buffers is a compile-time constant.
    if (wave == 4) {
        auto load_chunk = [&](auto par_c, int64_t cc, int slot) __attribute__((always_inline)) {
            constexpr int PAR = decltype(par_c)::value;
            if (cc >= nchunks) return;
            const int64_t r0 = seq0 + cc * CH;
            const int n = rows_of(cc);
            load_qk<DK>(PAR ? q_buf1 : q_buf0, PAR ? k_buf1 : k_buf0, q, k, r0, n, lane);
            load_v(PAR ? v_buf1 : v_buf0, v, r0, n, dv, j0, lane);
            const int r = min(lane, n - 1);
            const float bv = beta[r0 + r];
            const float av = has_alpha ? alpha[r0 + r] : 1.f;
            scan_chunk<DK>(sm, slot, bv, av, n, has_alpha, lane);  // slot = cc mod 3
        };
        if (nchunks > 0) {
            load_chunk(I0{}, 0, 0);
            wait_global();
            block_sync();
        }
        load_chunk(I1{}, 1, 1);  // step -1
        wait_global();
        block_sync();
        int sl = 2;  // (c+2) mod 3
        for (int64_t c = 0; c < nchunks; c += 2) {
            load_chunk(I0{}, c + 2, sl);
            wait_global();
            block_sync();
            sl = sl == 2 ? 0 : sl + 1;
            if (c + 1 < nchunks) {
                load_chunk(I1{}, c + 3, sl);
                wait_global();
                block_sync();
                sl = sl == 2 ? 0 : sl + 1;
            }
        }
        return;
    }

    // ---- prep waves ----------------------------------------------------------------------------
    const int pw = wave - 2;
    PrepRegs<DK, TD> pr;  // d of chunk c+1 at the start of step c

    // Prep wave PW in step c: k~, Gram/score tiles and block inverses of chunk c+1; d of chunk
    // c+2 into registers (clamped to the last chunk); s1 = (c+1) mod 3
    auto prep_step = [&](auto pw_c, int64_t c, int s1) __attribute__((always_inline)) {
        constexpr int PW = decltype(pw_c)::value;
        const int64_t c1 = c + 1, c2 = c + 2;
        if (c1 >= nchunks) return;
        const int b1 = static_cast<int>(c1 & 1);
        const uint16_t *qx = b1 ? q_buf1 : q_buf0;
        const uint16_t *kx = b1 ? k_buf1 : k_buf0;
        // k~ of the own blocks: fragments in registers, rows into LDS for the carry (all reads
        // first: the compiler cannot reorder the k reads across the k~ writes)
        v8s kt[2][NS];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int s = 0; s < NS; ++s) kt[j][s] = ld8(&kx[L::qk_at(16 * kblk(PW, j) + lr, 4 * s + lq)]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kb = kblk(PW, j);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint4 xu = __builtin_bit_cast(uint4, kt[j][s]);
                float dd[8];
                d_values(pr.d[j][s], dd, TD{});
                const uint32_t xw[4] = {xu.x, xu.y, xu.z, xu.w};
                uint32_t pk[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pk[e] = pack2(dd[2 * e] * bf_lo(xw[e]), dd[2 * e + 1] * bf_hi(xw[e]));
                const uint4 ku = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                kt[j][s] = __builtin_bit_cast(v8s, ku);
                *reinterpret_cast<uint4 *>(&sm.kt[b1][(16 * kb + lr) * L::KP + 32 * s + 8 * lq]) = ku;
            }
        }
        {
            const int64_t cd = c2 < nchunks ? c2 : c1;
            load_d_frag<DK, TD, PW>(pr, d, seq0 + cd * CH, rows_of(cd), lr, lq);
        }
        // tiles (i, kb) = K~_kb X_i^T (X = Q: scores, X = K: Gram), row block by row block;
        // the lane holds row 16i+lr, columns 16kb+4lq..+3
        constexpr int IMIN = kblk(PW, 0) < kblk(PW, 1) ? kblk(PW, 0) : kblk(PW, 1);
        // the fragments of row block i+1 are read before block i is processed
        v8s kf[NS], qf[NS], kf_n[NS], qf_n[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kf_n[s] = ld8(&kx[L::qk_at(16 * IMIN + lr, 4 * s + lq)]);
            qf_n[s] = ld8(&qx[L::qk_at(16 * IMIN + lr, 4 * s + lq)]);
        }
#pragma unroll
        for (int i = IMIN; i < NBLK; ++i) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                kf[s] = kf_n[s];
                qf[s] = qf_n[s];
            }
            if (i + 1 < NBLK) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    kf_n[s] = ld8(&kx[L::qk_at(16 * (i + 1) + lr, 4 * s + lq)]);
                    qf_n[s] = ld8(&qx[L::qk_at(16 * (i + 1) + lr, 4 * s + lq)]);
                }
            }
            const int r = 16 * i + lr;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kb = kblk(PW, j);
                if (kb > i) continue;
                v4f sc = zero4();
#pragma unroll
                for (int s = 0; s < NS; ++s) sc = mfma32(kt[j][s], qf[s], sc);
                if (i > kb) {
                    // off-diagonal: e^{g_r - g_s} = ea[r] cik eb[s], each factor <= 1
                    const int t = (i * (i - 1)) / 2 + kb;
                    const float rowf = sm.ea[s1][r] * sm.cik[s1][t];
                    const v4f eb4 = ld4(&sm.eb[s1][16 * kb + 4 * lq]);
                    v4f gm = zero4();
#pragma unroll
                    for (int s = 0; s < NS; ++s) gm = mfma32(kt[j][s], kf[s], gm);
                    const float growf = -sm.beta[s1][r] * rowf;
                    v4f pv, av;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pv[e] = (sc[e] * rowf) * eb4[e];
                        av[e] = (gm[e] * growf) * eb4[e];
                    }
                    *reinterpret_cast<uint2 *>(&sm.p[b1][r * L::CP + 16 * kb + 4 * lq]) = pack4u(pv);
                    *reinterpret_cast<uint2 *>(&sm.aneg[b1][t * 16 * L::DP + lr * L::DP + 4 * lq]) =
                        pack4u(av);
                } else {
                    // diagonal block: exact e^{g_r - g_s} (r = 16kb+lr, s = 16kb+4lq+e), shared
                    // by the score tile (s <= r) and N (s < r)
                    const float gr = sm.g[s1][r], bt = sm.beta[s1][r];
                    const v4f gs = ld4(&sm.g[s1][16 * kb + 4 * lq]);
                    v4f Gdt = zero4();  // G in the A layout: lane holds G[r][s]
#pragma unroll
                    for (int s = 0; s < NS; ++s) Gdt = mfma32(kt[j][s], kf[s], Gdt);
                    v4f pv, na;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ex = __expf(gr - gs[e]);
                        pv[e] = (4 * lq + e <= lr) ? ex * sc[e] : 0.f;
                        na[e] = (4 * lq + e < lr) ? (bt * ex) * Gdt[e] : 0.f;
                    }
                    *reinterpret_cast<uint2 *>(&sm.p[b1][r * L::CP + 16 * kb + 4 * lq]) = pack4u(pv);
                    diag_inverse<DK>(sm, b1, kb, lr, lq, na);
                }
            }
        }
    };

    if (nchunks > 0) {
        // prologue: d of chunk 0
        if (pw == 0) load_d_frag<DK, TD, 0>(pr, d, seq0, rows_of(0), lr, lq);
        else load_d_frag<DK, TD, 1>(pr, d, seq0, rows_of(0), lr, lq);
        wait_global();
        block_sync();
    }
    // one loop per prep wave, so its registers need no merging between the two variants
    auto prep_loop = [&](auto pw_c) __attribute__((always_inline)) {
        int sl1 = 0;  // (c+1) mod 3
        for (int64_t c = -1; c < nchunks; ++c) {
            const int sl2 = sl1 == 2 ? 0 : sl1 + 1;
            prep_step(pw_c, c, sl1);
            wait_global();
            block_sync();
            sl1 = sl2;
        }
    };
    if (pw == 0) prep_loop(I0{});
    else prep_loop(I1{});
}

template <int DK, typename TD>
hipError_t launch_typed(const ChunkArgs &a, hipStream_t stream) {
    const int nvt = a.dv / BV;
    const dim3 grid(static_cast<unsigned>(a.BH * nvt));
    hipLaunchKernelGGL((chunk_mfma_kernel<DK, TD>), grid, dim3(NW * 64), 0, stream,
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
