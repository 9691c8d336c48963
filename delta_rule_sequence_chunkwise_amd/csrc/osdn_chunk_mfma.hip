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
// One workgroup owns one (b,h) sequence and a slice of the value columns (value columns are
// independent given the chunk's A and P) and walks the chunks in order, one barrier per step.
// The slice is 32 columns wide (seven waves, numbered as below), or 16 (six waves: one state
// wave, the other roles numbered one lower) when the grid of 16-column slices still fits the
// device with one workgroup per compute unit (long sequences, few heads).  Each role runs its
// own loop over steps c = -2 .. nchunks-1:
//
// * State waves (0, 1), one per 16 value columns, process chunk c.  A state wave holds its
//   dk x 16 slice of M in VGPRs (fp32, the C layout of 16x16 MFMA tiles) for the whole
//   sequence and runs the state-dependent chain without touching LDS for M or U: R, the block
//   forward substitution U_i = D_i (R_i - sum_{k<i} A_ik U_k) (16x16x16 products; their output
//   layout equals their B-operand layout), the read-out O^T = (M^T Q^T) diag(gam) + U^T P^T,
//   the carry M <- gam_C M + K~^T (w U), and then K M and M^T Q^T of chunk c+1.
//   A pair of 16x16 C-layout tiles becomes one 16x16x32 operand fragment with two packs and
//   four lane swaps (v_permlane32_swap, v_permlane16_swap): lane (quarter q, column n) then
//   holds rows 8q..8q+7 of the 32-row pair, which is both the B layout of the pair and the
//   A layout of its transpose.  So every K-slot runs in natural order and each q, k and P
//   operand fragment is a single 16-byte LDS read.
// * Prep waves (2, 3) build chunk c+1's Gram and score tiles and the inverses
//   D_i = (I + A_ii)^{-1} of its diagonal blocks, computed in registers as
//   (I-N)(I+N^2)(I+N^4)(I+N^8) (N strictly lower, N^16 = 0), two blocks in lockstep.  The
//   tiles are split by column block: wave 2 takes blocks {0,3}, wave 3 blocks {1,2}.
// * Stager waves (4, 5) bring the k rows of chunk c+2 into LDS (two row blocks each) and write
//   k~ = d (.) k of those rows; d reaches their registers one step ahead.
// * The loader wave (6) brings q and v of chunk c+2, and beta and alpha of chunk c+3, into
//   LDS.  Prep wave 2 runs chunk c+2's decay scan after its tiles from those LDS copies: a
//   global load of its own would return only after the step's bulk loads ahead of it.
// With the channel-wise gate (GATE) the caller passes the gate-scaled q o G, k o G and
// k~ o (G_C / G), each chunk's product of gates G_C and its planes (P, the diagonal-block
// inverses, -A_ik) from the planes kernel: the stagers copy k~ in instead of forming it, prep
// wave 3 copies the planes in instead of forming them, and the carry scales the state's rows
// by G_C; the loader brings G_C into LDS with the other loads of its chunk.  For the backward a variant records the state
// at every chunk start (CKPT), with or without writing o (OUT).
// Loads stall the issuing wave while HBM drains them, and too many in flight at once thrash
// the CU's load queues; so they are issued in groups of at most 16 by waves whose other work
// is light, and each state wave shares its SIMD with a stager.
//
// q, k and v reach LDS by global_load_lds (16 bytes per lane; the 16-byte units of each q/k
// row are XOR-swizzled by the row index so fragment reads are bank-conflict free), double-
// buffered by chunk parity; the state waves read the v tile of chunk c+1 into registers at
// the end of step c.  P and the block inverses are double-buffered by chunk parity; k~ and
// the scan outputs, written two steps before their last use, by chunk mod 3.  Waves whose
// loads target LDS drain them before the end-of-step barrier.
#include <type_traits>

#include "osdn_internal.h"
#include "osdn_mfma.h"

namespace osdn {
namespace {

constexpr int CH = 64;                       // rows per chunk
constexpr int NBLK = CH / 16;                // 16-row blocks per chunk
constexpr int NOFF = NBLK * (NBLK - 1) / 2;  // off-diagonal 16x16 blocks of the Gram matrix
constexpr int VW = 16;                       // value columns per state wave
// A workgroup runs NSW state waves (one per 16 value columns of its slice), then 2 prep waves,
// 2 stagers and 1 loader: NSW + 5 waves, a slice of 16 NSW value columns.
__host__ __device__ constexpr int n_waves(int nsw) { return nsw + 5; }

template <int DK, bool GATE = false>
struct alignas(16) Lds {
    static constexpr int KU = DK / 8;   // 16-byte units per q/k/k~ row
    static constexpr int KP = DK;       // row pitch (bf16) of k~
    static constexpr int CP = CH + 8;   // row pitch (bf16) of P
    static constexpr int DP = 16;       // row pitch (bf16) of 16x16 blocks
    // Swizzles, so that the access patterns below touch each of the 64 four-byte LDS banks at
    // most once per cycle (16 lanes of a 16-byte access, 32 lanes of an 8-byte access):
    // * q/k tiles: 16-byte unit u of row r sits at unit u ^ fqk(r); fragment reads take one
    //   unit from each of 16 consecutive rows.
    __device__ static constexpr int fqk(int r) { return DK == 128 ? (r & 15) : ((r >> 1) & 7); }
    __device__ static constexpr int qk_at(int r, int u) { return (r * KU + (u ^ fqk(r))) * 8; }
    // * k~: 8-byte granule g of row r sits at granule g ^ 2 pk(r).  The tile is read three
    //   ways: 16-byte units of 16 consecutive rows (prep waves), written the same way
    //   (stagers), and read by transposing reads of four granules of rows k0..k0+3 and
    //   k0+8..k0+11 (state waves).  Measured on gfx950: a 16-byte read is served 16 lanes at a
    //   time from the 64 banks, lanes grouped by half-wave and by the parity of lane bits 2..4;
    //   a 16-byte write 8 lanes at a time from 32 banks; a transposing read 32 lanes at a time
    //   from 64.  pk (a linear map of the row's low four bits) keeps the writes and the
    //   transposing reads conflict-free.  With dk = 64 the prep reads are conflict-free too;
    //   with dk = 128 the map that also achieves that measured slower, so each of those reads
    //   takes two extra cycles.
    __device__ static constexpr int pk(int r) {
        const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
        return DK == 128 ? (b2 | (b0 << 1) | (b1 << 2) | (b3 << 3))
                         : (b2 | ((b0 ^ b2 ^ b3) << 1) | (b1 << 2));
    }
    __device__ static constexpr int kt_gr(int r, int g) { return r * KP + 4 * (g ^ (2 * pk(r))); }
    __device__ static constexpr int kt_at(int r, int u) { return kt_gr(r, 2 * u); }
    // * 16x16 blocks (pitch 16): granule g of row r at g ^ 2 ((r >> 3) & 1)
    __device__ static constexpr int blk(int r, int g) { return r * DP + 4 * (g ^ (((r >> 3) & 1) << 1)); }
    alignas(16) uint16_t kt[3][CH * KP];            // [chunk mod 3] k~, rows swizzled by kt_gr
    alignas(16) uint16_t p[2][CH * CP];             // [chunk parity] P, row-major
    alignas(16) uint16_t dinv[2][NBLK * 16 * DP];   // D_i = (I + A_ii)^{-1}, rows by blk
    alignas(16) uint16_t aneg[2][NOFF * 16 * DP];   // -A_ik (i > k), rows by blk
    alignas(16) float beta[3][CH];                  // [chunk mod 3] scan outputs
    alignas(16) float g[3][CH];
    alignas(16) float gam[3][CH];
    alignas(16) float w[3][CH];
    // decay factors of off-diagonal 16x16 tiles (i > k), all <= 1:
    // e^{g_r - g_s} = ea[r] * cik[t(i,k)] * eb[s] with ea[r] = e^{g_r - g_{16i}},
    // cik = e^{g_{16i} - g_{16k+15}}, eb[s] = e^{g_{16k+15} - g_s}
    alignas(16) float ea[3][CH];
    alignas(16) float eb[3][CH];
    alignas(16) float gc[GATE ? 3 : 1][GATE ? DK : 4];  // channel-wise gate: G_C of the chunk
    alignas(16) float cik[3][8];
    alignas(16) float rawb[2][CH];  // [chunk parity] beta and alpha as loaded, for the scan
    alignas(16) float rawa[2][CH];
    alignas(16) uint16_t ntile[NBLK][16 * 16];  // N of diagonal block kb, rows by blk (prep)
};

static_assert(Lds<128>::CP == kda_planes::kPPitch && Lds<64>::CP == kda_planes::kPPitch,
              "P pitch shared with the channel-gate planes");
static_assert(sizeof(Lds<128>::dinv[0]) == 2 * kda_planes::kDinv &&
              sizeof(Lds<128>::aneg[0]) == 2 * kda_planes::kAneg &&
              sizeof(Lds<128>::p[0]) == 2 * kda_planes::kP, "plane sizes");
static_assert(Lds<128>::blk(9, 1) == kda_planes::blk(9, 1) && Lds<64>::blk(3, 2) == kda_planes::blk(3, 2),
              "block layout shared with the channel-gate planes");

// Prep wave pw owns the Gram/score column blocks kblk(pw, 0), kblk(pw, 1)
__host__ __device__ constexpr int kblk(int pw, int j) { return pw == 0 ? (j == 0 ? 0 : 3) : (j == 0 ? 1 : 2); }

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

// rows [R0, R0 + NR) of one q or k chunk tile into LDS, 16-byte units XOR-swizzled by the
// row (one wave; rows past the end of the sequence re-read its last row); at most 16 loads of
// the wave in flight
template <int DK, int R0, int NR>
__device__ __forceinline__ void load_rows(uint16_t *dst, const uint16_t *src, int64_t row0, int n,
                                          int lane) {
    using L = Lds<DK>;
    constexpr int NLOAD = NR * L::KU / 64;
    static_assert(NR * L::KU % 64 == 0, "whole wave-loads");
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
        const int base = R0 * L::KU + i * 64;  // physical unit of lane 0
        const int pu = base + lane, r = pu / L::KU, lu = (pu % L::KU) ^ L::fqk(r);
        load_to_lds16(src + (row0 + min(r, n - 1)) * DK + 8 * lu, dst + 8 * base);
        if (i % 8 == 7 && i + 1 < NLOAD) wait_global8();
    }
}

// rows [R0, R0 + NR) of a row-major bf16 k~ tile into the k~ buffer (16-byte units swizzled by
// pk(r), the layout the stagers otherwise write): channel-wise gate, where k~ arrives pre-scaled
template <int DK, int R0, int NR>
__device__ __forceinline__ void load_kt_rows(uint16_t *dst, const uint16_t *src, int64_t row0, int n,
                                             int lane) {
    using L = Lds<DK>;
    constexpr int NLOAD = NR * L::KU / 64;
    static_assert(NR * L::KU % 64 == 0, "whole wave-loads");
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
        const int base = R0 * L::KU + i * 64;
        const int pu = base + lane, r = pu / L::KU, lu = (pu % L::KU) ^ L::pk(r);
        load_to_lds16(src + (row0 + min(r, n - 1)) * DK + 8 * lu, dst + 8 * base);
        if (i % 8 == 7 && i + 1 < NLOAD) wait_global8();
    }
}

// n16 16-byte units of a contiguous image into LDS (one wave, at most 16 loads in flight)
template <int N16>
__device__ __forceinline__ void copy_image(uint16_t *dst, const uint16_t *src, int lane) {
    constexpr int NLOAD = (N16 + 63) / 64;
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
        if (N16 % 64 == 0 || i + 1 < NLOAD || lane < N16 % 64)
            load_to_lds16(src + 8 * (64 * i + lane), dst + 8 * 64 * i);
        if (i % 8 == 7 && i + 1 < NLOAD) wait_global8();
    }
}

// the workgroup's 64 x 16 NSW slice of v into LDS as [value tile][row][16] (loader wave)
template <int NSW>
__device__ __forceinline__ void load_v(uint16_t *vb, const uint16_t *v, int64_t row0, int n,
                                       int dv, int j0, int lane) {
#pragma unroll
    for (int ii = 0; ii < 2 * NSW; ++ii) {
        const int vt = ii >> 1, h = ii & 1;
        const int r = 32 * h + (lane >> 1);
        load_to_lds16(v + (row0 + min(r, n - 1)) * dv + j0 + VW * vt + 8 * (lane & 1),
                      vb + (vt * CH + 32 * h) * VW);
    }
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
template <int DK, bool G>
__device__ __forceinline__ void scan_chunk(Lds<DK, G> &sm, int slot, float beta, float alpha, int n,
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

// D_kb = (I + N)^{-1} for the two diagonal blocks kb0, kb1 of a prep wave, in lockstep so the
// two dependent chains overlap.  Input: N in the A layout (lane holds N[lr][4lq+e]); the B
// layout (lane holds N[4lq+e][lr]) comes back through LDS with a transposing read.
template <int DK, bool G>
__device__ __forceinline__ void diag_inverse2(Lds<DK, G> &sm, int b, int kb0, int kb1, int lr,
                                              int lq, const v4f (&na)[2]) {
    using L = Lds<DK>;
    const int kb[2] = {kb0, kb1};
    v4s Na[2], Nb[2], N2a[2], N2b[2], N4a[2], N4b[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint2 u = pack4u(na[j]);
        *reinterpret_cast<uint2 *>(&sm.ntile[kb[j]][L::blk(lr, lq)]) = u;
        Na[j] = __builtin_bit_cast(v4s, u);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
        Nb[j] = ld_tr(&sm.ntile[kb[j]][L::blk(4 * lq + (lr >> 2), lr & 3)]);
    // squares in both layouts: X^2 (C = B layout) = X X;  (X^2)^T (C = A layout) = X^T X^T
    v4f X[2], Xt[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        X[j] = mfma16(Na[j], Nb[j], zero4());
        Xt[j] = mfma16(Nb[j], Na[j], zero4());
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        N2a[j] = pack4(Xt[j]);
        N2b[j] = pack4(X[j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        X[j] = mfma16(N2a[j], N2b[j], zero4());
        Xt[j] = mfma16(N2b[j], N2a[j], zero4());
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        N4a[j] = pack4(Xt[j]);
        N4b[j] = pack4(X[j]);
    }
    // D^T = (I - N^T)(I + N^2T)(I + N^4T)(I + N^8T), built in C layout = A layout of D;
    // the A operand N^T (A layout) is N in the B layout
    v4f Y[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) Y[j] = mfma16(N4b[j], N4a[j], zero4());  // (N^8)^T
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * lq + e == lr) Y[j][e] += 1.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) Y[j] = mfma16(N4b[j], pack4(Y[j]), Y[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) Y[j] = mfma16(N2b[j], pack4(Y[j]), Y[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint2 nb = __builtin_bit_cast(uint2, Nb[j]);
        const v4s mNb = __builtin_bit_cast(v4s, make_uint2(nb.x ^ 0x80008000u, nb.y ^ 0x80008000u));
        Y[j] = mfma16(mNb, pack4(Y[j]), Y[j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
        *reinterpret_cast<uint2 *>(&sm.dinv[b][kb[j] * 16 * L::DP + L::blk(lr, lq)]) =
            pack4u(Y[j]);
}

template <int DK, typename TD, bool GATE, bool CKPT, bool OUT, int NSW>
__global__ void __launch_bounds__(n_waves(NSW) * 64)
chunk_mfma_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const uint16_t *__restrict__ v, const TD *__restrict__ d,
                  const float *__restrict__ beta, const float *__restrict__ alpha,
                  const float *S0, uint16_t *__restrict__ o, float *S_T, int64_t BH,
                  int64_t T, int dv, const float *__restrict__ gcs, uint16_t *__restrict__ ckpt,
                  uint16_t *__restrict__ uout, const uint16_t *__restrict__ planes) {
    using L = Lds<DK, GATE>;
    constexpr int NS = DK / 32;   // 32-wide k-steps over the key features
    constexpr int NFT = DK / 16;  // 16-row feature tiles of the state
    constexpr int NW = n_waves(NSW);
    constexpr int BV = VW * NSW;  // value columns of the workgroup's slice
    // roles by wave: state waves first, then the prep waves, the stagers and the loader
    constexpr int W_PREP = NSW, W_STAGE = NSW + 2, W_LOAD = NSW + 4;

    __shared__ L sm;
    // q, k and v tiles by chunk parity: one __shared__ variable each, indexed by the parity,
    // so the compiler can tell reads of them from the writes into sm
    __shared__ alignas(16) uint16_t q_buf[2][CH * DK], k_buf[2][CH * DK];
    __shared__ alignas(16) uint16_t v_buf[2][BV * CH];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15;  // row (A) / column (B, C) index inside a 16-tile
    const int lq = lane >> 4;  // quarter: k-offset (A, B) / row group (C)

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
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // beta and alpha of chunk c reach LDS by DMA (loader wave, step c-3), so the scanning wave
    // issues no global load: behind the bulk loads of the step it would wait a memory round trip
    auto load_ba = [&](int64_t cc, int par) __attribute__((always_inline)) {
        const int64_t r = seq0 + cc * CH + min(lane, rows_of(cc) - 1);
        load_to_lds4(beta + r, &sm.rawb[par][0]);
        if (has_alpha) load_to_lds4(alpha + r, &sm.rawa[par][0]);
    };
    if (wave == W_LOAD && nchunks > 0) {
        load_ba(0, 0);
        wait_global();
    }
    // score tiles above the diagonal are read as zeros by the read-out and never written
    for (int i = tid; i < 2 * CH * L::CP; i += NW * 64) (&sm.p[0][0])[i] = 0;
    block_sync();

    // Every role runs steps c = -2 .. nchunks-1 with one barrier each.  In step c the state
    // waves process chunk c and form K M, M^T Q^T of chunk c+1; the prep waves build the
    // Gram/score tiles and block inverses of chunk c+1; the loader brings q, k, v of chunk
    // c+2 into LDS and scans it; the stager writes k~ of chunk c+2.

    if (wave < NSW) {
        // ---- state waves -----------------------------------------------------------------------
        const int ct = wave;  // value tile
        v4f M[NFT], KM[NBLK], Z[NBLK];
        v4s VT[NBLK];  // v tile of the next chunk (C layout of this wave's 16 columns)
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ft + 4 * lq + i, col = j0 + VW * ct + lr;
                M[ft][i] = S0 ? S0[(bh * DK + row) * dv + col] : 0.f;
            }

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

        int sl = 1;  // c mod 3
        for (int64_t c = -2; c < nchunks; ++c) {
            if (c >= 0) {
                // ---- chunk c: R, U, read-out, carry --------------------------------------------
                if constexpr (CKPT) {  // the state at this chunk's start in bf16, for the backward
                                       // (tiled by ckpt_at): row 16 ft + 4 lq + lr % 4, columns
                                       // 4 (lr / 4) .. +3 of the wave's 16 after a quad transpose
                    uint16_t *dst = ckpt + (bh * nchunks + c) * DK * dv +
                                    ckpt_at(4 * lq + (lr & 3), j0 + VW * ct + 4 * (lr >> 2), DK);
#pragma unroll
                    for (int ft = 0; ft < NFT; ++ft)  // rows 16 ft .. of the tile
                        *reinterpret_cast<uint2 *>(dst + 16 * 16 * ft) = pack4u(quad_transpose(M[ft], lane));
                }
                const int b = static_cast<int>(c & 1);
                const int n = rows_of(c);
                const int64_t row0 = seq0 + c * CH;
                // operands that do not depend on the chain, read first
                v4s dA[NBLK], aN[NOFF];
                v4f bt4[NBLK], gm4[NBLK], w4[NBLK];
                float gtok[NBLK];
#pragma unroll
                for (int rt = 0; rt < NBLK; ++rt) {
                    dA[rt] = ld4s(&sm.dinv[b][rt * 16 * L::DP + L::blk(lr, lq)]);
                    bt4[rt] = ld4(&sm.beta[sl][16 * rt + 4 * lq]);
                    gm4[rt] = ld4(&sm.gam[sl][16 * rt + 4 * lq]);
                    w4[rt] = ld4(&sm.w[sl][16 * rt + 4 * lq]);
                    gtok[rt] = sm.gam[sl][16 * rt + lr];
                }
#pragma unroll
                for (int u = 0; u < NOFF; ++u)
                    aN[u] = ld4s(&sm.aneg[b][u * 16 * L::DP + L::blk(lr, lq)]);
                const float gC = sm.gam[sl][CH - 1];
                // P^T fragments (B operand of the read-out): rows 16rt+lr, chunk rows 32s+8lq..
                v8s pf[NBLK][2];
#pragma unroll
                for (int rt = 0; rt < NBLK; ++rt)
#pragma unroll
                    for (int s = 0; s <= rt / 2; ++s)
                        pf[rt][s] = ld8(&sm.p[b][(16 * rt + lr) * L::CP + 32 * s + 8 * lq]);
                // K~^T fragments of the carry by transposing reads of row-major K~
                const uint16_t *ktc = sm.kt[sl];
                auto kt_frag = [&](int ft, int s) __attribute__((always_inline)) {
                    const int r = 32 * s + 8 * lq + (lr >> 2), g = 4 * ft + (lr & 3);
                    return cat8(ld_tr(&ktc[L::kt_gr(r, g)]), ld_tr(&ktc[L::kt_gr(r + 4, g)]));
                };
                // R = beta (V - gam (K M)) and U by block forward substitution; after U_0, U_1 the
                // first k-step of the carry and of the read-out can run beside U_2, U_3
                v4f U[NBLK];
                auto solve = [&](int i) __attribute__((always_inline)) {
                    v4f Y;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Y[e] = bt4[i][e] * (__uint_as_float(static_cast<uint32_t>(
                                                static_cast<uint16_t>(VT[i][e])) << 16) -
                                            gm4[i][e] * KM[i][e]);
#pragma unroll
                    for (int kb = 0; kb < i; ++kb)
                        Y = mfma16(aN[(i * (i - 1)) / 2 + kb], pack4(U[kb]), Y);
                    U[i] = mfma16(dA[i], pack4(Y), zero4());
                };
                solve(0);
                solve(1);
                const v8s ub0 = c_to_frag(U[0], U[1]);
                const v8s uwb0 = c_to_frag(w4[0] * U[0], w4[1] * U[1]);
                v4f acc[NFT], oacc[NBLK];
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) {
                    // channel-wise gate: the state's rows times the chunk's G_C (gam = 1 there)
                    const v4f m0 = GATE ? ld4(&sm.gc[sl][16 * ft + 4 * lq]) * M[ft] : gC * M[ft];
                    acc[ft] = mfma32(kt_frag(ft, 0), uwb0, m0);
                }
#pragma unroll
                for (int rt = 0; rt < NBLK; ++rt) oacc[rt] = mfma32(ub0, pf[rt][0], gtok[rt] * Z[rt]);
                solve(2);
                solve(3);
                const v8s ub1 = c_to_frag(U[2], U[3]);
                const v8s uwb1 = c_to_frag(w4[2] * U[2], w4[3] * U[3]);
                if constexpr (CKPT) {  // U for the backward, bf16, in the chunk's block of
                                       // column tiles (rows_at; the last chunk's block is padded
                                       // and its rows past the end are written as computed):
                                       // row 16 i + 4 lq + lr % 4, columns 4 (lr / 4) .. +3 of the
                                       // wave's 16 after a quad transpose
                    if (uout) {
                        uint16_t *ub = uout + (bh * nchunks + c) * CH * dv;
#pragma unroll
                        for (int i = 0; i < NBLK; ++i) {
                            const uint2 pk = pack4u(quad_transpose(U[i], lane));
                            *reinterpret_cast<uint2 *>(
                                ub + rows_at(16 * i + 4 * lq + (lr & 3), j0 + VW * ct + 4 * (lr >> 2))) = pk;
                        }
                    }
                }
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) M[ft] = mfma32(kt_frag(ft, 1), uwb1, acc[ft]);
                // read-out O^T = (M^T Q^T) diag(gam) + U^T P^T: lane holds O[16rt+lr][4 columns];
                // rows past the chunk's last valid row fall outside the buffer range and are
                // dropped by the store
                const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                    o + row0 * dv, 0, n * dv * 2, 0x00020000);
#pragma unroll
                for (int rt = 0; rt < NBLK && OUT; ++rt) {
                    v4f a = oacc[rt];
                    if (rt >= 2) a = mfma32(ub1, pf[rt][1], a);
                    const uint2 pk = pack4u(a);
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2{pk.x, pk.y}, orsrc, ((16 * rt + lr) * dv + j0 + VW * ct + 4 * lq) * 2,
                        0, 0);
                }
            }
            // K M, M^T Q^T and v of chunk c+1
            if (c + 1 >= 0 && c + 1 < nchunks) {
                const int p1 = static_cast<int>((c + 1) & 1);
                products(q_buf[p1], k_buf[p1], v_buf[p1]);
            }
            block_sync();  // the read-out stores need not complete before the barrier
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

    if (wave == W_LOAD) {
        // ---- loader wave: q and v of chunk c+2 into LDS, and the decay scan of chunk c+2 ------
        // Issuing the loads stalls while HBM drains them, so a wave with little other work
        // issues them; the parity of the target buffers is a compile-time constant.
        auto load_step = [&](auto par_c, int64_t cc, int slot) __attribute__((always_inline)) {
            constexpr int PAR = decltype(par_c)::value;  // cc mod 2
            // channel-wise gate: the chunk's G_C, through registers into LDS
            const bool has_gc = GATE && cc >= 0 && cc < nchunks && lane < DK / 4;
            float4 gcv = make_float4(1.f, 1.f, 1.f, 1.f);
            if constexpr (GATE) {
                if (has_gc) gcv = *reinterpret_cast<const float4 *>(gcs + (bh * nchunks + cc) * DK + 4 * lane);
            }
            if (cc >= 0 && cc < nchunks) {
                const int64_t r0 = seq0 + cc * CH;
                const int n = rows_of(cc);
                load_rows<DK, 0, CH>(q_buf[PAR], q, r0, n, lane);
                load_v<NSW>(v_buf[PAR], v, r0, n, dv, j0, lane);
            }
            if (cc + 1 >= 0 && cc + 1 < nchunks) load_ba(cc + 1, PAR ^ 1);
            wait_global();
            if constexpr (GATE) {
                if (has_gc) *reinterpret_cast<float4 *>(&sm.gc[slot][4 * lane]) = gcv;
            }
            block_sync();
        };
        int sl2 = 0;  // (c+2) mod 3
        for (int64_t c = -2; c < nchunks; c += 2) {
            load_step(I0{}, c + 2, sl2);
            sl2 = sl2 == 2 ? 0 : sl2 + 1;
            if (c + 1 < nchunks) {
                load_step(I1{}, c + 3, sl2);
                sl2 = sl2 == 2 ? 0 : sl2 + 1;
            }
        }
        return;
    }

    if constexpr (GATE) {
        if (wave == W_STAGE || wave == W_STAGE + 1) {
            // ---- stager waves (channel-wise gate): the gate-scaled k rows of chunk c+2 into the
            // k buffer and its gate-scaled k~ rows (passed in d) into the k~ buffer ------------
            const uint16_t *ktg = reinterpret_cast<const uint16_t *>(d);
            auto gstager = [&](auto h_c) __attribute__((always_inline)) {
                constexpr int H = decltype(h_c)::value;
                auto stage_step = [&](auto par_c, int64_t cc, int slot) __attribute__((always_inline)) {
                    constexpr int PAR = decltype(par_c)::value;  // cc mod 2
                    if (cc < nchunks) {
                        load_rows<DK, 32 * H, 32>(k_buf[PAR], k, seq0 + cc * CH, rows_of(cc), lane);
                        load_kt_rows<DK, 32 * H, 32>(sm.kt[slot], ktg, seq0 + cc * CH, rows_of(cc), lane);
                        wait_global();
                    }
                    block_sync();
                };
                int sl2 = 0;  // (c+2) mod 3
                for (int64_t c = -2; c < nchunks; c += 2) {
                    stage_step(I0{}, c + 2, sl2);
                    sl2 = sl2 == 2 ? 0 : sl2 + 1;
                    if (c + 1 < nchunks) {
                        stage_step(I1{}, c + 3, sl2);
                        sl2 = sl2 == 2 ? 0 : sl2 + 1;
                    }
                }
            };
            if (wave == W_STAGE) gstager(I0{});
            else gstager(I1{});
            return;
        }
    }

    if (wave == W_STAGE || wave == W_STAGE + 1) {
        // ---- stager waves: k rows of chunk c+2 into LDS, then k~ = d (.) k of chunk c+2 -------
        // Stager h owns row blocks 2h, 2h+1.  d is loaded into registers one step before it is
        // used, block by block as soon as the block's registers are free (lane (q, n) holds
        // row 16 kb + n, features 32 s + 8 q .. +7).
        constexpr int DU = sizeof(TD) * 8 / 16;  // uint4 per 8 values of d
        uint4 dreg[2][NS][DU];
        auto stager = [&](auto h_c) __attribute__((always_inline)) {
            constexpr int H = decltype(h_c)::value;
            auto load_dblock = [&](int64_t cc, int j) __attribute__((always_inline)) {
                const int64_t row = seq0 + cc * CH + min(16 * (2 * H + j) + lr, rows_of(cc) - 1);
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(d + row * DK + 32 * s + 8 * lq);
#pragma unroll
                    for (int e = 0; e < DU; ++e) dreg[j][s][e] = src[e];
                }
            };
            if (nchunks > 0) {
                load_dblock(0, 0);
                load_dblock(0, 1);
            }
            auto stage_step = [&](auto par_c, int64_t cc, int slot) __attribute__((always_inline)) {
                constexpr int PAR = decltype(par_c)::value;  // cc mod 2
                if (cc < nchunks) {
                    load_rows<DK, 32 * H, 32>(k_buf[PAR], k, seq0 + cc * CH, rows_of(cc), lane);
                    wait_global();  // this chunk's k rows and d registers
                    const int64_t cn = cc + 1 < nchunks ? cc + 1 : nchunks - 1;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int kb = 2 * H + j;
                        v8s kr[NS];
#pragma unroll
                        for (int s = 0; s < NS; ++s)
                            kr[s] = ld8(&k_buf[PAR][L::qk_at(16 * kb + lr, 4 * s + lq)]);
#pragma unroll
                        for (int s = 0; s < NS; ++s) {
                            float dd[8];
                            d_values(dreg[j][s], dd, TD{});
                            const uint4 xu = __builtin_bit_cast(uint4, kr[s]);
                            const uint32_t xw[4] = {xu.x, xu.y, xu.z, xu.w};
                            uint32_t pk[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                pk[e] = pack2(dd[2 * e] * bf_lo(xw[e]), dd[2 * e + 1] * bf_hi(xw[e]));
                            *reinterpret_cast<uint4 *>(&sm.kt[slot][L::kt_at(16 * kb + lr, 4 * s + lq)]) =
                                make_uint4(pk[0], pk[1], pk[2], pk[3]);
                        }
                        load_dblock(cn, j);  // d of chunk c+3 (clamped to the last chunk)
                    }
                }
                block_sync();  // the d loads stay in flight across the barrier
            };
            int sl2 = 0;  // (c+2) mod 3
            for (int64_t c = -2; c < nchunks; c += 2) {
                stage_step(I0{}, c + 2, sl2);
                sl2 = sl2 == 2 ? 0 : sl2 + 1;
                if (c + 1 < nchunks) {
                    stage_step(I1{}, c + 3, sl2);
                    sl2 = sl2 == 2 ? 0 : sl2 + 1;
                }
            }
        };
        if (wave == W_STAGE) stager(I0{});
        else stager(I1{});
        return;
    }

    // ---- prep waves: Gram/score tiles and block inverses of chunk c+1 ----------------------------
    // Prep wave PW owns the column blocks kblk(PW, 0), kblk(PW, 1); s1 = (c+1) mod 3
    auto prep_step = [&](auto pw_c, int64_t c, int s1) __attribute__((always_inline)) {
        constexpr int PW = decltype(pw_c)::value;
        const int64_t c1 = c + 1;
        if (c1 < 0 || c1 >= nchunks) return;
        const int b1 = static_cast<int>(c1 & 1);
        const uint16_t *qx = q_buf[b1];
        const uint16_t *kx = k_buf[b1];
        const uint16_t *ktx = sm.kt[s1];
        // k~, k and q rows of the own blocks (all reads first: the compiler cannot move them
        // across the LDS writes below)
        v8s kt[2][NS], kr[2][NS], qd[2][NS];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int row = 16 * kblk(PW, j) + lr;
                kt[j][s] = ld8(&ktx[L::kt_at(row, 4 * s + lq)]);
                kr[j][s] = ld8(&kx[L::qk_at(row, 4 * s + lq)]);
                qd[j][s] = ld8(&qx[L::qk_at(row, 4 * s + lq)]);
            }
        // the decay factors and gates of every tile of the step, read before the first LDS
        // write (the compiler cannot move them above it)
        constexpr int IMIN = (kblk(PW, 0) < kblk(PW, 1) ? kblk(PW, 0) : kblk(PW, 1)) + 1;
        float hgr[2], hbt[2], hear[NBLK], hnbr[NBLK], hcik[NOFF];
        v4f hgs[2], heb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kb = kblk(PW, j);
            hgr[j] = sm.g[s1][16 * kb + lr];
            hbt[j] = sm.beta[s1][16 * kb + lr];
            hgs[j] = ld4(&sm.g[s1][16 * kb + 4 * lq]);
            heb[j] = ld4(&sm.eb[s1][16 * kb + 4 * lq]);
        }
#pragma unroll
        for (int i = IMIN; i < NBLK; ++i) {
            hear[i] = sm.ea[s1][16 * i + lr];
            hnbr[i] = -sm.beta[s1][16 * i + lr];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kb = kblk(PW, j);
                if (kb < i) hcik[(i * (i - 1)) / 2 + kb] = sm.cik[s1][(i * (i - 1)) / 2 + kb];
            }
        }
        // diagonal blocks: tile (kb, kb) = K~_kb X_kb^T, the lane holds row r = 16kb+lr,
        // columns s = 16kb+4lq..+3; exact e^{g_r - g_s} shared by the score tile (s <= r)
        // and N (s < r); then both block inverses in lockstep
        v4f na[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kb = kblk(PW, j);
            const int r = 16 * kb + lr;
            v4f sc = zero4(), Gdt = zero4();
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                sc = mfma32(kt[j][s], qd[j][s], sc);
                Gdt = mfma32(kt[j][s], kr[j][s], Gdt);  // G in the A layout: lane holds G[r][s]
            }
            const float gr = hgr[j], bt = hbt[j];
            const v4f gs = hgs[j];
            v4f pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ex = __expf(gr - gs[e]);
                pv[e] = (4 * lq + e <= lr) ? ex * sc[e] : 0.f;
                na[j][e] = (4 * lq + e < lr) ? (bt * ex) * Gdt[e] : 0.f;
            }
            *reinterpret_cast<uint2 *>(&sm.p[b1][r * L::CP + 16 * kb + 4 * lq]) = pack4u(pv);
        }
        diag_inverse2<DK>(sm, b1, kblk(PW, 0), kblk(PW, 1), lr, lq, na);
        // off-diagonal tiles (i, kb), i > kb, row block by row block; the fragments of the
        // next row block are read before the current one is processed.  The lane holds row
        // 16i+lr, columns 16kb+4lq..+3; e^{g_r - g_s} = ea[r] cik eb[s], each factor <= 1.
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
            const float ear = hear[i], nbr = hnbr[i];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kb = kblk(PW, j);
                if (kb >= i) continue;
                v4f sc = zero4(), gm = zero4();
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    sc = mfma32(kt[j][s], qf[s], sc);
                    gm = mfma32(kt[j][s], kf[s], gm);
                }
                const int t = (i * (i - 1)) / 2 + kb;
                const float rowf = ear * hcik[t];
                const float growf = nbr * rowf;
                const v4f eb4 = heb[j];
                v4f pv, av;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pv[e] = (sc[e] * rowf) * eb4[e];
                    av[e] = (gm[e] * growf) * eb4[e];
                }
                *reinterpret_cast<uint2 *>(&sm.p[b1][r * L::CP + 16 * kb + 4 * lq]) = pack4u(pv);
                *reinterpret_cast<uint2 *>(&sm.aneg[b1][t * 16 * L::DP + L::blk(lr, lq)]) =
                    pack4u(av);
            }
        }
    };
    // one loop per prep wave, so its registers need no merging between the two variants.
    // Prep wave 0 also runs the decay scan of chunk c+2 after its tiles (it issues no memory
    // instruction, so neither its LDS writes nor its scan wait for loads); the loader brought
    // that chunk's beta and alpha into LDS a step earlier.
    // L2 warm-up (the second prep wave, plain forward): two steps before the loader and the
    // stagers load chunk cc, this workgroup touches its share (1/nvt) of the chunk's 128-byte
    // lines of q, k, d and v with one dword load each, so that their loads hit L2 instead of
    // waiting on HBM.  The values are only waited for two steps later (an empty asm use).
    constexpr int QL = DK * 2 / 128;                 // 128-byte lines per row of q (and k)
    constexpr int DL = DK * int(sizeof(TD)) / 128;   // ... of d
    constexpr int PFN = (2 * QL + DL + 2 + 1) / 2;   // loads per lane (at most 2 lines of v a
                                                     // row, at least 2 workgroups a sequence)
    constexpr int PFD = 2;                           // prefetch distance in chunks
    const int VL = dv * 2 / 128;                     // ... of v
    const int RL = 2 * QL + DL + VL;                 // lines per row, all four tensors
    auto prefetch = [&](int64_t cc, uint32_t (&pf)[PFN]) __attribute__((always_inline)) {
        const int n = cc < nchunks ? rows_of(cc) : 0;
        const int total = n * RL, per = (total + nvt - 1) / nvt, first = vt * per;
#pragma unroll
        for (int i = 0; i < PFN; ++i) {
            const int li = 64 * i + lane, l = first + li;
            uint32_t x = 0;
            if (li < per && l < total) {
                const int row = l / RL, w = l % RL;
                const int64_t tr = seq0 + cc * CH + row;
                const char *p;
                if (w < QL) p = reinterpret_cast<const char *>(q + tr * DK) + 128 * w;
                else if (w < 2 * QL) p = reinterpret_cast<const char *>(k + tr * DK) + 128 * (w - QL);
                else if (w < 2 * QL + DL) p = reinterpret_cast<const char *>(d + tr * DK) + 128 * (w - 2 * QL);
                else p = reinterpret_cast<const char *>(v + tr * dv) + 128 * (w - 2 * QL - DL);
                x = *reinterpret_cast<const uint32_t *>(p);
            }
            pf[i] = x;
        }
    };
    // one loop per prep wave, so its registers need no merging between the two variants.
    // Prep wave 0 also runs the decay scan of chunk c+2 after its tiles (it issues no memory
    // instruction, so neither its LDS writes nor its scan wait for loads); the loader brought
    // that chunk's beta and alpha into LDS a step earlier.
    auto prep_loop = [&](auto pw_c) __attribute__((always_inline)) {
        constexpr int PW = decltype(pw_c)::value;
        constexpr bool PF = !GATE && !CKPT && PW == 1;  // (with the checkpoint stores in the
                                                         // way, the warmed lines were evicted
                                                         // before use: +38 MB fetched)
        uint32_t pfa[PFN], pfb[PFN];
#pragma unroll
        for (int i = 0; i < PFN; ++i) pfa[i] = pfb[i] = 0;
        int sl1 = 2;  // (c+1) mod 3; (c+2) mod 3 is the slot after it
        auto body = [&](int64_t c, uint32_t (&pf)[PFN]) __attribute__((always_inline)) {
            if constexpr (PF) {
#pragma unroll
                for (int i = 0; i < PFN; ++i) asm volatile("" ::"v"(pf[i]));  // from step c-2
                prefetch(c + 2 + PFD, pf);
            }
            if constexpr (!GATE) {
                prep_step(pw_c, c, sl1);
            } else if constexpr (PW == 1) {
                // channel-wise gate: chunk c+1's planes (P, the block inverses, -A_ik) are
                // copied in as formed by the planes kernel
                namespace KP = kda_planes;
                const int64_t c1 = c + 1;
                if (c1 >= 0 && c1 < nchunks) {
                    const int b1 = static_cast<int>(c1 & 1);
                    const uint16_t *img = planes + (bh * nchunks + c1) * KP::kElems;
                    copy_image<KP::kP / 8>(sm.p[b1], img, lane);
                    copy_image<KP::kDinv / 8>(sm.dinv[b1], img + KP::kP, lane);
                    copy_image<KP::kAneg / 8>(sm.aneg[b1], img + KP::kP + KP::kDinv, lane);
                    wait_global();
                }
            }
            if constexpr (PW == 0) {
                const int64_t cc = c + 2;
                if (cc < nchunks) {
                    const int sl2 = sl1 == 2 ? 0 : sl1 + 1;
                    const int par = static_cast<int>(cc & 1);
                    scan_chunk<DK>(sm, sl2, sm.rawb[par][lane], has_alpha ? sm.rawa[par][lane] : 1.f,
                                   rows_of(cc), has_alpha, lane);
                }
            }
            block_sync();
            sl1 = sl1 == 2 ? 0 : sl1 + 1;
        };
        for (int64_t c = -2; c < nchunks; c += 2) {
            body(c, pfa);
            if (c + 1 < nchunks) body(c + 1, pfb);
        }
        if constexpr (PF) {
#pragma unroll
            for (int i = 0; i < PFN; ++i) asm volatile("" ::"v"(pfa[i]), "v"(pfb[i]));
        }
    };
    if (wave == W_PREP) prep_loop(I0{});
    else prep_loop(I1{});
}

// compute units of the current device (cached per device)
int device_cus() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int DK, typename TD>
hipError_t launch_typed(const ChunkArgs &a, hipStream_t stream) {
    // Plain forward: where even 16-column slices (one state wave a workgroup) leave the grid
    // within one workgroup per compute unit, take them: the per-chunk chain of a workgroup is
    // no longer, and twice as many compute units walk the sequences (long sequences, few heads).
    const bool narrow = !a.gcs && !a.ckpt && a.BH * (a.dv / VW) <= device_cus();
    const int nvt = a.dv / (narrow ? VW : 2 * VW);
    const dim3 grid(static_cast<unsigned>(a.BH * nvt));
    if (narrow) {
        hipLaunchKernelGGL((chunk_mfma_kernel<DK, TD, false, false, true, 1>), grid,
                           dim3(n_waves(1) * 64), 0, stream, static_cast<const uint16_t *>(a.q),
                           static_cast<const uint16_t *>(a.k), static_cast<const uint16_t *>(a.v),
                           static_cast<const TD *>(a.d), a.beta, a.alpha, a.S0,
                           static_cast<uint16_t *>(a.o), a.S_T, a.BH, a.T, a.dv, a.gcs,
                           static_cast<uint16_t *>(a.ckpt), static_cast<uint16_t *>(a.uout), a.planes);
        return hipGetLastError();
    }
#define OSDN_CHUNK_LAUNCH(GATE, CKPT, OUT)                                                    \
    hipLaunchKernelGGL((chunk_mfma_kernel<DK, TD, GATE, CKPT, OUT, 2>), grid,                 \
                       dim3(n_waves(2) * 64), 0,                                              \
                       stream, static_cast<const uint16_t *>(a.q),                             \
                       static_cast<const uint16_t *>(a.k), static_cast<const uint16_t *>(a.v), \
                       static_cast<const TD *>(a.d), a.beta, a.alpha, a.S0,                    \
                       static_cast<uint16_t *>(a.o), a.S_T, a.BH, a.T, a.dv, a.gcs,            \
                       static_cast<uint16_t *>(a.ckpt), static_cast<uint16_t *>(a.uout),       \
                       a.planes)
    if (a.gcs) OSDN_CHUNK_LAUNCH(true, false, true);
    else if (a.ckpt && a.o) OSDN_CHUNK_LAUNCH(false, true, true);
    else if (a.ckpt) OSDN_CHUNK_LAUNCH(false, true, false);
    else OSDN_CHUNK_LAUNCH(false, false, true);
#undef OSDN_CHUNK_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_fwd_mfma(const ChunkArgs &a, hipStream_t stream) {
    if (a.gcs)  // channel-wise gate: d carries the gate-scaled k~ (bf16)
        return a.dk == 64 ? launch_typed<64, bf16_t>(a, stream) : launch_typed<128, bf16_t>(a, stream);
    if (a.dk == 64)
        return a.d_dtype == OSDN_F32 ? launch_typed<64, float>(a, stream)
                                     : launch_typed<64, bf16_t>(a, stream);
    return a.d_dtype == OSDN_F32 ? launch_typed<128, float>(a, stream)
                                 : launch_typed<128, bf16_t>(a, stream);
}

}  // namespace osdn
