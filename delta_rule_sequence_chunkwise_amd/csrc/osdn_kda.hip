// Channel-wise (Kimi Delta Attention) gate for OSDN, gfx950: the per-token diagonal decay
// Diag(a_t) of Erase-then-Delta Attention, section 2.2, eq. 5 (section 3.2, eq. 7), with the
// OSDN write key k~ = d (.) k (OSDN technical summary, section 2.1):
//
//   M_t = Diag(a_t) M_{t-1} + b_t k~_t (v_t - (Diag(a_t) M_{t-1})^T k_t)^T ,   o_t = M_t^T q_t
//
// Chunkwise (derived here; the pages give no chunk form), with G_r = prod_{t<=r} a_t from the
// chunk start and rho(s->r) = prod_{s<t<=r} a_t, per key feature:
//
//   (I + A) U = diag(b) (V - (K o G) M0),   A[r,s] = b_r sum_f k_rf k~_sf rho_f(s->r)  (s < r)
//   O = (Q o G) M0 + P U,                   P[r,s] = sum_f q_rf k~_sf rho_f(s->r)      (s <= r)
//   M_C = Diag(G_C) M0 + (K~ o rho(.->C))^T U
//
// The ratio rho sits inside the dk-long inner products, so it is folded into the operands of the
// matrix products -- as products of gates only, each at most 1, never as G_r / G_s (a running
// product from the chunk start underflows after a few strong gates, and its reciprocal then
// overflows).  Pairs (r, s) in different 16-row blocks i > j are anchored at the last row e of
// block j: x_r = prod_{e<t<=r} a_t, y_s = prod_{s<t<=e} a_t.  Inside a block, the pair falls
// into different halves of one 2h-row segment for exactly one h in {8, 4, 2, 1}, and is anchored
// at the boundary of those halves; one product per h covers all such pairs, and its other
// entries are dropped.  The diagonal takes factor 1.  The segment products come level by level
// from the sibling segment's total (a lane swap), so no factor is ever divided.
//
// kda_planes_kernel does this for every chunk in parallel (one workgroup of four waves per
// chunk, wave i on rows 16i..16i+15, lane (row, quarter) holding 8 features of each 32-wide
// k-step in registers, which is both the A and the B layout of the 16x16x32 products), and
// writes for the forward: q o G, k o G, k~ o rho(.->C) (bf16), G_C, and the chunk planes -- P,
// the diagonal-block inverses (I + A_ii)^{-1} (the forward's own series on bf16 matrix cores)
// and -A_ik (bf16, in the forward's LDS layout).  The matrix-core forward's GATE variant copies these in
// instead of forming them.  (The fp32 path forms the exact ratios itself; see the fp32 kernel.)
//
// The decode step applies Diag(a) to the state's rows in place of the scalar gate.
#include "osdn_internal.h"
#include "osdn_mfma.h"

namespace osdn {
namespace {

constexpr int kPlanesThreads = 512;  // 8 waves: (16-row block, half of the key features)

// 8 consecutive inputs as fp32
__device__ __forceinline__ void load8(const float *p, float *o) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t *p, float *o) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o[2 * e] = bf_lo(w[e]);
        o[2 * e + 1] = bf_hi(w[e]);
    }
}
__device__ __forceinline__ void load8(const uint16_t *p, float *o) {
    load8(reinterpret_cast<const bf16_t *>(p), o);
}
// 8 fp32 products x * f rounded to one bf16 fragment
__device__ __forceinline__ v8s frag8(const float *x, const float *f) {
    return __builtin_bit_cast(v8s, make_uint4(pack2(x[0] * f[0], x[1] * f[1]), pack2(x[2] * f[2], x[3] * f[3]),
                                              pack2(x[4] * f[4], x[5] * f[5]), pack2(x[6] * f[6], x[7] * f[7])));
}
// 8 bf16 values (4 packed words) times 8 fp32 factors, rounded to one bf16 fragment
__device__ __forceinline__ v8s frag8p(const uint32_t *x, const float *f) {
    return __builtin_bit_cast(v8s, make_uint4(pack2(bf_lo(x[0]) * f[0], bf_hi(x[0]) * f[1]),
                                              pack2(bf_lo(x[1]) * f[2], bf_hi(x[1]) * f[3]),
                                              pack2(bf_lo(x[2]) * f[4], bf_hi(x[2]) * f[5]),
                                              pack2(bf_lo(x[3]) * f[6], bf_hi(x[3]) * f[7])));
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int DK, typename TD>
__global__ void __launch_bounds__(kPlanesThreads)
kda_planes_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const TD *__restrict__ d, const float *__restrict__ a,
                  const float *__restrict__ beta, uint16_t *__restrict__ qp,
                  uint16_t *__restrict__ kp, uint16_t *__restrict__ ktp,
                  uint16_t *__restrict__ planes, float *__restrict__ gcs, int64_t T,
                  int64_t nchunks, int64_t total) {
    namespace KP = kda_planes;
    constexpr int NS = DK / 32;   // 32-wide k-steps
    constexpr int NSH = NS / 2;   // k-steps of one feature half
    constexpr int NV = NSH * 8;   // feature values per lane: k-step s0 + s, element e -> 32 (s0 + s) + 8 lq + e
    __shared__ alignas(16) float btot[4][DK];                        // product of a block's 16 gates
    __shared__ alignas(16) uint16_t ycol[3][NS][64 * 8];             // k~ o (suffix product), B fragments
    __shared__ alignas(16) float sbeta[KP::kRows];
    __shared__ alignas(16) float part[2][10][2][64 * 4];             // partial tiles per feature half
    __shared__ alignas(16) uint16_t sN[4][256];                      // N of each block, for its A layout

    const int tid = threadIdx.x;
    const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = w8 & 3, fh = w8 >> 2;  // row block, feature half
    const int s0 = fh * NSH;
    const int lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int r = 16 * w + lr;               // row in the chunk
    auto feat = [&](int i) __attribute__((always_inline)) { return 32 * (s0 + i / 8) + 8 * lq + i % 8; };

    // The workgroups are persistent: each takes every gridDim.x-th (sequence, chunk) and loads
    // the lane's row of the next one (gates, q and k packed as bf16 pairs, d, beta) while it
    // works on the current one.  Rows past the end: gate 1, zero operands, beta 0.
    float pa[NV], pd[NV], pb;
    uint32_t pq[NV / 2], pk[NV / 2];
    auto fetch = [&](int64_t sg) __attribute__((always_inline)) {
        const int64_t bh_ = sg / nchunks, t_ = (sg % nchunks) * KP::kRows + r;
        if (sg < total && t_ < T) {
            const int64_t off = (bh_ * T + t_) * DK;
#pragma unroll
            for (int s = 0; s < NSH; ++s) {
                const int f0 = feat(8 * s);
                load8(a + off + f0, pa + 8 * s);
                const uint4 uq = *reinterpret_cast<const uint4 *>(q + off + f0);
                const uint4 uk = *reinterpret_cast<const uint4 *>(k + off + f0);
                pq[4 * s] = uq.x; pq[4 * s + 1] = uq.y; pq[4 * s + 2] = uq.z; pq[4 * s + 3] = uq.w;
                pk[4 * s] = uk.x; pk[4 * s + 1] = uk.y; pk[4 * s + 2] = uk.z; pk[4 * s + 3] = uk.w;
                load8(d + off + f0, pd + 8 * s);
            }
            pb = beta[bh_ * T + t_];
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                pa[i] = 1.f;
                pd[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < NV / 2; ++i) pq[i] = pk[i] = 0u;
            pb = 0.f;
        }
    };
    fetch(blockIdx.x);
    for (int64_t seg = blockIdx.x; seg < total; seg += gridDim.x) {
    const int64_t bh = seg / nchunks, c = seg % nchunks;
    const int64_t t = c * KP::kRows + r;     // row in the sequence
    const bool valid = t < T;
    const int64_t rowoff = (bh * T + (valid ? t : 0)) * DK;
    // the lane's row: gates, q, k (packed: qv[4 s + e] holds elements 2 e, 2 e + 1 of k-step
    // s), k~ = d o k
    float av[NV], ktv[NV];
    uint32_t qv[NV / 2], kv[NV / 2];
#pragma unroll
    for (int i = 0; i < NV; ++i) av[i] = pa[i];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) {
        qv[i] = pq[i];
        kv[i] = pk[i];
        ktv[2 * i] = pd[2 * i] * bf_lo(pk[i]);
        ktv[2 * i + 1] = pd[2 * i + 1] * bf_hi(pk[i]);
    }
    if (fh == 0 && lq == 0) sbeta[r] = pb;
    fetch(seg + gridDim.x);

    // segment products of the gates: pre = inclusive prefix, suf = exclusive suffix, tot = whole
    // segment, per feature, over the lane's aligned h-row segment (h = 1, 2, 4, 8, 16)
    float pre[NV], suf[NV], tot[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        pre[i] = av[i];
        suf[i] = 1.f;
        tot[i] = av[i];
    }
    v4f accA = zero4(), accP = zero4();  // diagonal block, C layout: row 4 lq + e, column lr
    // pairs with row r in the upper h-half and column s in the lower h-half of one 2h-segment
    auto level = [&](auto h_c) __attribute__((always_inline)) {
        constexpr int H = decltype(h_c)::value;
        constexpr int SH = H == 1 ? 1 : H == 2 ? 2 : H == 4 ? 3 : 4;  // log2(2H)
        const bool up = (lr & H) != 0;
        v4f ca = zero4(), cp = zero4();
#pragma unroll
        for (int s = 0; s < NSH; ++s) {
            float fx[8], fy[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                fx[e] = up ? pre[8 * s + e] : 0.f;
                fy[e] = up ? 0.f : suf[8 * s + e];
            }
            const v8s y = frag8(ktv + 8 * s, fy);
            ca = mfma32(frag8p(kv + 4 * s, fx), y, ca);
            cp = mfma32(frag8p(qv + 4 * s, fx), y, cp);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 4 * lq + e;
            if (((row ^ lr) >> SH) == 0) {
                accA[e] += ca[e];
                accP[e] += cp[e];
            }
        }
    };
    // h -> 2h: the sibling h-segment's total arrives by a lane swap that stays inside the
    // 2h-segment (any lane of the sibling holds the same total)
    auto grow = [&](auto h_c, auto ctrl_c) __attribute__((always_inline)) {
        constexpr int H = decltype(h_c)::value;
        constexpr int CTRL = decltype(ctrl_c)::value;
        const bool lower = (lr & H) == 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const float sib = dpp_mov<CTRL>(tot[i]);
            pre[i] = lower ? pre[i] : sib * pre[i];
            suf[i] = lower ? suf[i] * sib : suf[i];
            tot[i] = tot[i] * sib;
        }
    };
    using std::integral_constant;
    level(integral_constant<int, 1>{});
    grow(integral_constant<int, 1>{}, integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    level(integral_constant<int, 2>{});
    grow(integral_constant<int, 2>{}, integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
    level(integral_constant<int, 4>{});
    grow(integral_constant<int, 4>{}, integral_constant<int, 0x141>{});  // row_half_mirror
    level(integral_constant<int, 8>{});
    grow(integral_constant<int, 8>{}, integral_constant<int, 0x140>{});  // row_mirror
    {  // the diagonal of P: factor 1
        v4f cp = zero4();
#pragma unroll
        for (int s = 0; s < NSH; ++s) {
            const float *ts = ktv + 8 * s;
            const v8s xq = __builtin_bit_cast(v8s, make_uint4(qv[4 * s], qv[4 * s + 1], qv[4 * s + 2], qv[4 * s + 3]));
            const v8s xt = __builtin_bit_cast(v8s, make_uint4(pack2(ts[0], ts[1]), pack2(ts[2], ts[3]),
                                                              pack2(ts[4], ts[5]), pack2(ts[6], ts[7])));
            cp = mfma32(xq, xt, cp);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * lq + e == lr) accP[e] += cp[e];
    }
    // pre, suf, tot now span the lane's 16-row block
    if (lr == 0) {
#pragma unroll
        for (int s = 0; s < NSH; ++s) {
            float *dst = &btot[w][feat(8 * s)];
            *reinterpret_cast<float4 *>(dst) = make_float4(tot[8 * s], tot[8 * s + 1], tot[8 * s + 2], tot[8 * s + 3]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(tot[8 * s + 4], tot[8 * s + 5], tot[8 * s + 6], tot[8 * s + 7]);
        }
    }
    if (w < 3) {
#pragma unroll
        for (int s = 0; s < NSH; ++s)
            *reinterpret_cast<v8s *>(&ycol[w][s0 + s][8 * lane]) = frag8(ktv + 8 * s, suf + 8 * s);
    }
    __syncthreads();

    // products over other blocks' totals, 8 features at a time from LDS
    auto mul_btot = [&](float *x, int m) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < NSH; ++s) {
            const float *src = &btot[m][feat(8 * s)];
            const v4f b0 = ld4(src), b1 = ld4(src + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * s + e] *= b0[e];
                x[8 * s + 4 + e] *= b1[e];
            }
        }
    };
    // the forward's operands: q o G, k o G with G = (blocks before) o pre; k~ o rho(.->C) =
    // k~ o suf o (blocks after); G_C = the product of all four block totals
    {
        float g[NV], h[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            g[i] = pre[i];
            h[i] = suf[i];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m < w) mul_btot(g, m);
            if (m > w) mul_btot(h, m);
        }
        if (valid) {
#pragma unroll
            for (int s = 0; s < NSH; ++s) {
                const int64_t o = rowoff + feat(8 * s);
                *reinterpret_cast<v8s *>(qp + o) = frag8p(qv + 4 * s, g + 8 * s);
                *reinterpret_cast<v8s *>(kp + o) = frag8p(kv + 4 * s, g + 8 * s);
                *reinterpret_cast<v8s *>(ktp + o) = frag8(ktv + 8 * s, h + 8 * s);
            }
        }
        if (w == 3 && lr == 15) {  // G at the chunk's last row: (blocks 0..2) o the block's total
#pragma unroll
            for (int s = 0; s < NSH; ++s) {
                float *dst = gcs + seg * DK + feat(8 * s);
                *reinterpret_cast<float4 *>(dst) = make_float4(g[8 * s], g[8 * s + 1], g[8 * s + 2], g[8 * s + 3]);
                *reinterpret_cast<float4 *>(dst + 4) = make_float4(g[8 * s + 4], g[8 * s + 5], g[8 * s + 6], g[8 * s + 7]);
            }
        }
    }

    // tiles (w, j), j < w: rows anchored at the last row of block j.  Each half's partial
    // products go to LDS (slot w: the diagonal tile; 4 + w (w - 1) / 2 + j: tile (w, j))
    float cross[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) cross[i] = 1.f;
    *reinterpret_cast<v4f *>(&part[fh][w][0][4 * lane]) = accA;
    *reinterpret_cast<v4f *>(&part[fh][w][1][4 * lane]) = accP;
#pragma unroll
    for (int j = 2; j >= 0; --j) {
        if (j < w) {
            v4f ca = zero4(), cp = zero4();
#pragma unroll
            for (int s = 0; s < NSH; ++s) {
                float fx[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) fx[e] = pre[8 * s + e] * cross[8 * s + e];
                const v8s y = *reinterpret_cast<const v8s *>(&ycol[j][s0 + s][8 * lane]);
                ca = mfma32(frag8p(kv + 4 * s, fx), y, ca);
                cp = mfma32(frag8p(qv + 4 * s, fx), y, cp);
            }
            const int slot = 4 + (w * (w - 1)) / 2 + j;
            *reinterpret_cast<v4f *>(&part[fh][slot][0][4 * lane]) = ca;
            *reinterpret_cast<v4f *>(&part[fh][slot][1][4 * lane]) = cp;
            mul_btot(cross, j);
        }
    }
    __syncthreads();

    // the two halves summed: half 0 finishes the diagonal block (P, and the inverse of
    // I + A_ii), half 1 the off-diagonal tiles (P and -A_ij)
    uint16_t *img = planes + seg * KP::kElems;
    uint16_t *pimg = img, *dimg = img + KP::kP, *aimg = img + KP::kP + KP::kDinv;
    const v4f b4 = ld4(&sbeta[16 * w + 4 * lq]);  // beta of the rows 4 lq + e of this block
    // after a quad transpose the lane holds row 4 lq + (lr & 3), columns 4 (lr >> 2) .. +3
    const int trow = 4 * lq + (lr & 3), tg = lr >> 2;
    auto tile_sum = [&](int slot, int m) __attribute__((always_inline)) {
        return ld4(&part[0][slot][m][4 * lane]) + ld4(&part[1][slot][m][4 * lane]);
    };
    auto store_p = [&](int j, v4f x) __attribute__((always_inline)) {
        *reinterpret_cast<uint2 *>(pimg + (16 * w + trow) * KP::kPPitch + 16 * j + 4 * tg) =
            pack4u(quad_transpose(x, lane));
    };
    if (fh == 1) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            if (j < w) {
                const int slot = 4 + (w * (w - 1)) / 2 + j;
                *reinterpret_cast<uint2 *>(aimg + (slot - 4) * 256 + KP::blk(trow, tg)) =
                    pack4u(quad_transpose(-b4 * tile_sum(slot, 0), lane));
                store_p(j, tile_sum(slot, 1));
            }
        }
    } else {
    store_p(w, tile_sum(w, 1));
    for (int j = w + 1; j < 4; ++j) store_p(j, zero4());
    // D = (I + N)^{-1}, N = diag(beta) A_ii strictly lower (so N^16 = 0), as
    // (I - N)(I + N^2)(I + N^4)(I + N^8) on bf16 matrix cores.  N's C layout is its B layout; its
    // A layout comes back through LDS.  The result, in the C layout of D^T = the A layout of D
    // (lane holds row lr, columns 4 lq .. +3), is stored as the forward keeps it.
    const v4f nC = b4 * tile_sum(w, 0);
    uint16_t *scr = &sN[w][0];
    *reinterpret_cast<uint2 *>(scr + KP::blk(trow, tg)) = pack4u(quad_transpose(nC, lane));
    asm volatile("" ::: "memory");
    const v4s Na = ld4s(scr + KP::blk(lr, lq)), Nb = pack4(nC);
    v4f X = mfma16(Na, Nb, zero4()), Xt = mfma16(Nb, Na, zero4());  // N^2 (B layout), its transpose
    const v4s N2a = pack4(Xt), N2b = pack4(X);
    X = mfma16(N2a, N2b, zero4());
    Xt = mfma16(N2b, N2a, zero4());
    const v4s N4a = pack4(Xt), N4b = pack4(X);
    v4f Y = mfma16(N4b, N4a, zero4());  // (N^8)^T
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (4 * lq + e == lr) Y[e] += 1.f;
    Y = mfma16(N4b, pack4(Y), Y);
    Y = mfma16(N2b, pack4(Y), Y);
    const uint2 nb = __builtin_bit_cast(uint2, Nb);
    Y = mfma16(__builtin_bit_cast(v4s, make_uint2(nb.x ^ 0x80008000u, nb.y ^ 0x80008000u)), pack4(Y), Y);
    *reinterpret_cast<uint2 *>(dimg + w * 256 + KP::blk(lr, lq)) = pack4u(Y);
    }
    __syncthreads();  // the next chunk reuses the LDS
    }
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
    for (int i = 0; i < RPT; ++i) m[i] = load_stream(&Mrow[(rg + i * RG) * TPR + cg]);

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
        store_stream(&Mrow[row * TPR + cg], mn);
    }
}

// one persistent workgroup per compute unit (its registers allow no second)
int compute_units() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, cu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cu > 0)
            n = cu;
        else
            n = 256;
    }
    return n;
}

template <int DK, typename TD>
hipError_t planes_typed(const KdaPrepArgs &a, hipStream_t stream) {
    const int64_t total = a.BH * a.nchunks;
    const dim3 grid(static_cast<unsigned>(total < compute_units() ? total : compute_units()));
    hipLaunchKernelGGL((kda_planes_kernel<DK, TD>), grid, dim3(kPlanesThreads), 0, stream,
                       static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
                       static_cast<const TD *>(a.d), a.alpha_ch, a.beta,
                       static_cast<uint16_t *>(a.qp), static_cast<uint16_t *>(a.kp),
                       static_cast<uint16_t *>(a.ktp), a.planes, a.gcs, a.T, a.nchunks, total);
    return hipGetLastError();
}

template <int DK>
hipError_t planes_dk(const KdaPrepArgs &a, hipStream_t stream) {
    return a.d_dtype == OSDN_F32 ? planes_typed<DK, float>(a, stream)
                                 : planes_typed<DK, bf16_t>(a, stream);
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

hipError_t launch_kda_planes(const KdaPrepArgs &a, hipStream_t stream) {
    return a.dk == 64 ? planes_dk<64>(a, stream) : planes_dk<128>(a, stream);
}

hipError_t launch_step_kda(const StepArgs &a, hipStream_t stream) {
    if (a.dk == 64) return a.dv == 64 ? step_dims<64, 64>(a, stream) : step_dims<64, 128>(a, stream);
    return a.dv == 64 ? step_dims<128, 64>(a, stream) : step_dims<128, 128>(a, stream);
}

}  // namespace osdn
