// Device helpers shared by the gfx950 matrix-core kernels of libosdn: bf16 MFMA operands and
// products, LDS access forms (including the transposing read), global-to-LDS copies, wait and
// barrier forms, and cross-lane sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "osdn_internal.h"

namespace osdn {

typedef short v8s __attribute__((__vector_size__(8 * sizeof(short))));
typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
typedef float v4f __attribute__((__vector_size__(4 * sizeof(float))));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

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
// 4 bytes from global memory straight into LDS: lane l's bytes land at lds_base + 4 l
__device__ __forceinline__ void load_to_lds4(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds((glb_void_t *)(g), (lds_void_t *)(lds_base), 4, 0, 0);
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
// at most 8 vector memory operations of this wave still in flight: issuing loads in groups
// of 8 with this wait between them keeps the CU's load queues from thrashing
__device__ __forceinline__ void wait_global8() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0f78);  // vmcnt(8)
    asm volatile("" ::: "memory");
}
// at most N vector memory operations of this wave still in flight
template <int N>
__device__ __forceinline__ void wait_global_n() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

// Element (f, col) of a bf16 dk x dv state (or state-gradient) checkpoint of one chunk, stored as
// dv / 16 tiles of dk x 16, each tile contiguous: a wave owns 16 value columns, so its 8-byte-
// per-lane store of 16 rows covers 512 contiguous bytes (row-major, it would write sixteen
// 32-byte pieces of separate rows)
__host__ __device__ constexpr int64_t ckpt_at(int f, int col, int dk) {
    return (static_cast<int64_t>(col >> 4) * dk + f) * 16 + (col & 15);
}
// Element (row r, value column col) of a 64-row chunk's block of a bf16 per-row buffer of the
// backward (U, dR): dv / 16 contiguous 64 x 16 column tiles, for the same reason
__host__ __device__ constexpr int rows_at(int r, int col) { return ((col >> 4) * 64 + r) * 16 + (col & 15); }

// x + (x of the lane selected by the DPP control), 0 where the control selects no lane
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false);
    return x + __int_as_float(y);
}
// x summed over each aligned group of G lanes (G = 1, 2, 4, 8 or 16), every lane receiving its
// group's sum, on DPP: the two quad swaps, then the half-row and row mirrors
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "lane group");
    if constexpr (G >= 2) x = dpp_add<0xb1, 0xf>(x);   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) x = dpp_add<0x4e, 0xf>(x);   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) x = dpp_add<0x141, 0xf>(x);  // row_half_mirror
    if constexpr (G >= 16) x = dpp_add<0x140, 0xf>(x); // row_mirror
    return x;
}

__device__ __forceinline__ float lane_value(float x, int l) {  // x of lane l (wave-uniform)
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// x summed with the lanes 16 and 32 away: each 16-lane row receives the sum of the four rows
// at its own position (the two row swaps v_permlane32_swap and v_permlane16_swap)
__device__ __forceinline__ float sum_rows(float x) {
    const uint32_t b = __float_as_uint(x);
    const u32x2 s = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    const float y = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    const uint32_t c = __float_as_uint(y);
    const u32x2 t = __builtin_amdgcn_permlane16_swap(c, c, false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// sum of x over the 16 lanes of each row (inclusive prefix sums by DPP row shifts), valid in
// the row's last lane
__device__ __forceinline__ float row16_total(float x) {
    x = dpp_add<0x111, 0xf>(x);  // row_shr:1
    x = dpp_add<0x112, 0xf>(x);  // row_shr:2
    x = dpp_add<0x114, 0xf>(x);  // row_shr:4
    return dpp_add<0x118, 0xf>(x);  // row_shr:8
}
// inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each 16-lane row, then
// the last lane of rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3
__device__ __forceinline__ float wave_prefix(float x) {
    x = dpp_add<0x111, 0xf>(x);  // row_shr:1
    x = dpp_add<0x112, 0xf>(x);  // row_shr:2
    x = dpp_add<0x114, 0xf>(x);  // row_shr:4
    x = dpp_add<0x118, 0xf>(x);  // row_shr:8
    x = dpp_add<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
    return dpp_add<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
}
// inclusive suffix sum over the 64 lanes (lane r receives the sum of lanes r .. 63): shifts
// by 1, 2, 4, 8 towards lower lanes inside each 16-lane row, then the totals of the later rows,
// read from their first lanes
__device__ __forceinline__ float wave_suffix(float x, int lane) {
    x = dpp_add<0x101, 0xf>(x);  // row_shl:1
    x = dpp_add<0x102, 0xf>(x);  // row_shl:2
    x = dpp_add<0x104, 0xf>(x);  // row_shl:4
    x = dpp_add<0x108, 0xf>(x);  // row_shl:8
    const float t1 = lane_value(x, 16), t2 = lane_value(x, 32), t3 = lane_value(x, 48);
    const int row = lane >> 4;
    const float later = row == 0 ? (t3 + t2) + t1 : (row == 1 ? t3 + t2 : (row == 2 ? t3 : 0.f));
    return x + later;
}
// 4 x 4 transpose inside each quad of lanes by two DPP exchange stages: lane 4a + l holds
// x[e] = X[l][e] on entry and X[e][l] on return.  On a 16x16 tile in the MFMA C layout (lane
// (q, n) holds rows 4q..4q+3 of column n) lane (q, n) then holds row 4q + (n & 3), columns
// 4 (n >> 2) .. +3, ready for one vector store.
__device__ __forceinline__ v4f quad_transpose(v4f x, int lane) {
    const bool o1 = lane & 1, o2 = lane & 2;
    auto xch = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
    };
    using X1 = std::integral_constant<int, 0xB1>;  // quad_perm [1, 0, 3, 2]
    using X2 = std::integral_constant<int, 0x4E>;  // quad_perm [2, 3, 0, 1]
    const float r01 = xch(o1 ? x[0] : x[1], X1{}), r23 = xch(o1 ? x[2] : x[3], X1{});
    v4f z;
    z[0] = o1 ? r01 : x[0];
    z[1] = o1 ? x[1] : r01;
    z[2] = o1 ? r23 : x[2];
    z[3] = o1 ? x[3] : r23;
    const float r02 = xch(o2 ? z[0] : z[2], X2{}), r13 = xch(o2 ? z[1] : z[3], X2{});
    v4f y;
    y[0] = o2 ? r02 : z[0];
    y[2] = o2 ? z[2] : r02;
    y[1] = o2 ? r13 : z[1];
    y[3] = o2 ? z[3] : r13;
    return y;
}

// four consecutive outputs from fp32 accumulators: 16 bytes (fp32) or 8 bytes (bf16)
__device__ __forceinline__ void store4(float *p, v4f x) {
    *reinterpret_cast<v4f *>(p) = x;
}
__device__ __forceinline__ void store4(bf16_t *p, v4f x) {
    *reinterpret_cast<uint2 *>(p) = pack4u(x);
}

}  // namespace osdn
