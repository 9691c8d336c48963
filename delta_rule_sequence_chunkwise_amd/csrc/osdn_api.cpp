// libosdn host layer: argument validation and kernel dispatch behind the C ABI of osdn.h.
// Every check runs before anything is enqueued; a failed check returns its status and
// touches no memory.
#include <stdint.h>

#include "osdn_internal.h"

namespace {

struct Range {
    uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Range range_of(const void *p, int64_t bytes) {
    Range r;
    if (p && bytes > 0) {
        r.lo = reinterpret_cast<uintptr_t>(p);
        r.hi = r.lo + static_cast<uintptr_t>(bytes);
    }
    return r;
}

bool overlap(const Range &a, const Range &b) {
    return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t n) {
    return (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

// a*b*... without signed overflow; false if the product exceeds `limit`
bool mul_ok(int64_t &acc, int64_t x, int64_t limit) {
    if (x < 0) return false;
    if (x != 0 && acc > limit / x) return false;
    acc *= x;
    return true;
}

int64_t elem_size(osdn_dtype t) { return t == OSDN_BF16 ? 2 : 4; }
bool dtype_ok(osdn_dtype t) { return t == OSDN_F32 || t == OSDN_BF16; }
bool head_dim_ok(int32_t n) { return n == 64 || n == 128; }

// Largest element count any tensor may hold: keeps every byte offset (and every index the
// kernels form in 64-bit arithmetic) far from overflow.
constexpr int64_t kMaxElems = int64_t(1) << 46;

}  // namespace

extern "C" {

const char *osdn_status_string(osdn_status s) {
    switch (s) {
        case OSDN_OK: return "ok";
        case OSDN_ERR_NULL: return "a required pointer is NULL";
        case OSDN_ERR_SHAPE: return "invalid size or element-count overflow";
        case OSDN_ERR_UNSUPPORTED: return "unsupported dk/dv/chunk/dtype combination";
        case OSDN_ERR_ALIGN: return "misaligned pointer";
        case OSDN_ERR_ALIAS: return "output overlaps memory it must not overlap";
        case OSDN_ERR_LAUNCH: return "HIP launch failed";
        case OSDN_ERR_SCRATCH: return "problem needs more scratch than the no-allocation entry point holds";
    }
    return "unknown status";
}

int32_t osdn_abi_version(void) { return OSDN_ABI_VERSION; }

}  // extern "C"

namespace {

int64_t states_bytes(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv, osdn_dtype qkv,
                     int64_t *u_offset);

// The chunkwise forward: validation, then the launch.  With want_states, `states` receives the
// state at every chunk start ([B,H,nchunks,dk,dv]; bf16 for bf16 inputs, else fp32; the
// chunk size is then the backward's) and, for bf16 inputs, the pseudo-values U of every row
// after them.
osdn_status chunk_fwd_impl(const void *q, const void *k, const void *v, const float *beta,
                           const void *d, const float *alpha, const float *S0, void *o,
                           float *S_T, void *states, bool want_states, int64_t B, int64_t H,
                           int64_t T, int32_t dk, int32_t dv, int32_t chunk, osdn_dtype qkv,
                           osdn_dtype d_dtype, void *stream) {
    if (B < 0 || H < 0 || T < 0) return OSDN_ERR_SHAPE;
    if (!dtype_ok(qkv) || !dtype_ok(d_dtype)) return OSDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return OSDN_ERR_UNSUPPORTED;
    if (qkv == OSDN_BF16 ? chunk != 64 : (chunk != 16 && chunk != 32 && chunk != 64))
        return OSDN_ERR_UNSUPPORTED;

    int64_t BH = 1, tok = 1, st = 1;
    if (!mul_ok(BH, B, kMaxElems) || !mul_ok(BH, H, kMaxElems)) return OSDN_ERR_SHAPE;
    tok = BH;
    if (!mul_ok(tok, T, kMaxElems)) return OSDN_ERR_SHAPE;
    int64_t nqk = tok, nv = tok;
    if (!mul_ok(nqk, dk, kMaxElems) || !mul_ok(nv, dv, kMaxElems)) return OSDN_ERR_SHAPE;
    st = BH;
    if (!mul_ok(st, int64_t(dk) * dv, kMaxElems)) return OSDN_ERR_SHAPE;
    if (BH > int64_t(0x7fffffff) / 4) return OSDN_ERR_SHAPE;  // grid: BH x (dv / 32) groups

    int64_t nsb = 0, uoff = 0;  // bytes of the states buffer; where U starts in it
    if (want_states) {
        nsb = states_bytes(B, H, T, dk, dv, qkv, &uoff);
        if (nsb < 0) return OSDN_ERR_SHAPE;
    }

    if (BH == 0) return OSDN_OK;
    if (T > 0 && (!q || !k || !v || !beta || !d || !o || (want_states && !states)))
        return OSDN_ERR_NULL;
    if (T == 0 && !S_T) return OSDN_OK;

    const int64_t eq = elem_size(qkv), ed = elem_size(d_dtype);
    if (T > 0) {
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d, 16) ||
            !aligned(o, 16) || !aligned(beta, 4) || (alpha && !aligned(alpha, 4)) ||
            (want_states && !aligned(states, 16)))
            return OSDN_ERR_ALIGN;
    }
    if ((S0 && !aligned(S0, 16)) || (S_T && !aligned(S_T, 16))) return OSDN_ERR_ALIGN;

    const int64_t n_tok = T > 0 ? tok : 0;
    const Range rq = range_of(q, n_tok ? nqk * eq : 0), rk = range_of(k, n_tok ? nqk * eq : 0);
    const Range rv = range_of(v, n_tok ? nv * eq : 0), rd = range_of(d, n_tok ? nqk * ed : 0);
    const Range rb = range_of(beta, n_tok * 4), ra = range_of(alpha, n_tok * 4);
    const Range rs0 = range_of(S0, st * 4), rst = range_of(S_T, st * 4);
    const Range ro = range_of(o, n_tok ? nv * eq : 0);
    for (const Range *in : {&rq, &rk, &rv, &rd, &rb, &ra, &rs0, &rst})
        if (overlap(ro, *in)) return OSDN_ERR_ALIAS;
    for (const Range *in : {&rq, &rk, &rv, &rd, &rb, &ra})
        if (overlap(rst, *in)) return OSDN_ERR_ALIAS;
    if (overlap(rst, rs0) && (rst.lo != rs0.lo)) return OSDN_ERR_ALIAS;
    const Range rsts = range_of(want_states ? states : nullptr, n_tok ? nsb : 0);
    for (const Range *x : {&rq, &rk, &rv, &rd, &rb, &ra, &rs0, &rst, &ro})
        if (overlap(rsts, *x)) return OSDN_ERR_ALIAS;

    osdn::ChunkArgs a{q, k, v, d, beta, alpha, S0, o, S_T, BH, T, dk, dv, chunk, qkv, d_dtype};
    if (want_states && T > 0) {
        a.ckpt = states;
        if (qkv == OSDN_BF16) a.uout = static_cast<char *>(states) + uoff;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = qkv == OSDN_BF16 ? osdn::launch_chunk_fwd_mfma(a, s)
                                            : osdn::launch_chunk_fwd_f32math(a, s);
    return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

osdn_status osdn_chunk_fwd(const void *q, const void *k, const void *v, const float *beta,
                           const void *d, const float *alpha, const float *S0, void *o,
                           float *S_T, int64_t B, int64_t H, int64_t T, int32_t dk,
                           int32_t dv, int32_t chunk, osdn_dtype qkv, osdn_dtype d_dtype,
                           void *stream) {
    return chunk_fwd_impl(q, k, v, beta, d, alpha, S0, o, S_T, nullptr, false, B, H, T, dk, dv,
                          chunk, qkv, d_dtype, stream);
}

osdn_status osdn_step(const void *q, const void *k, const void *v, const float *beta,
                      const void *d, const float *alpha, float *S, void *o, int64_t B,
                      int64_t H, int32_t dk, int32_t dv, osdn_dtype qkv, osdn_dtype d_dtype,
                      void *stream) {
    if (B < 0 || H < 0) return OSDN_ERR_SHAPE;
    if (!dtype_ok(qkv) || !dtype_ok(d_dtype)) return OSDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return OSDN_ERR_UNSUPPORTED;
    int64_t BH = 1;
    if (!mul_ok(BH, B, kMaxElems) || !mul_ok(BH, H, kMaxElems)) return OSDN_ERR_SHAPE;
    int64_t st = BH;
    if (!mul_ok(st, int64_t(dk) * dv, kMaxElems)) return OSDN_ERR_SHAPE;
    if (BH > int64_t(0x7fffffff)) return OSDN_ERR_SHAPE;
    if (BH == 0) return OSDN_OK;
    if (!q || !k || !v || !beta || !d || !S || !o) return OSDN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d, 16) ||
        !aligned(o, 16) || !aligned(S, 16) || !aligned(beta, 4) ||
        (alpha && !aligned(alpha, 4)))
        return OSDN_ERR_ALIGN;

    const int64_t eq = elem_size(qkv), ed = elem_size(d_dtype);
    const Range rq = range_of(q, BH * dk * eq), rk = range_of(k, BH * dk * eq);
    const Range rv = range_of(v, BH * dv * eq), rd = range_of(d, BH * dk * ed);
    const Range rb = range_of(beta, BH * 4), ra = range_of(alpha, BH * 4);
    const Range rS = range_of(S, st * 4), ro = range_of(o, BH * dv * eq);
    for (const Range *in : {&rq, &rk, &rv, &rd, &rb, &ra, &rS})
        if (overlap(ro, *in)) return OSDN_ERR_ALIAS;
    for (const Range *in : {&rq, &rk, &rv, &rd, &rb, &ra})
        if (overlap(rS, *in)) return OSDN_ERR_ALIAS;

    osdn::StepArgs a{q, k, v, d, beta, alpha, S, o, BH, dk, dv, qkv, d_dtype};
    const hipError_t err = osdn::launch_step(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
}

osdn_status osdn_precond_scan(const void *k, const float *beta, const float *r,
                              const float *d1, float eta, void *d, float *d_next, int64_t B,
                              int64_t H, int64_t T, int32_t dk, int32_t chunk,
                              osdn_dtype k_dtype, osdn_dtype d_dtype, void *stream) {
    if (B < 0 || H < 0 || T < 0) return OSDN_ERR_SHAPE;
    if (!dtype_ok(k_dtype) || !dtype_ok(d_dtype)) return OSDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk)) return OSDN_ERR_UNSUPPORTED;
    if (chunk != 1 && !(chunk == 64 && k_dtype == OSDN_BF16)) return OSDN_ERR_UNSUPPORTED;

    int64_t BH = 1, tok = 1, nk = 1, st = 1;
    if (!mul_ok(BH, B, kMaxElems) || !mul_ok(BH, H, kMaxElems)) return OSDN_ERR_SHAPE;
    tok = BH;
    if (!mul_ok(tok, T, kMaxElems)) return OSDN_ERR_SHAPE;
    nk = tok;
    if (!mul_ok(nk, dk, kMaxElems)) return OSDN_ERR_SHAPE;
    st = BH;
    if (!mul_ok(st, dk, kMaxElems)) return OSDN_ERR_SHAPE;
    if (BH > int64_t(0x7fffffff)) return OSDN_ERR_SHAPE;  // one workgroup per sequence

    if (BH == 0) return OSDN_OK;
    if (T > 0 && (!k || !beta || !d)) return OSDN_ERR_NULL;
    if (T == 0 && !d_next) return OSDN_OK;

    const int64_t ek = elem_size(k_dtype), ed = elem_size(d_dtype);
    if (T > 0) {
        if (!aligned(k, 16) || !aligned(d, 16) || !aligned(beta, 4) || (r && !aligned(r, 4)))
            return OSDN_ERR_ALIGN;
    }
    if ((d1 && !aligned(d1, 16)) || (d_next && !aligned(d_next, 16))) return OSDN_ERR_ALIGN;

    const int64_t n_tok = T > 0 ? tok : 0;
    const Range rk = range_of(k, n_tok ? nk * ek : 0), rd = range_of(d, n_tok ? nk * ed : 0);
    const Range rb = range_of(beta, n_tok * 4), rr = range_of(r, n_tok * 4);
    const Range r1 = range_of(d1, st * 4), rn = range_of(d_next, st * 4);
    for (const Range *in : {&rk, &rb, &rr, &r1, &rn})
        if (overlap(rd, *in)) return OSDN_ERR_ALIAS;
    for (const Range *in : {&rk, &rb, &rr})
        if (overlap(rn, *in)) return OSDN_ERR_ALIAS;
    if (overlap(rn, r1) && rn.lo != r1.lo) return OSDN_ERR_ALIAS;

    osdn::PrecondArgs a{k, beta, r, d1, eta, d, d_next, BH, T, dk, chunk, k_dtype, d_dtype};
    const hipError_t err = osdn::launch_precond(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
}

osdn_status osdn_precond_step(const void *k, const float *beta, const float *r, float *dstate,
                              void *d_out, float eta, int64_t B, int64_t H, int32_t dk,
                              osdn_dtype k_dtype, osdn_dtype d_dtype, void *stream) {
    if (B < 0 || H < 0) return OSDN_ERR_SHAPE;
    if (!dtype_ok(k_dtype) || !dtype_ok(d_dtype)) return OSDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk)) return OSDN_ERR_UNSUPPORTED;
    int64_t BH = 1;
    if (!mul_ok(BH, B, kMaxElems) || !mul_ok(BH, H, kMaxElems)) return OSDN_ERR_SHAPE;
    int64_t st = BH;
    if (!mul_ok(st, dk, kMaxElems)) return OSDN_ERR_SHAPE;
    if (BH > int64_t(0x7fffffff)) return OSDN_ERR_SHAPE;
    if (BH == 0) return OSDN_OK;
    if (!k || !beta || !dstate) return OSDN_ERR_NULL;
    if (!aligned(k, 16) || !aligned(dstate, 16) || (d_out && !aligned(d_out, 16)) ||
        !aligned(beta, 4) || (r && !aligned(r, 4)))
        return OSDN_ERR_ALIGN;

    const int64_t ek = elem_size(k_dtype), ed = elem_size(d_dtype);
    const Range rk = range_of(k, st * ek), rb = range_of(beta, BH * 4), rr = range_of(r, BH * 4);
    const Range rs = range_of(dstate, st * 4), ro = range_of(d_out, st * ed);
    for (const Range *in : {&rk, &rb, &rr, &rs})
        if (overlap(ro, *in)) return OSDN_ERR_ALIAS;
    for (const Range *in : {&rk, &rb, &rr})
        if (overlap(rs, *in)) return OSDN_ERR_ALIAS;

    // one token of the serial scan, reading and writing the state in place
    osdn::PrecondArgs a{k, beta, r, dstate, eta, d_out, dstate, BH, 1, dk, 1, k_dtype, d_dtype};
    const hipError_t err = osdn::launch_precond(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
}

namespace {

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

// byte offsets of the channel-wise gate's workspace (bf16 inputs): the gate-scaled q, k, k~
// ([BH, T, dk] bf16 each), the chunk planes ([BH, nchunks, kda_planes::kElems] bf16) and G_C
// ([BH, nchunks, dk] fp32).  fp32 inputs need none (the fp32 kernel forms the ratios itself).
struct KdaLayout {
    int64_t q, k, kt, planes, g, total;
};

bool kda_layout(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t chunk, osdn_dtype qkv,
                KdaLayout &L) {
    if (B < 0 || H < 0 || T < 0 || !dtype_ok(qkv) || !head_dim_ok(dk)) return false;
    if (qkv == OSDN_BF16 ? chunk != 64 : (chunk != 16 && chunk != 32 && chunk != 64))
        return false;
    int64_t n = 1;
    if (!mul_ok(n, B, kMaxElems) || !mul_ok(n, H, kMaxElems) || !mul_ok(n, T, kMaxElems) ||
        !mul_ok(n, dk, kMaxElems))
        return false;
    int64_t ng = 1, np = 1;
    if (!mul_ok(ng, B, kMaxElems) || !mul_ok(ng, H, kMaxElems) ||
        !mul_ok(ng, (T + chunk - 1) / chunk, kMaxElems))
        return false;
    np = ng;
    if (!mul_ok(ng, dk, kMaxElems) || !mul_ok(np, osdn::kda_planes::kElems, kMaxElems))
        return false;
    L = KdaLayout{};
    if (qkv != OSDN_BF16) return true;
    L.k = round256(n * 2);
    L.kt = L.k + round256(n * 2);
    L.planes = L.kt + round256(n * 2);
    L.g = L.planes + round256(np * 2);
    L.total = L.g + round256(ng * 4);
    return true;
}

}  // namespace

int64_t osdn_chunk_fwd_kda_workspace(int64_t B, int64_t H, int64_t T, int32_t dk,
                                     int32_t chunk, osdn_dtype qkv) {
    KdaLayout L;
    return kda_layout(B, H, T, dk, chunk, qkv, L) ? L.total : -1;
}

osdn_status osdn_chunk_fwd_kda(const void *q, const void *k, const void *v, const float *beta,
                               const void *d, const float *alpha_ch, const float *S0, void *o,
                               float *S_T, void *workspace, int64_t workspace_bytes,
                               int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                               int32_t chunk, osdn_dtype qkv, osdn_dtype d_dtype,
                               void *stream) {
    if (B < 0 || H < 0 || T < 0) return OSDN_ERR_SHAPE;
    if (!dtype_ok(qkv) || !dtype_ok(d_dtype)) return OSDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return OSDN_ERR_UNSUPPORTED;
    if (qkv == OSDN_BF16 ? chunk != 64 : (chunk != 16 && chunk != 32 && chunk != 64))
        return OSDN_ERR_UNSUPPORTED;
    KdaLayout W;
    if (!kda_layout(B, H, T, dk, chunk, qkv, W)) return OSDN_ERR_SHAPE;
    int64_t BH = 1, tok = 1, st = 1;
    if (!mul_ok(BH, B, kMaxElems) || !mul_ok(BH, H, kMaxElems)) return OSDN_ERR_SHAPE;
    tok = BH;
    if (!mul_ok(tok, T, kMaxElems)) return OSDN_ERR_SHAPE;
    int64_t nqk = tok, nv = tok;
    if (!mul_ok(nqk, dk, kMaxElems) || !mul_ok(nv, dv, kMaxElems)) return OSDN_ERR_SHAPE;
    st = BH;
    if (!mul_ok(st, int64_t(dk) * dv, kMaxElems)) return OSDN_ERR_SHAPE;
    if (BH > int64_t(0x7fffffff) / 4) return OSDN_ERR_SHAPE;
    const int64_t nchunks = (T + chunk - 1) / chunk;
    if (BH * nchunks > int64_t(0x7fffffff)) return OSDN_ERR_SHAPE;  // planes grid

    if (BH == 0) return OSDN_OK;
    if (T > 0 && (!q || !k || !v || !beta || !d || !alpha_ch || !o || (W.total > 0 && !workspace)))
        return OSDN_ERR_NULL;
    if (T == 0 && !S_T) return OSDN_OK;
    if (T > 0 && workspace_bytes < W.total) return OSDN_ERR_SHAPE;

    const int64_t eq = elem_size(qkv), ed = elem_size(d_dtype);
    if (T > 0) {
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d, 16) ||
            !aligned(o, 16) || !aligned(beta, 4) || !aligned(alpha_ch, 16) ||
            (W.total > 0 && !aligned(workspace, 256)))
            return OSDN_ERR_ALIGN;
    }
    if ((S0 && !aligned(S0, 16)) || (S_T && !aligned(S_T, 16))) return OSDN_ERR_ALIGN;

    const int64_t n_tok = T > 0 ? tok : 0;
    const Range rq = range_of(q, n_tok ? nqk * eq : 0), rk = range_of(k, n_tok ? nqk * eq : 0);
    const Range rv = range_of(v, n_tok ? nv * eq : 0), rd = range_of(d, n_tok ? nqk * ed : 0);
    const Range rb = range_of(beta, n_tok * 4), ra = range_of(alpha_ch, n_tok ? nqk * 4 : 0);
    const Range rs0 = range_of(S0, st * 4), rst = range_of(S_T, st * 4);
    const Range ro = range_of(o, n_tok ? nv * eq : 0);
    const Range rw = range_of(workspace, T > 0 ? W.total : 0);
    for (const Range *in : {&rq, &rk, &rv, &rd, &rb, &ra, &rs0, &rst})
        if (overlap(ro, *in)) return OSDN_ERR_ALIAS;
    for (const Range *in : {&rq, &rk, &rv, &rd, &rb, &ra})
        if (overlap(rst, *in)) return OSDN_ERR_ALIAS;
    if (overlap(rst, rs0) && (rst.lo != rs0.lo)) return OSDN_ERR_ALIAS;
    for (const Range *in : {&rq, &rk, &rv, &rd, &rb, &ra, &rs0, &rst, &ro})
        if (overlap(rw, *in)) return OSDN_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (qkv != OSDN_BF16) {  // fp32: the kernel forms the exact per-feature ratios itself
        osdn::ChunkArgs a{q, k, v, d, beta, nullptr, S0, o, S_T, BH, T, dk, dv, chunk, qkv,
                          d_dtype};
        a.alpha_ch = alpha_ch;
        const hipError_t err = osdn::launch_chunk_fwd_f32math(a, s);
        return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
    }
    if (T == 0) {  // S_T = S0 (or 0)
        osdn::ChunkArgs a{q, k, v, d, beta, nullptr, S0, o, S_T, BH, T, dk, dv, chunk, qkv,
                          d_dtype};
        const hipError_t err = osdn::launch_chunk_fwd_mfma(a, s);
        return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
    }
    char *ws = static_cast<char *>(workspace);
    float *gcs = reinterpret_cast<float *>(ws + W.g);
    uint16_t *planes = reinterpret_cast<uint16_t *>(ws + W.planes);
    osdn::KdaPrepArgs p{q, k, d, alpha_ch, beta, ws + W.q, ws + W.k, ws + W.kt, planes, gcs,
                        BH, T, nchunks, dk, d_dtype};
    if (osdn::launch_kda_planes(p, s) != hipSuccess) return OSDN_ERR_LAUNCH;
    osdn::ChunkArgs a{ws + W.q, ws + W.k, v, ws + W.kt, beta, nullptr, S0, o, S_T, BH, T, dk,
                      dv, chunk, qkv, OSDN_BF16, gcs};
    a.planes = planes;
    const hipError_t err = osdn::launch_chunk_fwd_mfma(a, s);
    return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
}

osdn_status osdn_step_kda(const void *q, const void *k, const void *v, const float *beta,
                          const void *d, const float *alpha_ch, float *S, void *o, int64_t B,
                          int64_t H, int32_t dk, int32_t dv, osdn_dtype qkv,
                          osdn_dtype d_dtype, void *stream) {
    if (B < 0 || H < 0) return OSDN_ERR_SHAPE;
    if (!dtype_ok(qkv) || !dtype_ok(d_dtype)) return OSDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return OSDN_ERR_UNSUPPORTED;
    int64_t BH = 1;
    if (!mul_ok(BH, B, kMaxElems) || !mul_ok(BH, H, kMaxElems)) return OSDN_ERR_SHAPE;
    int64_t st = BH;
    if (!mul_ok(st, int64_t(dk) * dv, kMaxElems)) return OSDN_ERR_SHAPE;
    if (BH > int64_t(0x7fffffff)) return OSDN_ERR_SHAPE;
    if (BH == 0) return OSDN_OK;
    if (!q || !k || !v || !beta || !d || !alpha_ch || !S || !o) return OSDN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d, 16) ||
        !aligned(o, 16) || !aligned(S, 16) || !aligned(beta, 4) || !aligned(alpha_ch, 4))
        return OSDN_ERR_ALIGN;

    const int64_t eq = elem_size(qkv), ed = elem_size(d_dtype);
    const Range rq = range_of(q, BH * dk * eq), rk = range_of(k, BH * dk * eq);
    const Range rv = range_of(v, BH * dv * eq), rd = range_of(d, BH * dk * ed);
    const Range rb = range_of(beta, BH * 4), ra = range_of(alpha_ch, BH * dk * 4);
    const Range rS = range_of(S, st * 4), ro = range_of(o, BH * dv * eq);
    for (const Range *in : {&rq, &rk, &rv, &rd, &rb, &ra, &rS})
        if (overlap(ro, *in)) return OSDN_ERR_ALIAS;
    for (const Range *in : {&rq, &rk, &rv, &rd, &rb, &ra})
        if (overlap(rS, *in)) return OSDN_ERR_ALIAS;

    osdn::StepArgs a{q, k, v, d, beta, alpha_ch, S, o, BH, dk, dv, qkv, d_dtype};
    const hipError_t err = osdn::launch_step_kda(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// bytes of each of the two state checkpoints of the backward, [BH, nchunks, dk, dv] (bf16 for
// bf16 inputs, fp32 for fp32 inputs); -1 if the sizes are invalid
int64_t bwd_ckpt_bytes(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv, osdn_dtype qkv) {
    if (B < 0 || H < 0 || T < 0 || !dtype_ok(qkv) || !head_dim_ok(dk) || !head_dim_ok(dv))
        return -1;
    const int64_t C = osdn::bwd_chunk_size(qkv);
    int64_t n = 1;
    if (!mul_ok(n, B, kMaxElems) || !mul_ok(n, H, kMaxElems) ||
        !mul_ok(n, (T + C - 1) / C, kMaxElems) || !mul_ok(n, int64_t(dk) * dv, kMaxElems))
        return -1;
    return round256(n * (qkv == OSDN_BF16 ? 2 : 4));
}

// bytes of each per-row buffer of the backward (bf16 inputs: U and dR, bf16, per sequence and
// 64-row chunk dv/16 contiguous 64 x 16 column tiles, the last chunk padded:
// [BH, nchunks, dv/16, 64, 16]; fp32 inputs: none); called after bwd_ckpt_bytes has accepted
// the sizes
int64_t bwd_rows_bytes(int64_t B, int64_t H, int64_t T, int32_t dv, osdn_dtype qkv) {
    if (qkv != OSDN_BF16) return 0;
    const int64_t C = osdn::bwd_chunk_size(qkv);
    int64_t n = 2 * C;
    if (!mul_ok(n, B, kMaxElems) || !mul_ok(n, H, kMaxElems) ||
        !mul_ok(n, (T + C - 1) / C, kMaxElems) || !mul_ok(n, dv, kMaxElems))
        return -1;
    return round256(n);
}

// bytes of the per-chunk planes of the backward (bf16 inputs, per chunk: three bf16 64 x 64
// planes, the inverse's hi and lo and the scores, and K~ as 64 x dk bf16; fp32 inputs: none);
// called after bwd_ckpt_bytes has accepted the sizes
int64_t bwd_tinv_bytes(int64_t B, int64_t H, int64_t T, int32_t dk, osdn_dtype qkv) {
    if (qkv != OSDN_BF16) return 0;
    const int64_t C = osdn::bwd_chunk_size(qkv);
    int64_t n = 1;
    if (!mul_ok(n, B, kMaxElems) || !mul_ok(n, H, kMaxElems) ||
        !mul_ok(n, (T + C - 1) / C, kMaxElems) || !mul_ok(n, 3 * C * C + C * dk, kMaxElems))
        return -1;
    return round256(n * 2);
}

// bytes of the training pair's states buffer: the checkpoints, then (bf16 inputs) U of every
// row from 256 bytes-aligned *u_offset on; -1 if the sizes are invalid
int64_t states_bytes(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv, osdn_dtype qkv,
                     int64_t *u_offset) {
    const int64_t ck = bwd_ckpt_bytes(B, H, T, dk, dv, qkv);
    if (ck < 0) return -1;
    const int64_t ub = bwd_rows_bytes(B, H, T, dv, qkv);
    if (ub < 0) return -1;
    *u_offset = ck;
    return ck + ub;
}

}  // namespace

extern "C" {

int64_t osdn_chunk_bwd_workspace(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                                 osdn_dtype qkv) {
    const int64_t b = bwd_ckpt_bytes(B, H, T, dk, dv, qkv);
    if (b < 0) return -1;
    const int64_t t = bwd_tinv_bytes(B, H, T, dk, qkv);
    if (t < 0) return -1;
    const int64_t u = bwd_rows_bytes(B, H, T, dv, qkv);
    return u < 0 ? -1 : 2 * b + t + 2 * u;
}

int64_t osdn_chunk_bwd_states_workspace(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                                        osdn_dtype qkv) {
    const int64_t b = bwd_ckpt_bytes(B, H, T, dk, dv, qkv);
    if (b < 0) return -1;
    const int64_t t = bwd_tinv_bytes(B, H, T, dk, qkv);
    if (t < 0) return -1;
    const int64_t u = bwd_rows_bytes(B, H, T, dv, qkv);
    return u < 0 ? -1 : b + t + u;
}

}  // extern "C"

namespace {

// The backward: validation, then the launches.  With states_given, `states` holds the state at
// every chunk start from the forward (osdn_chunk_fwd_states) and is not recomputed.
osdn_status chunk_bwd_impl(const void *q, const void *k, const void *v, const float *beta,
                           const void *d, const float *alpha, const float *S0,
                           const void *grad_o, const float *grad_S_T, const void *states,
                           bool states_given, void *grad_q, void *grad_k, void *grad_v,
                           float *grad_beta, void *grad_d, float *grad_alpha, float *grad_S0,
                           void *workspace, int64_t workspace_bytes, int64_t B, int64_t H,
                           int64_t T, int32_t dk, int32_t dv, osdn_dtype qkv,
                           osdn_dtype d_dtype, void *stream) {
    if (B < 0 || H < 0 || T < 0) return OSDN_ERR_SHAPE;
    if (!dtype_ok(qkv) || !dtype_ok(d_dtype)) return OSDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return OSDN_ERR_UNSUPPORTED;
    const int64_t ck = bwd_ckpt_bytes(B, H, T, dk, dv, qkv);
    if (ck < 0) return OSDN_ERR_SHAPE;
    const int64_t tk = bwd_tinv_bytes(B, H, T, dk, qkv);
    if (tk < 0) return OSDN_ERR_SHAPE;
    const int64_t ub = bwd_rows_bytes(B, H, T, dv, qkv);
    if (ub < 0) return OSDN_ERR_SHAPE;
    // workspace: [M0 checkpoints] dMC checkpoints, chunk planes, [U] dR; the bracketed parts
    // only when the states are not given (they are then the caller's)
    const int64_t m0b = states_given ? 0 : ck, u0b = states_given ? 0 : ub;
    const int64_t wsb = m0b + ck + tk + u0b + ub;
    int64_t BH = 1;
    if (!mul_ok(BH, B, kMaxElems) || !mul_ok(BH, H, kMaxElems)) return OSDN_ERR_SHAPE;
    int64_t tok = BH, st = BH;
    if (!mul_ok(tok, T, kMaxElems) || !mul_ok(st, int64_t(dk) * dv, kMaxElems))
        return OSDN_ERR_SHAPE;
    int64_t nqk = tok, nv = tok;
    if (!mul_ok(nqk, dk, kMaxElems) || !mul_ok(nv, dv, kMaxElems)) return OSDN_ERR_SHAPE;
    const int64_t C = osdn::bwd_chunk_size(qkv), nch = (T + C - 1) / C;
    if (BH * nch > int64_t(0x7fffffff) || BH * (dv / 32) > int64_t(0x7fffffff))
        return OSDN_ERR_SHAPE;  // grid sizes

    if (BH == 0) return OSDN_OK;
    if (T > 0 && (!q || !k || !v || !beta || !d || !grad_o || !grad_q || !grad_k || !grad_v ||
                  !grad_beta || !grad_d || !workspace || (states_given && !states)))
        return OSDN_ERR_NULL;
    if (T == 0 && !grad_S0) return OSDN_OK;
    if (T > 0 && workspace_bytes < wsb) return OSDN_ERR_SHAPE;
    if (!alpha) grad_alpha = nullptr;

    const int64_t eq = elem_size(qkv), ed = elem_size(d_dtype);
    if (T > 0) {
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d, 16) ||
            !aligned(grad_o, 16) || !aligned(grad_q, 16) || !aligned(grad_k, 16) ||
            !aligned(grad_v, 16) || !aligned(grad_d, 16) || !aligned(beta, 4) ||
            !aligned(grad_beta, 4) || (alpha && !aligned(alpha, 4)) ||
            (grad_alpha && !aligned(grad_alpha, 4)) || !aligned(workspace, 256) ||
            (states_given && !aligned(states, 16)))
            return OSDN_ERR_ALIGN;
    }
    if ((S0 && !aligned(S0, 16)) || (grad_S_T && !aligned(grad_S_T, 16)) ||
        (grad_S0 && !aligned(grad_S0, 16)))
        return OSDN_ERR_ALIGN;

    const int64_t nt = T > 0 ? tok : 0;
    const Range rq = range_of(q, nt ? nqk * eq : 0), rk = range_of(k, nt ? nqk * eq : 0);
    const Range rv = range_of(v, nt ? nv * eq : 0), rd = range_of(d, nt ? nqk * ed : 0);
    const Range rb = range_of(beta, nt * 4), ra = range_of(alpha, alpha ? nt * 4 : 0);
    const Range rs0 = range_of(S0, st * 4), rgo = range_of(grad_o, nt ? nv * eq : 0);
    const Range rgst = range_of(grad_S_T, st * 4);
    int64_t nsb = 0, uoff = 0;  // bytes of the forward's states buffer; where U starts in it
    if (states_given) {
        nsb = states_bytes(B, H, T, dk, dv, qkv, &uoff);
        if (nsb < 0) return OSDN_ERR_SHAPE;
    }
    const Range rsts = range_of(states_given ? states : nullptr, nt ? nsb : 0);
    const Range gq = range_of(grad_q, nt ? nqk * eq : 0), gk = range_of(grad_k, nt ? nqk * eq : 0);
    const Range gv = range_of(grad_v, nt ? nv * eq : 0), gd = range_of(grad_d, nt ? nqk * ed : 0);
    const Range gb = range_of(grad_beta, nt * 4), ga = range_of(grad_alpha, grad_alpha ? nt * 4 : 0);
    const Range gs0 = range_of(grad_S0, st * 4);
    const Range rw = range_of(workspace, T > 0 ? wsb : 0);
    const Range *outs[] = {&gq, &gk, &gv, &gd, &gb, &ga, &gs0, &rw};
    const Range *ins[] = {&rq, &rk, &rv, &rd, &rb, &ra, &rs0, &rgo, &rgst, &rsts};
    for (int i = 0; i < 8; ++i) {
        for (const Range *in : ins)
            if (overlap(*outs[i], *in)) return OSDN_ERR_ALIAS;
        for (int j = i + 1; j < 8; ++j)
            if (overlap(*outs[i], *outs[j])) return OSDN_ERR_ALIAS;
    }

    char *ws = static_cast<char *>(workspace);
    char *sts = static_cast<char *>(const_cast<void *>(states));
    osdn::BwdArgs a{q, k, v, d, beta, alpha, S0, grad_o, grad_S_T, grad_q, grad_k, grad_v,
                    grad_beta, grad_alpha, grad_d, grad_S0,
                    T > 0 ? (states_given ? static_cast<void *>(sts) : ws) : nullptr,
                    T > 0 ? ws + m0b : nullptr, states_given,
                    T > 0 && tk > 0 ? reinterpret_cast<uint16_t *>(ws + m0b + ck) : nullptr,
                    T > 0 && ub > 0
                        ? reinterpret_cast<uint16_t *>(states_given ? sts + uoff
                                                                    : ws + m0b + ck + tk)
                        : nullptr,
                    T > 0 && ub > 0 ? reinterpret_cast<uint16_t *>(ws + m0b + ck + tk + u0b)
                                    : nullptr,
                    BH, T, dk, dv, qkv, d_dtype};
    const hipError_t err = osdn::launch_chunk_bwd(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

osdn_status osdn_chunk_bwd(const void *q, const void *k, const void *v, const float *beta,
                           const void *d, const float *alpha, const float *S0,
                           const void *grad_o, const float *grad_S_T, void *grad_q,
                           void *grad_k, void *grad_v, float *grad_beta, void *grad_d,
                           float *grad_alpha, float *grad_S0, void *workspace,
                           int64_t workspace_bytes, int64_t B, int64_t H, int64_t T, int32_t dk,
                           int32_t dv, osdn_dtype qkv, osdn_dtype d_dtype, void *stream) {
    return chunk_bwd_impl(q, k, v, beta, d, alpha, S0, grad_o, grad_S_T, nullptr, false, grad_q,
                          grad_k, grad_v, grad_beta, grad_d, grad_alpha, grad_S0, workspace,
                          workspace_bytes, B, H, T, dk, dv, qkv, d_dtype, stream);
}

int64_t osdn_chunk_states_bytes(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                                osdn_dtype qkv) {
    int64_t uoff = 0;
    return states_bytes(B, H, T, dk, dv, qkv, &uoff);
}

osdn_status osdn_chunk_fwd_states(const void *q, const void *k, const void *v,
                                  const float *beta, const void *d, const float *alpha,
                                  const float *S0, void *o, float *S_T, void *states, int64_t B,
                                  int64_t H, int64_t T, int32_t dk, int32_t dv, osdn_dtype qkv,
                                  osdn_dtype d_dtype, void *stream) {
    if (!dtype_ok(qkv)) return OSDN_ERR_UNSUPPORTED;
    return chunk_fwd_impl(q, k, v, beta, d, alpha, S0, o, S_T, states, true, B, H, T, dk, dv,
                          osdn::bwd_chunk_size(qkv), qkv, d_dtype, stream);
}

osdn_status osdn_chunk_bwd_states(const void *q, const void *k, const void *v,
                                  const float *beta, const void *d, const float *alpha,
                                  const float *S0, const void *states, const void *grad_o,
                                  const float *grad_S_T, void *grad_q, void *grad_k,
                                  void *grad_v, float *grad_beta, void *grad_d,
                                  float *grad_alpha, float *grad_S0, void *workspace,
                                  int64_t workspace_bytes, int64_t B, int64_t H, int64_t T,
                                  int32_t dk, int32_t dv, osdn_dtype qkv, osdn_dtype d_dtype,
                                  void *stream) {
    return chunk_bwd_impl(q, k, v, beta, d, alpha, S0, grad_o, grad_S_T, states, true, grad_q,
                          grad_k, grad_v, grad_beta, grad_d, grad_alpha, grad_S0, workspace,
                          workspace_bytes, B, H, T, dk, dv, qkv, d_dtype, stream);
}

}  // extern "C"

namespace {

constexpr int64_t kGateBwdChunk = 32;  // rows per chunk of the channel-wise gate's backward

// bytes of each of the two fp32 checkpoints of the channel-wise gate's backward,
// [BH, nchunks, dk, dv]; -1 if the sizes are invalid
int64_t bwd_gate_ckpt_bytes(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                            osdn_dtype qkv) {
    if (B < 0 || H < 0 || T < 0 || !dtype_ok(qkv) || !head_dim_ok(dk) || !head_dim_ok(dv))
        return -1;
    int64_t n = 4;
    if (!mul_ok(n, B, kMaxElems) || !mul_ok(n, H, kMaxElems) ||
        !mul_ok(n, (T + kGateBwdChunk - 1) / kGateBwdChunk, kMaxElems) ||
        !mul_ok(n, int64_t(dk) * dv, kMaxElems))
        return -1;
    return round256(n);
}

// bytes of the channel-wise gate backward's score tiles AS and P of every chunk,
// [BH, nchunks, 2, C, C] fp32 (valid sizes assumed: checked by bwd_gate_ckpt_bytes)
int64_t bwd_gate_score_bytes(int64_t B, int64_t H, int64_t T) {
    return round256(B * H * ((T + kGateBwdChunk - 1) / kGateBwdChunk) * 3 * kGateBwdChunk *
                    kGateBwdChunk * 4);  // AS, P and T of every chunk
}

}  // namespace

extern "C" {

int64_t osdn_chunk_bwd_kda_workspace(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                                     osdn_dtype qkv) {
    const int64_t b = bwd_gate_ckpt_bytes(B, H, T, dk, dv, qkv);
    return b < 0 ? -1 : 2 * b + bwd_gate_score_bytes(B, H, T);
}

osdn_status osdn_chunk_bwd_kda(const void *q, const void *k, const void *v, const float *beta,
                               const void *d, const float *alpha_ch, const float *S0,
                               const void *grad_o, const float *grad_S_T, void *grad_q,
                               void *grad_k, void *grad_v, float *grad_beta, void *grad_d,
                               float *grad_alpha_ch, float *grad_S0, void *workspace,
                               int64_t workspace_bytes, int64_t B, int64_t H, int64_t T,
                               int32_t dk, int32_t dv, osdn_dtype qkv, osdn_dtype d_dtype,
                               void *stream) {
    if (B < 0 || H < 0 || T < 0) return OSDN_ERR_SHAPE;
    if (!dtype_ok(qkv) || !dtype_ok(d_dtype)) return OSDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return OSDN_ERR_UNSUPPORTED;
    const int64_t ck = bwd_gate_ckpt_bytes(B, H, T, dk, dv, qkv);
    if (ck < 0) return OSDN_ERR_SHAPE;
    const int64_t wsb = 2 * ck + bwd_gate_score_bytes(B, H, T);
    int64_t BH = 1;
    if (!mul_ok(BH, B, kMaxElems) || !mul_ok(BH, H, kMaxElems)) return OSDN_ERR_SHAPE;
    int64_t tok = BH, st = BH;
    if (!mul_ok(tok, T, kMaxElems) || !mul_ok(st, int64_t(dk) * dv, kMaxElems))
        return OSDN_ERR_SHAPE;
    int64_t nqk = tok, nv = tok;
    if (!mul_ok(nqk, dk, kMaxElems) || !mul_ok(nv, dv, kMaxElems)) return OSDN_ERR_SHAPE;
    const int64_t nch = (T + kGateBwdChunk - 1) / kGateBwdChunk;
    if (BH * nch > int64_t(0x7fffffff) || BH * (dv / 32) > int64_t(0x7fffffff))
        return OSDN_ERR_SHAPE;  // grid sizes

    if (BH == 0) return OSDN_OK;
    if (T > 0 && (!q || !k || !v || !beta || !d || !alpha_ch || !grad_o || !grad_q || !grad_k ||
                  !grad_v || !grad_beta || !grad_d || !workspace))
        return OSDN_ERR_NULL;
    if (T == 0 && !grad_S0) return OSDN_OK;
    if (T > 0 && workspace_bytes < wsb) return OSDN_ERR_SHAPE;

    const int64_t eq = elem_size(qkv), ed = elem_size(d_dtype);
    if (T > 0) {
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d, 16) ||
            !aligned(grad_o, 16) || !aligned(grad_q, 16) || !aligned(grad_k, 16) ||
            !aligned(grad_v, 16) || !aligned(grad_d, 16) || !aligned(beta, 4) ||
            !aligned(alpha_ch, 16) || !aligned(grad_beta, 4) ||
            (grad_alpha_ch && !aligned(grad_alpha_ch, 4)) || !aligned(workspace, 256))
            return OSDN_ERR_ALIGN;
    }
    if ((S0 && !aligned(S0, 16)) || (grad_S_T && !aligned(grad_S_T, 16)) ||
        (grad_S0 && !aligned(grad_S0, 16)))
        return OSDN_ERR_ALIGN;

    const int64_t nt = T > 0 ? tok : 0;
    const Range rq = range_of(q, nt ? nqk * eq : 0), rk = range_of(k, nt ? nqk * eq : 0);
    const Range rv = range_of(v, nt ? nv * eq : 0), rd = range_of(d, nt ? nqk * ed : 0);
    const Range rb = range_of(beta, nt * 4), ra = range_of(alpha_ch, nt ? nqk * 4 : 0);
    const Range rs0 = range_of(S0, st * 4), rgo = range_of(grad_o, nt ? nv * eq : 0);
    const Range rgst = range_of(grad_S_T, st * 4);
    const Range gq = range_of(grad_q, nt ? nqk * eq : 0), gk = range_of(grad_k, nt ? nqk * eq : 0);
    const Range gv = range_of(grad_v, nt ? nv * eq : 0), gd = range_of(grad_d, nt ? nqk * ed : 0);
    const Range gb = range_of(grad_beta, nt * 4);
    const Range ga = range_of(grad_alpha_ch, grad_alpha_ch && nt ? nqk * 4 : 0);
    const Range gs0 = range_of(grad_S0, st * 4);
    const Range rw = range_of(workspace, T > 0 ? wsb : 0);
    const Range *outs[] = {&gq, &gk, &gv, &gd, &gb, &ga, &gs0, &rw};
    const Range *ins[] = {&rq, &rk, &rv, &rd, &rb, &ra, &rs0, &rgo, &rgst};
    for (int i = 0; i < 8; ++i) {
        for (const Range *in : ins)
            if (overlap(*outs[i], *in)) return OSDN_ERR_ALIAS;
        for (int j = i + 1; j < 8; ++j)
            if (overlap(*outs[i], *outs[j])) return OSDN_ERR_ALIAS;
    }

    char *ws = static_cast<char *>(workspace);
    osdn::BwdArgs a{q, k, v, d, beta, nullptr, S0, grad_o, grad_S_T, grad_q, grad_k, grad_v,
                    grad_beta, nullptr, grad_d, grad_S0,
                    T > 0 ? static_cast<void *>(ws) : nullptr, T > 0 ? ws + ck : nullptr, false,
                    nullptr, nullptr, nullptr, BH, T, dk, dv, qkv, d_dtype};
    a.alpha_ch = alpha_ch;
    a.galpha_ch = grad_alpha_ch;
    a.scores = T > 0 ? reinterpret_cast<float *>(ws + 2 * ck) : nullptr;
    const hipError_t err = osdn::launch_chunk_bwd_gate(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? OSDN_OK : OSDN_ERR_LAUNCH;
}

}  // extern "C"
