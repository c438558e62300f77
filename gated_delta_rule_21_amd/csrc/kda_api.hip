// kda_api.hip -- the extern "C" entry points declared in include/kda.h:
// argument checks, the prefill workspace plan, and kernel launches on the
// caller's stream.  Nothing here allocates device memory or synchronises,
// except the opt-in cu_seqlens check (KDA_DEBUG_CHECK_CU=1).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

static_assert(KDA_MAX_PREFILL_SEGMENTS == kda::kMaxSegments, "segment limit");
static_assert(KDA_MAX_DECODE_WINDOW == kda::kMaxWindow, "window limit");

namespace {

bool supported_dim(int dk, int dv) { return dk == dv && (dk == 32 || dk == 64 || dk == 128); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t io_size(kda_dtype t) { return t == KDA_F32 ? 4 : 2; }

// [a, a + na) and [b, b + nb) overlap (byte ranges); empty ranges never do.
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool debug_check_cu() {
    const char *e = std::getenv("KDA_DEBUG_CHECK_CU");
    return e && e[0] == '1';
}

}  // namespace

extern "C" {

const char *kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case KDA_ERR_NULL_POINTER: return "required pointer is NULL";
        case KDA_ERR_UNSUPPORTED_DIM: return "unsupported head dim (need dk == dv in {32, 64, 128})";
        case KDA_ERR_UNSUPPORTED_DTYPE: return "unsupported io dtype";
        case KDA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case KDA_ERR_HIP: return "HIP kernel launch failed";
        case KDA_ERR_ALIAS: return "output overlaps an input";
        case KDA_ERR_SCRATCH_TOO_SMALL: return "sizes need more workspace than the no-alloc scratch holds";
    }
    return "unknown kda status";
}

const char *kda_build_info(void) {
    return "kda gfx950: chunk 64, bf16 MFMA 16x16x32 with split-precision operands, "
           "fp32 MFMA 16x16x4, d in {32,64,128}";
}

}  // extern "C"

namespace {

// Segment count of a call: the caller's, or the automatic choice (0).
// -1 for an out-of-range request.
int segments_of(const kda_prefill_options *opt, int N, int T, int H, int d) {
    const int s = opt ? opt->segments : 0;
    if (s < 0 || s > KDA_MAX_PREFILL_SEGMENTS) return -1;
    return s > 0 ? s : kda::choose_segments(N, T, H, d);
}

bool checkpoints_requested(const kda_prefill_options *opt) {
    return opt && (opt->checkpoints || opt->checkpoint_offsets);
}

// Chunk blocks of a call: the caller's, or the automatic choice (0); 1 where
// the pipeline does not apply (fp32 path, segments, checkpoints).  -1 for an
// out-of-range request or one that conflicts with forced segments.
int blocks_of(const kda_prefill_options *opt, int N, int T, int H, int d, bool f32io, int P, bool fused = false) {
    const int b = opt ? opt->blocks : 0;
    if (b < 0 || b > KDA_MAX_PREFILL_BLOCKS) return -1;
    if (b > 1 && opt->segments > 1) return -1;
    if (f32io || P > 1 || checkpoints_requested(opt)) return 1;
    return b > 0 ? b : kda::choose_blocks(N, T, H, d, fused);
}

// Segment count of a call once forced blocks are taken into account: on the
// bf16 path without checkpoints, blocks >= 2 with automatic segments mean one
// segment.
int segments_with_blocks(const kda_prefill_options *opt, int N, int T, int H, int d, bool f32io) {
    if (opt && opt->blocks > 1 && opt->segments == 0 && !f32io && !checkpoints_requested(opt)) return 1;
    return segments_of(opt, N, T, H, d);
}

size_t prefill_ws(int N, int T, int H, int dk, int dv, kda_dtype io_dtype, const kda_prefill_options *opt,
                  bool fused = false) {
    if (io_dtype != KDA_BF16 && io_dtype != KDA_F32) return 0;
    if (!supported_dim(dk, dv) || N < 0 || T < 0 || H <= 0) return 0;
    const int P = segments_with_blocks(opt, N, T, H, dk, io_dtype == KDA_F32);
    if (P < 1) return 0;
    const int B = blocks_of(opt, N, T, H, dk, io_dtype == KDA_F32, P, fused);
    if (B < 1) return 0;
    kda::PrefillPlan p;
    if (!kda::plan_prefill(N, T, H, dk, dv, io_dtype == KDA_F32, P, B, &p, fused)) return 0;
    return p.total;
}

}  // namespace

extern "C" {

size_t kda_prefill_workspace_size(int N, int T, int H, int dk, int dv, kda_dtype io_dtype) {
    return prefill_ws(N, T, H, dk, dv, io_dtype, nullptr);
}

size_t kda_prefill_ex_workspace_size(int N, int T, int H, int dk, int dv, kda_dtype io_dtype,
                                     const kda_prefill_options *options) {
    if (checkpoints_requested(options) &&
        (options->checkpoint_interval <= 0 || options->checkpoint_interval % 64 != 0))
        return 0;
    return prefill_ws(N, T, H, dk, dv, io_dtype, options);
}

size_t kda_prefill_fused_workspace_size(int N, int T, int H, int dk, int dv, kda_dtype io_dtype,
                                        const kda_prefill_options *options) {
    if (io_dtype != KDA_BF16) return 0;
    if (checkpoints_requested(options) || (options && options->checkpoint_interval != 0)) return 0;
    return prefill_ws(N, T, H, dk, dv, io_dtype, options, true);
}

int kda_prefill_segments(int N, int T, int H, int dk, int dv, kda_dtype io_dtype) {
    if (io_dtype != KDA_BF16 && io_dtype != KDA_F32) return 0;
    if (!supported_dim(dk, dv) || N < 0 || T < 0 || H <= 0) return 0;
    return kda::choose_segments(N, T, H, dk);
}

}  // extern "C"

namespace {

int prefill_impl(kda_dtype io_dtype, const void *q, const void *k, const void *v, const float *z,
                 const float *A, const float *beta, const float *h0, const int32_t *cu_seqlens, int N,
                 int T, int H, int dk, int dv, void *o, float *hT, const kda_prefill_options *opt,
                 void *workspace, size_t workspace_bytes, void *stream, const kda::FusedIO *fx = nullptr) {
    if (io_dtype != KDA_BF16 && io_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED_DTYPE;
    float *ck = opt ? opt->checkpoints : nullptr;
    int32_t *ck_offsets = opt ? opt->checkpoint_offsets : nullptr;
    const int interval = (ck || ck_offsets) ? opt->checkpoint_interval : 0;
    if ((ck || ck_offsets) && (interval <= 0 || interval % 64 != 0)) return KDA_ERR_INVALID_ARGUMENT;
    const int P = segments_with_blocks(opt, N, T, H, dk, io_dtype == KDA_F32);
    if (P < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (N < 0 || T < 0 || H <= 0) return KDA_ERR_INVALID_ARGUMENT;
    const int B = blocks_of(opt, N, T, H, dk, io_dtype == KDA_F32, P, fx != nullptr);
    if (B < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(dk, dv)) return KDA_ERR_UNSUPPORTED_DIM;
    if (!A || !cu_seqlens || !workspace) return KDA_ERR_NULL_POINTER;
    if (T > 0 && (!z || !beta || !o)) return KDA_ERR_NULL_POINTER;
    if (T > 0 && !fx && (!q || !k || !v)) return KDA_ERR_NULL_POINTER;
    const void *ptrs[] = {q, k, v, z, A, beta, h0, cu_seqlens, o, hT, ck, ck_offsets};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_MISALIGNED;

    kda::PrefillPlan plan;
    if (!kda::plan_prefill(N, T, H, dk, dv, io_dtype == KDA_F32, P, B, &plan, fx != nullptr))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < plan.total) return KDA_ERR_WORKSPACE_TOO_SMALL;

    const size_t tok = (size_t)T * H;
    const size_t o_bytes = tok * dv * io_size(io_dtype);
    const size_t st_bytes = (size_t)N * H * dv * dk * 4;
    const struct { const void *p; size_t n; } ins[] = {
        {q, tok * dk * io_size(io_dtype)}, {k, tok * dk * io_size(io_dtype)},
        {v, tok * dv * io_size(io_dtype)}, {z, tok * dk * 4}, {A, (size_t)H * 4},
        {beta, tok * 4}, {cu_seqlens, (size_t)(N + 1) * 4}, {h0, st_bytes},
        {workspace, plan.total}};
    for (const auto &in : ins) {
        if (overlaps(o, o_bytes, in.p, in.n)) return KDA_ERR_ALIAS;
        if (in.p != h0 && overlaps(hT, st_bytes, in.p, in.n)) return KDA_ERR_ALIAS;
    }
    if (fx) {
        // the fused call's inputs and the conv window it writes
        const size_t xb = tok * dk * io_size(io_dtype), wb = (size_t)H * dk * 16;
        const size_t win_bytes = (size_t)N * 3 * H * 3 * dk * io_size(io_dtype);
        const struct { const void *p; size_t n; } fin[] = {
            {fx->xq, xb}, {fx->xk, xb}, {fx->xv, xb}, {fx->wq, wb}, {fx->wk, wb}, {fx->wv, wb},
            {fx->win_in, win_bytes}, {fx->g, o_bytes}, {fx->w, (size_t)dv * 4}};
        for (const auto &in : fin) {
            if (overlaps(o, o_bytes, in.p, in.n) || overlaps(hT, st_bytes, in.p, in.n)) return KDA_ERR_ALIAS;
            if (!(in.p == fx->win_in && fx->win_out == fx->win_in) && overlaps(fx->win_out, win_bytes, in.p, in.n))
                return KDA_ERR_ALIAS;
        }
        for (const auto &in : ins)
            if (overlaps(fx->win_out, win_bytes, in.p, in.n)) return KDA_ERR_ALIAS;
        if (overlaps(fx->win_out, win_bytes, o, o_bytes) || overlaps(fx->win_out, win_bytes, hT, st_bytes))
            return KDA_ERR_ALIAS;
    }
    if (hT && h0 && hT != h0 && overlaps(hT, st_bytes, h0, st_bytes)) return KDA_ERR_ALIAS;
    if (overlaps(o, o_bytes, hT, st_bytes)) return KDA_ERR_ALIAS;
    // checkpoints and their offsets overlap nothing else
    const size_t ck_bytes = interval > 0 ? (size_t)(T / interval) * H * dv * dk * 4 : 0;
    const size_t off_bytes = (size_t)(N + 1) * 4;
    for (const auto &in : ins)
        if (overlaps(ck, ck_bytes, in.p, in.n) || overlaps(ck_offsets, off_bytes, in.p, in.n)) return KDA_ERR_ALIAS;
    if (overlaps(ck, ck_bytes, o, o_bytes) || overlaps(ck, ck_bytes, hT, st_bytes) ||
        overlaps(ck_offsets, off_bytes, o, o_bytes) || overlaps(ck_offsets, off_bytes, hT, st_bytes) ||
        overlaps(ck, ck_bytes, ck_offsets, off_bytes))
        return KDA_ERR_ALIAS;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (debug_check_cu()) {
        std::vector<int32_t> cu(N + 1);
        if (hipMemcpyAsync(cu.data(), cu_seqlens, sizeof(int32_t) * (N + 1), hipMemcpyDeviceToHost,
                           st) != hipSuccess ||
            hipStreamSynchronize(st) != hipSuccess)
            return KDA_ERR_HIP;
        if (cu[0] != 0 || cu[N] != T) return KDA_ERR_INVALID_ARGUMENT;
        for (int n = 0; n < N; ++n)
            if (cu[n + 1] < cu[n]) return KDA_ERR_INVALID_ARGUMENT;
    }

    kda::PrefillArgs a;
    a.f32io = io_dtype == KDA_F32;
    a.q = q; a.k = k; a.v = v; a.z = z; a.A = A; a.beta = beta; a.h0 = h0;
    a.cu = cu_seqlens;
    a.N = N; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
    a.o = o; a.hT = hT;
    a.ck = ck_bytes > 0 ? ck : nullptr;
    a.ck_offsets = ck_offsets;
    a.ck_interval = interval;
    a.ws = static_cast<unsigned char *>(workspace);
    a.plan = plan;
    a.stream = st;
    a.fused = fx;
    return kda::launch_prefill(a) == 0 ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int kda_prefill(kda_dtype io_dtype, const void *q, const void *k, const void *v, const float *z,
                const float *A, const float *beta, const float *h0, const int32_t *cu_seqlens,
                int N, int T, int H, int dk, int dv, void *o, float *hT, void *workspace,
                size_t workspace_bytes, void *stream) {
    return prefill_impl(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o, hT, nullptr,
                        workspace, workspace_bytes, stream);
}

int kda_prefill_ex(kda_dtype io_dtype, const void *q, const void *k, const void *v, const float *z,
                   const float *A, const float *beta, const float *h0, const int32_t *cu_seqlens, int N,
                   int T, int H, int dk, int dv, void *o, float *hT, const kda_prefill_options *options,
                   void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o, hT, options,
                        workspace, workspace_bytes, stream);
}

int kda_prefill_fused(kda_dtype io_dtype, const void *xq, const void *xk, const void *xv, const float *wq,
                      const float *wk, const float *wv, const void *conv_state_in, void *conv_state_out,
                      const float *z, const float *A, const float *beta, const float *h0, const int32_t *cu_seqlens,
                      int N, int T, int H, int dk, int dv, const void *gate, const float *norm_weight, float eps,
                      void *y, float *hT, void *workspace, size_t workspace_bytes, void *stream) {
    return kda_prefill_fused_ex(io_dtype, xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, z, A, beta, h0,
                                cu_seqlens, N, T, H, dk, dv, gate, norm_weight, eps, y, hT, nullptr, workspace,
                                workspace_bytes, stream);
}

int kda_prefill_fused_ex(kda_dtype io_dtype, const void *xq, const void *xk, const void *xv, const float *wq,
                         const float *wk, const float *wv, const void *conv_state_in, void *conv_state_out,
                         const float *z, const float *A, const float *beta, const float *h0,
                         const int32_t *cu_seqlens, int N, int T, int H, int dk, int dv, const void *gate,
                         const float *norm_weight, float eps, void *y, float *hT, const kda_prefill_options *options,
                         void *workspace, size_t workspace_bytes, void *stream) {
    if (io_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED_DTYPE;
    // the gated output mode stores no state checkpoints
    if (checkpoints_requested(options) || (options && options->checkpoint_interval != 0))
        return KDA_ERR_INVALID_ARGUMENT;
    if (N < 0 || T < 0 || H <= 0 || !(eps >= 0.f)) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(dk, dv)) return KDA_ERR_UNSUPPORTED_DIM;
    if (!wq || !wk || !wv || !norm_weight) return KDA_ERR_NULL_POINTER;
    if (T > 0 && (!xq || !xk || !xv || !gate)) return KDA_ERR_NULL_POINTER;
    const void *ptrs[] = {xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, gate, norm_weight};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    kda::FusedIO fx;
    fx.xq = xq; fx.xk = xk; fx.xv = xv;
    fx.wq = wq; fx.wk = wk; fx.wv = wv;
    fx.win_in = conv_state_in; fx.win_out = conv_state_out;
    fx.g = gate; fx.w = norm_weight; fx.eps = eps;
    return prefill_impl(io_dtype, nullptr, nullptr, nullptr, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, y, hT,
                        options, workspace, workspace_bytes, stream, &fx);
}

size_t kda_prefill_backward_workspace_size(int N, int T, int H, int dk, int dv, kda_dtype io_dtype,
                                           const kda_prefill_options *options) {
    if (io_dtype != KDA_BF16 && io_dtype != KDA_F32) return 0;
    if (!supported_dim(dk, dv) || N < 0 || T < 0 || H <= 0) return 0;
    if (checkpoints_requested(options) || (options && options->checkpoint_interval != 0)) return 0;
    const int P = segments_of(options, N, T, H, dk);
    if (P < 1) return 0;
    kda::BackwardPlan p;
    if (!kda::plan_backward(N, T, H, dk, io_dtype == KDA_F32, P, &p)) return 0;
    return p.total;
}

int kda_prefill_backward(kda_dtype io_dtype, const void *q, const void *k, const void *v, const float *z,
                         const float *A, const float *beta, const float *h0, const int32_t *cu_seqlens,
                         int N, int T, int H, int dk, int dv, const void *grad_o, const float *grad_hT,
                         float *grad_q, float *grad_k, float *grad_v, float *grad_z, float *grad_beta,
                         float *grad_A, float *grad_h0, const kda_prefill_options *options, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (io_dtype != KDA_BF16 && io_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED_DTYPE;
    if (N < 0 || T < 0 || H <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (checkpoints_requested(options) || (options && options->checkpoint_interval != 0))
        return KDA_ERR_INVALID_ARGUMENT;
    const int P = segments_of(options, N, T, H, dk);
    if (P < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(dk, dv)) return KDA_ERR_UNSUPPORTED_DIM;
    if (!A || !cu_seqlens || !workspace || !grad_A) return KDA_ERR_NULL_POINTER;
    if (T > 0 && (!q || !k || !v || !z || !beta || !grad_o || !grad_q || !grad_k || !grad_v || !grad_z ||
                  !grad_beta))
        return KDA_ERR_NULL_POINTER;
    const void *ptrs[] = {q, k, v, z, A, beta, h0, cu_seqlens, grad_o, grad_hT, grad_q, grad_k,
                          grad_v, grad_z, grad_beta, grad_A, grad_h0};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_MISALIGNED;

    kda::BackwardPlan plan;
    if (!kda::plan_backward(N, T, H, dk, io_dtype == KDA_F32, P, &plan)) return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < plan.total) return KDA_ERR_WORKSPACE_TOO_SMALL;

    // every output overlaps no input, no workspace and no other output
    const size_t tok = (size_t)T * H, io = io_size(io_dtype);
    const size_t st_bytes = (size_t)N * H * dv * dk * 4;
    const struct { const void *p; size_t n; } ins[] = {
        {q, tok * dk * io}, {k, tok * dk * io}, {v, tok * dv * io}, {z, tok * dk * 4},
        {A, (size_t)H * 4}, {beta, tok * 4}, {cu_seqlens, (size_t)(N + 1) * 4}, {h0, st_bytes},
        {grad_o, tok * dv * io}, {grad_hT, st_bytes}, {workspace, plan.total}};
    const struct { const void *p; size_t n; } outs[] = {
        {grad_q, tok * dk * 4}, {grad_k, tok * dk * 4}, {grad_v, tok * dv * 4}, {grad_z, tok * dk * 4},
        {grad_beta, tok * 4}, {grad_A, (size_t)H * 4}, {grad_h0, st_bytes}};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const auto &in : ins)
            if (overlaps(outs[i].p, outs[i].n, in.p, in.n)) return KDA_ERR_ALIAS;
        for (size_t j = 0; j < i; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return KDA_ERR_ALIAS;
    }

    kda::BackwardArgs a;
    a.f32io = io_dtype == KDA_F32;
    a.q = q; a.k = k; a.v = v; a.z = z; a.A = A; a.beta = beta; a.h0 = h0;
    a.cu = cu_seqlens;
    a.N = N; a.T = T; a.H = H; a.d = dk;
    a.dO = grad_o; a.dhT = grad_hT;
    a.gq = grad_q; a.gk = grad_k; a.gv = grad_v; a.gz = grad_z; a.gbeta = grad_beta; a.gA = grad_A;
    a.gh0 = grad_h0;
    a.ws = static_cast<unsigned char *>(workspace);
    a.plan = plan;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    return kda::launch_prefill_backward(a) == 0 ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode(kda_dtype io_dtype, const void *q, const void *k, const void *v, const float *z,
               const float *A, const float *beta, float *S_inout, int N, int H, int dk, int dv,
               void *o, void *stream) {
    if (io_dtype != KDA_BF16 && io_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED_DTYPE;
    if (N < 0 || H <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(dk, dv)) return KDA_ERR_UNSUPPORTED_DIM;
    if (!A) return KDA_ERR_NULL_POINTER;
    if (N > 0 && (!q || !k || !v || !z || !beta || !S_inout || !o)) return KDA_ERR_NULL_POINTER;
    const void *ptrs[] = {q, k, v, z, A, beta, S_inout, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const size_t nh = (size_t)N * H;
    const size_t st_bytes = nh * dv * dk * 4, o_bytes = nh * dv * io_size(io_dtype);
    const struct { const void *p; size_t n; } ins[] = {
        {q, nh * dk * io_size(io_dtype)}, {k, nh * dk * io_size(io_dtype)},
        {v, nh * dv * io_size(io_dtype)}, {z, nh * dk * 4}, {A, (size_t)H * 4}, {beta, nh * 4}};
    for (const auto &in : ins)
        if (overlaps(o, o_bytes, in.p, in.n) || overlaps(S_inout, st_bytes, in.p, in.n))
            return KDA_ERR_ALIAS;
    if (overlaps(o, o_bytes, S_inout, st_bytes)) return KDA_ERR_ALIAS;

    kda::DecodeArgs a;
    a.f32io = io_dtype == KDA_F32;
    a.q = q; a.k = k; a.v = v; a.z = z; a.A = A; a.beta = beta;
    a.S = S_inout; a.o = o;
    a.N = N; a.H = H; a.dk = dk; a.dv = dv;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    return kda::launch_decode(a) == 0 ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_fused(kda_dtype io_dtype, const void *xq, const void *xk, const void *xv, const float *wq,
                     const float *wk, const float *wv, const void *conv_state_in, void *conv_state_out,
                     const float *z, const float *A, const float *beta, float *S_inout, const void *gate,
                     const float *norm_weight, float eps, int N, int H, int dk, int dv, void *y, void *stream) {
    if (io_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED_DTYPE;
    if (N < 0 || H <= 0 || !(eps >= 0.f)) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(dk, dv)) return KDA_ERR_UNSUPPORTED_DIM;
    if (!A || !wq || !wk || !wv || !norm_weight) return KDA_ERR_NULL_POINTER;
    if (N > 0 && (!xq || !xk || !xv || !z || !beta || !S_inout || !gate || !y)) return KDA_ERR_NULL_POINTER;
    const void *ptrs[] = {xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, z, A, beta, S_inout, gate,
                          norm_weight, y};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const size_t nh = (size_t)N * H, d = (size_t)dk;
    const size_t st_bytes = nh * d * d * 4, y_bytes = nh * d * 2, win_bytes = nh * 3 * 3 * d * 2;
    const struct { const void *p; size_t n; } ins[] = {
        {xq, nh * d * 2}, {xk, nh * d * 2}, {xv, nh * d * 2}, {wq, (size_t)H * d * 16}, {wk, (size_t)H * d * 16},
        {wv, (size_t)H * d * 16}, {z, nh * d * 4}, {A, (size_t)H * 4}, {beta, nh * 4}, {gate, y_bytes},
        {norm_weight, d * 4}};
    for (const auto &in : ins)
        if (overlaps(y, y_bytes, in.p, in.n) || overlaps(S_inout, st_bytes, in.p, in.n) ||
            (conv_state_out && overlaps(conv_state_out, win_bytes, in.p, in.n)))
            return KDA_ERR_ALIAS;
    if (overlaps(y, y_bytes, S_inout, st_bytes)) return KDA_ERR_ALIAS;
    if (conv_state_out && (overlaps(conv_state_out, win_bytes, y, y_bytes) ||
                           overlaps(conv_state_out, win_bytes, S_inout, st_bytes)))
        return KDA_ERR_ALIAS;
    if (conv_state_in && (overlaps(conv_state_in, win_bytes, y, y_bytes) ||
                          overlaps(conv_state_in, win_bytes, S_inout, st_bytes)))
        return KDA_ERR_ALIAS;
    // the window is read and written by the same thread: in place, or disjoint
    if (conv_state_in && conv_state_out && conv_state_in != conv_state_out &&
        overlaps(conv_state_in, win_bytes, conv_state_out, win_bytes))
        return KDA_ERR_ALIAS;

    kda::DecodeFusedArgs a;
    a.xq = xq; a.xk = xk; a.xv = xv;
    a.wq = wq; a.wk = wk; a.wv = wv;
    a.win_in = conv_state_in; a.win_out = conv_state_out;
    a.z = z; a.A = A; a.beta = beta; a.S = S_inout;
    a.gate = gate; a.norm_w = norm_weight; a.eps = eps; a.y = y;
    a.N = N; a.H = H; a.d = dk;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    return kda::launch_decode_fused(a) == 0 ? KDA_OK : KDA_ERR_HIP;
}

int kda_qkv_shortconv(kda_dtype io_dtype, const void *xq, const void *xk, const void *xv, const float *wq,
                      const float *wk, const float *wv, const int32_t *cu_seqlens, int N, int T, int H, int dk,
                      int dv, const void *conv_state_in, void *conv_state_out, void *q, void *k, void *v,
                      void *stream) {
    if (io_dtype != KDA_BF16 && io_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED_DTYPE;
    if (N < 0 || T < 0 || H <= 0 || (T > 0 && N == 0)) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(dk, dv)) return KDA_ERR_UNSUPPORTED_DIM;
    if (!cu_seqlens || !wq || !wk || !wv) return KDA_ERR_NULL_POINTER;
    if (T > 0 && (!xq || !xk || !xv || !q || !k || !v)) return KDA_ERR_NULL_POINTER;
    const void *ptrs[] = {xq, xk, xv, wq, wk, wv, cu_seqlens, conv_state_in, conv_state_out, q, k, v};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const size_t io = io_size(io_dtype), tok = (size_t)T * H * dk * io;
    const size_t win = (size_t)N * 3 * H * 3 * dk * io;
    const struct { const void *p; size_t n; } ins[] = {
        {xq, tok}, {xk, tok}, {xv, tok}, {wq, (size_t)H * dk * 16}, {wk, (size_t)H * dk * 16},
        {wv, (size_t)H * dk * 16}, {cu_seqlens, (size_t)(N + 1) * 4}, {conv_state_in, win}};
    const struct { const void *p; size_t n; } outs[] = {{q, tok}, {k, tok}, {v, tok}, {conv_state_out, win}};
    for (const auto &ot : outs) {
        for (const auto &in : ins)
            if (!(ot.p == conv_state_out && in.p == conv_state_in && ot.p == in.p) && overlaps(ot.p, ot.n, in.p, in.n))
                return KDA_ERR_ALIAS;
        for (const auto &o2 : outs)
            if (&o2 != &ot && overlaps(ot.p, ot.n, o2.p, o2.n)) return KDA_ERR_ALIAS;
    }
    kda::FeatureArgs a;
    a.f32io = io_dtype == KDA_F32;
    a.xq = xq; a.xk = xk; a.xv = xv; a.wq = wq; a.wk = wk; a.wv = wv;
    a.cu = cu_seqlens; a.N = N; a.T = T; a.H = H; a.d = dk;
    a.win_in = conv_state_in; a.win_out = conv_state_out;
    a.q = q; a.k = k; a.v = v;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    return kda::launch_features(a) == 0 ? KDA_OK : KDA_ERR_HIP;
}

int kda_output_gate(kda_dtype io_dtype, const void *o, const void *g, const float *w, float eps, int T, int H,
                    int dv, void *y, void *stream) {
    if (io_dtype != KDA_BF16 && io_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED_DTYPE;
    if (T < 0 || H <= 0 || !(eps >= 0.f)) return KDA_ERR_INVALID_ARGUMENT;
    if (!(dv == 32 || dv == 64 || dv == 128)) return KDA_ERR_UNSUPPORTED_DIM;
    if (!w) return KDA_ERR_NULL_POINTER;
    if (T > 0 && (!o || !g || !y)) return KDA_ERR_NULL_POINTER;
    const void *ptrs[] = {o, g, w, y};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const size_t n = (size_t)T * H * dv * io_size(io_dtype);
    // y may be o or g exactly (every element is read before it is written), nothing else
    if ((y != o && overlaps(y, n, o, n)) || (y != g && overlaps(y, n, g, n)) || overlaps(y, n, w, (size_t)dv * 4))
        return KDA_ERR_ALIAS;
    kda::GateArgs a;
    a.f32io = io_dtype == KDA_F32;
    a.o = o; a.g = g; a.w = w; a.eps = eps; a.T = T; a.H = H; a.dv = dv; a.y = y;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    return kda::launch_output_gate(a) == 0 ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_window(kda_dtype io_dtype, const void *rk, const void *rv, const float *rz,
                      const float *rbeta, const int32_t *n_accept, int Lr, const void *q, const void *k,
                      const void *v, const float *z, const float *beta, int L, const float *A,
                      float *S_inout, int N, int H, int dk, int dv, void *o, int commit_window,
                      void *stream) {
    if (io_dtype != KDA_BF16 && io_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED_DTYPE;
    if (N < 0 || H <= 0 || Lr < 0 || L < 0 || Lr > KDA_MAX_DECODE_WINDOW || L > KDA_MAX_DECODE_WINDOW ||
        (commit_window != 0 && commit_window != 1))
        return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(dk, dv)) return KDA_ERR_UNSUPPORTED_DIM;
    if (!A) return KDA_ERR_NULL_POINTER;
    if (N > 0 && !S_inout) return KDA_ERR_NULL_POINTER;
    if (N > 0 && Lr > 0 && (!rk || !rv || !rz || !rbeta || !n_accept)) return KDA_ERR_NULL_POINTER;
    if (N > 0 && L > 0 && (!q || !k || !v || !z || !beta || !o)) return KDA_ERR_NULL_POINTER;
    const void *ptrs[] = {rk, rv, rz, rbeta, n_accept, q, k, v, z, beta, A, S_inout, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const size_t nh = (size_t)N * H, io = io_size(io_dtype);
    const size_t st_bytes = nh * dv * dk * 4, o_bytes = nh * L * dv * io;
    const size_t r = nh * Lr, w = nh * L;
    const struct { const void *p; size_t n; } ins[] = {
        {rk, r * dk * io}, {rv, r * dv * io}, {rz, r * dk * 4}, {rbeta, r * 4}, {n_accept, (size_t)N * 4},
        {q, w * dk * io}, {k, w * dk * io}, {v, w * dv * io}, {z, w * dk * 4}, {beta, w * 4},
        {A, (size_t)H * 4}};
    for (const auto &in : ins)
        if (overlaps(o, o_bytes, in.p, in.n) || overlaps(S_inout, st_bytes, in.p, in.n)) return KDA_ERR_ALIAS;
    if (overlaps(o, o_bytes, S_inout, st_bytes)) return KDA_ERR_ALIAS;

    kda::DecodeWindowArgs a;
    a.f32io = io_dtype == KDA_F32;
    a.rk = rk; a.rv = rv; a.rz = rz; a.rbeta = rbeta; a.n_accept = n_accept; a.Lr = Lr;
    a.q = q; a.k = k; a.v = v; a.z = z; a.beta = beta; a.L = L;
    a.A = A; a.S = S_inout; a.o = o;
    a.N = N; a.H = H; a.dk = dk; a.dv = dv;
    a.commit_window = commit_window == 1;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    return kda::launch_decode_window(a) == 0 ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
