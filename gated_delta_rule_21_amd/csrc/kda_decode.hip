// kda_decode.hip -- single-token KDA decode step for gfx950.
//
// One workgroup per (sequence, head).  The fp32 state S (dv rows of dk
// floats, [dv][dk] in memory) streams through once: every row is read with
// 16-byte loads, updated in registers and written back in place.  Per row j
// (prediction-error form of "Hybrid KDA–MLA：Kimi K3 注意力机制解析", core
// update; "Kimi K3：架构、训练与推理系统研究" §3.1):
//   Sbar_j = alpha * S_j                       (alpha = exp(g), per key channel)
//   p_j    = Sbar_j . k,   r_j = Sbar_j . q    (two reductions across the row's lanes)
//   e_j    = v_j - p_j
//   S_j    = Sbar_j + beta e_j k
//   o_j    = S_j . q = r_j + beta e_j (k . q)
// The row's key channels are spread over LPR = dk/16 neighbouring lanes with
// 16 channels each, so the reductions are log2(LPR) lane exchanges inside a
// wavefront and no LDS or barrier is needed.  A workgroup has one thread per
// (row, 16 channels) up to 1024 threads, so at d = 128 every thread owns one
// 64-byte piece of one row: the whole 64 KiB state of a head is in flight at
// once, which is what keeps the HBM queues full.  The state is the only large
// stream (2 * dk * dv * 4 bytes per head), which makes the kernel HBM-bound
// ("Kimi K3：架构…" §11.4, §13.2).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV, bool F32IO>
__global__ void __launch_bounds__(1024) decode_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ z, const float *__restrict__ A, const float *__restrict__ beta,
    float *__restrict__ S, void *__restrict__ o, int H) {
    constexpr int LPR = DK / 16;                 // lanes per state row
    constexpr int THREADS = (DV * LPR < 1024) ? DV * LPR : 1024;
    constexpr int ROWS_PER_PASS = THREADS / LPR;
    constexpr int PASSES = DV / ROWS_PER_PASS;
    static_assert(PASSES * ROWS_PER_PASS == DV, "row split");

    const int pair = blockIdx.x;                 // n * H + h
    const int h = pair % H;
    const int t = threadIdx.x;
    const int cl = t % LPR;                      // lane within the row
    const int rg = t / LPR;                      // row within the pass

    float *Sp = S + (size_t)pair * DV * DK;
    // The state is the stream: issue every load of this thread's rows first,
    // before the small per-head inputs, so that no state load waits behind
    // the gate arithmetic.
    f32x4 s[PASSES][4];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int row = rg + ROWS_PER_PASS * p;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            s[p][m] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(Sp + (size_t)row * DK + 4 * (cl + LPR * m)));
    }

    __builtin_amdgcn_sched_barrier(0);  // keep the state loads ahead of everything else
    // Key channels owned by this lane: float4 groups cl + LPR * m, m = 0..3.
    const size_t krow = (size_t)pair * DK;
    float kk[16], qq[16], aa[16];
    const float ea = __expf(A[h]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int c0 = 4 * (cl + LPR * m);
        const f32x4 zv = *reinterpret_cast<const f32x4 *>(z + krow + c0);
        const f32x4 kv = load_io4<F32IO>(k, krow + c0);
        const f32x4 qv = load_io4<F32IO>(q, krow + c0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            kk[4 * m + j] = kv[j];
            qq[4 * m + j] = qv[j];
            aa[4 * m + j] = exp2f(gate_log2(ea, zv[j]));
        }
    }
    const float b = beta[pair];

    // k . q over the full row (reduced across the LPR lanes).
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) kq += kk[i] * qq[i];
    kq = lane_group_sum<LPR>(kq);

#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int row = rg + ROWS_PER_PASS * p;
        float sb[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sb[4 * m + j] = aa[4 * m + j] * s[p][m][j];
        }
        float pk = 0.f, pq = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            pk += sb[i] * kk[i];
            pq += sb[i] * qq[i];
        }
        pk = lane_group_sum<LPR>(pk);
        pq = lane_group_sum<LPR>(pq);
        const float e = load_io<F32IO>(v, (size_t)pair * DV + row) - pk;
        const float be = b * e;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = sb[4 * m + j] + be * kk[4 * m + j];
            __builtin_nontemporal_store(
                w, reinterpret_cast<f32x4 *>(Sp + (size_t)row * DK + 4 * (cl + LPR * m)));
        }
        if (cl == 0) store_io<F32IO>(o, (size_t)pair * DV + row, pq + be * kq);
    }
}

// The fused decode step ("Kimi K3：架构、训练与推理系统研究" §13.2: the
// production decode kernel runs ShortConv, the input norms, the gate, the KDA
// recurrence and the output norm in one loop over the state).  Per (sequence,
// head), around decode_kernel's update (bf16 inputs, dk = dv = D):
//   * the feature path of the new token ("Kimi K3：架构…" §3.2): ShortConv(4)
//     over the carried window and the token, Swish, L2Norm for q and k, kept
//     in fp32 (the update is fp32 VALU work, so nothing asks for a rounding);
//   * the window shifted by one token (§3.4), written back in place or to a
//     second buffer;
//   * y = Sigmoid(g) * RMSNorm(o) over the head's D outputs (§3.3), with o kept
//     in fp32 (only y is rounded).
// The first 3 D / 4 threads compute the features (q, k and v each a group of
// D / 4 lanes with 4 channels, inside one wavefront, so the L2 norms are lane
// exchanges), the decay factors of the key channels and the new window; every
// thread then takes its channels from LDS after one barrier.  The sum of o^2
// over the rows takes a second barrier.
// Four packed bf16 as fp32 (exact).
__device__ __forceinline__ f32x4 bf16x4_to_quad(u32x2 w) {
    return f32x4{bf16_lo_half(w[0]), bf16_hi_half(w[0]), bf16_lo_half(w[1]), bf16_hi_half(w[1])};
}

template <int D>
__global__ void __launch_bounds__(1024) decode_fused_kernel(
    const uint16_t *__restrict__ xq, const uint16_t *__restrict__ xk, const uint16_t *__restrict__ xv,
    const float *__restrict__ wq, const float *__restrict__ wk, const float *__restrict__ wv, const uint16_t *win_in,
    uint16_t *win_out, const float *__restrict__ z, const float *__restrict__ A, const float *__restrict__ beta,
    float *__restrict__ S, const uint16_t *__restrict__ gate, const float *__restrict__ norm_w, float eps,
    uint16_t *__restrict__ y, int H) {
    constexpr int LPR = D / 16;                  // lanes per state row
    constexpr int THREADS = D * LPR;             // one pass: every row at once
    constexpr int G = D / 4;                     // feature lanes per tensor
    constexpr int NW = THREADS / 64;
    constexpr int CW = 3 * D;                    // window channels per head: q | k | v
    static_assert(THREADS <= 1024 && THREADS % 64 == 0 && 3 * G <= THREADS, "one pass");
    __shared__ __attribute__((aligned(16))) float fq[D], fk[D], fv[D], fa[D];
    __shared__ float part[NW];

    const int pair = blockIdx.x;                 // n * H + h
    const int n = pair / H, h = pair % H;
    const int t = threadIdx.x;
    const int cl = t % LPR;                      // lane within the row
    const int row = t / LPR;

    float *Sp = S + (size_t)pair * D * D;
    f32x4 s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sp + (size_t)row * D + 4 * (cl + LPR * m)));
    __builtin_amdgcn_sched_barrier(0);  // the state loads first, as in decode_kernel

    if (t < 3 * G) {
        const int which = t / G, c0 = 4 * (t % G);
        const uint16_t *x = which == 0 ? xq : which == 1 ? xk : xv;
        const float *w = which == 0 ? wq : which == 1 ? wk : wv;
        // taps 0..2 meet the window's tokens (oldest first), tap 3 the new token
        u32x2 raw[4];
#pragma unroll
        for (int j = 0; j < 3; ++j)
            raw[j] = win_in ? *reinterpret_cast<const u32x2 *>(win_in + ((size_t)(n * 3 + j) * H + h) * CW + which * D + c0)
                            : u32x2{0u, 0u};
        raw[3] = *reinterpret_cast<const u32x2 *>(x + (size_t)pair * D + c0);
        const f32x4 *wt = reinterpret_cast<const f32x4 *>(w + ((size_t)h * D + c0) * 4);
        f32x4 f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x4 wc = wt[c];
            float u = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) u += wc[i] * bf16x4_to_quad(raw[i])[c];
            f[c] = swish(u);
        }
        if (which < 2) {
            float ss = f[0] * f[0] + f[1] * f[1] + f[2] * f[2] + f[3] * f[3];
            ss = lane_group_sum<G>(ss);
            f = f * fast_rsq(ss);
        }
        float *dst = which == 0 ? fq : which == 1 ? fk : fv;
        *reinterpret_cast<f32x4 *>(dst + c0) = f;
        if (which == 1) {
            const f32x4 zv = *reinterpret_cast<const f32x4 *>(z + (size_t)pair * D + c0);
            const float ea = __expf(A[h]);
            f32x4 al;
#pragma unroll
            for (int j = 0; j < 4; ++j) al[j] = exp2f(gate_log2(ea, zv[j]));
            *reinterpret_cast<f32x4 *>(fa + c0) = al;
        }
        // the window after this token; this thread alone reads and writes these
        // elements, so win_out may be win_in
        if (win_out) {
#pragma unroll
            for (int j = 0; j < 3; ++j)
                *reinterpret_cast<u32x2 *>(win_out + ((size_t)(n * 3 + j) * H + h) * CW + which * D + c0) = raw[j + 1];
        }
    }
    __syncthreads();

    float kk[16], qq[16], aa[16];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int c0 = 4 * (cl + LPR * m);
        const f32x4 kv = *reinterpret_cast<const f32x4 *>(fk + c0);
        const f32x4 qv = *reinterpret_cast<const f32x4 *>(fq + c0);
        const f32x4 av = *reinterpret_cast<const f32x4 *>(fa + c0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            kk[4 * m + j] = kv[j];
            qq[4 * m + j] = qv[j];
            aa[4 * m + j] = av[j];
        }
    }
    const float b = beta[pair];
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) kq += kk[i] * qq[i];
    kq = lane_group_sum<LPR>(kq);

    float sb[16];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) sb[4 * m + j] = aa[4 * m + j] * s[m][j];
    float pk = 0.f, pq = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        pk += sb[i] * kk[i];
        pq += sb[i] * qq[i];
    }
    pk = lane_group_sum<LPR>(pk);
    pq = lane_group_sum<LPR>(pq);
    const float be = b * (fv[row] - pk);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = sb[4 * m + j] + be * kk[4 * m + j];
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(Sp + (size_t)row * D + 4 * (cl + LPR * m)));
    }
    const float o = pq + be * kq;

    // RMS over the head's D outputs: per wave over its rows' first lanes, then
    // the NW wave sums in a fixed order
    float ss = cl == 0 ? o * o : 0.f;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) ss += __shfl_xor(ss, off, 64);
    if ((t & 63) == 0) part[t >> 6] = ss;
    __syncthreads();
    if (cl == 0) {
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) tot += part[i];
        const float inv = fast_rsq(tot * (1.f / D) + eps);
        const float g = bf16_bits_to_f32(gate[(size_t)pair * D + row]);
        const float yv = o * inv * norm_w[row] * fast_rcp(1.f + __expf(-g));
        reinterpret_cast<__bf16 *>(y)[(size_t)pair * D + row] = (__bf16)yv;
    }
}

template <int D>
static int launch_decode_fused_t(const DecodeFusedArgs &a) {
    hipLaunchKernelGGL((decode_fused_kernel<D>), dim3((unsigned)(a.N * a.H)), dim3(D * (D / 16)), 0, a.stream,
                       static_cast<const uint16_t *>(a.xq), static_cast<const uint16_t *>(a.xk),
                       static_cast<const uint16_t *>(a.xv), a.wq, a.wk, a.wv,
                       static_cast<const uint16_t *>(a.win_in), static_cast<uint16_t *>(a.win_out), a.z, a.A,
                       a.beta, a.S, static_cast<const uint16_t *>(a.gate), a.norm_w, a.eps,
                       static_cast<uint16_t *>(a.y), a.H);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_decode_fused(const DecodeFusedArgs &a) {
    if (a.N == 0) return 0;
    switch (a.d) {
        case 32: return launch_decode_fused_t<32>(a);
        case 64: return launch_decode_fused_t<64>(a);
        case 128: return launch_decode_fused_t<128>(a);
    }
    return -1;
}

template <int D, bool F32IO>
static int launch_decode_t(const DecodeArgs &a) {
    constexpr int LPR = D / 16;
    constexpr int THREADS = (D * LPR < 1024) ? D * LPR : 1024;
    dim3 grid((unsigned)(a.N * a.H));
    hipLaunchKernelGGL((decode_kernel<D, D, F32IO>), grid, dim3(THREADS), 0, a.stream, a.q, a.k,
                       a.v, a.z, a.A, a.beta, a.S, a.o, a.H);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_decode(const DecodeArgs &a) {
    if (a.N == 0) return 0;
    const bool f32 = a.f32io;
    switch (a.dk) {
        case 32: return f32 ? launch_decode_t<32, true>(a) : launch_decode_t<32, false>(a);
        case 64: return f32 ? launch_decode_t<64, true>(a) : launch_decode_t<64, false>(a);
        case 128: return f32 ? launch_decode_t<128, true>(a) : launch_decode_t<128, false>(a);
    }
    return -1;
}

}  // namespace kda
