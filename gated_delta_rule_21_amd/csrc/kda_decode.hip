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
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) kq += __shfl_xor(kq, off, 64);

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
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) {
            pk += __shfl_xor(pk, off, 64);
            pq += __shfl_xor(pq, off, 64);
        }
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
