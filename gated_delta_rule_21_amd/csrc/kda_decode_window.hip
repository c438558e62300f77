// kda_decode_window.hip -- multi-token decode with replay for gfx950.
//
// Speculative decoding advances the recurrent state with every draft token,
// and a state updated in place cannot be rolled back when drafts are
// rejected.  The pages' answer ("Kimi K3：架构、训练与推理系统研究" §11.3 and
// §13.2; the orkas.ai K3 post, section on serving costs) is to keep the
// committed state, cache the small projected inputs of the draft window, and
// once the verifier has decided, replay the accepted tokens on chip in the
// same pass that processes the next window.
//
// One workgroup per (sequence, head), laid out like decode_kernel: each
// thread owns 16 key channels of one state row (row = value channel).  Per
// call and (sequence, head):
//   1. the state streams in once (16-byte loads, issued first);
//   2. the replay tokens' and the window's inputs are staged in LDS, with the
//      gate alpha = exp(g_min * sigmoid(e^A z)) computed on the way;
//   3. the first n_accept[n] replay tokens advance the state (no output);
//   4. the committed state streams out once (unless nothing changed);
//   5. the window tokens advance a register copy of the state and write
//      o_t = S_t^T q_t; the copy is discarded (or, with commit_window, it is
//      the state written back in step 4's place).
// The per-token update is the prediction-error form of the recurrence
// ("Hybrid KDA–MLA：Kimi K3 注意力机制解析", core update; "Kimi K3：架构、训练与推理系统研究" §3.1):
//   Sbar = alpha * S (per key channel),  e = v - Sbar^T k,
//   S = Sbar + beta k e^T,  o = S^T q = Sbar^T q + beta e (k . q).
#include "kda_chunk.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// LDS image of one token: alpha, k (and q for window tokens) over dk, v over
// dv, then beta; all fp32.
struct WindowLds {
    int dk, dv;
    __host__ __device__ int replay_floats() const { return 2 * dk + dv + 4; }
    __host__ __device__ int window_floats() const { return 3 * dk + dv + 4; }
    __host__ __device__ size_t bytes(int Lr, int L) const {
        return ((size_t)Lr * replay_floats() + (size_t)L * window_floats()) * 4;
    }
};

template <int DK, int DV, bool F32IO>
__global__ void __launch_bounds__(1024) decode_window_kernel(
    const void *__restrict__ rk, const void *__restrict__ rv, const float *__restrict__ rz,
    const float *__restrict__ rbeta, const int32_t *__restrict__ n_accept, int Lr,
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ z, const float *__restrict__ beta, int L, const float *__restrict__ A,
    float *__restrict__ S, void *__restrict__ o, int H, int commit_window) {
    constexpr int LPR = DK / 16;                 // lanes per state row
    constexpr int THREADS = DV * LPR;
    static_assert(THREADS <= 1024, "one pass over the rows");
    constexpr int RF = 2 * DK + DV + 4, WF = 3 * DK + DV + 4;   // floats per staged token
    extern __shared__ __attribute__((aligned(16))) float lds[];

    const int pair = blockIdx.x;                 // n * H + h
    const int n = pair / H, h = pair % H;
    const int t = threadIdx.x;
    const int cl = t % LPR;                      // lane within the row
    const int row = t / LPR;                     // value channel

    float *Sp = S + (size_t)pair * DV * DK;
    f32x4 s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sp + (size_t)row * DK + 4 * (cl + LPR * m)));
    __builtin_amdgcn_sched_barrier(0);  // keep the state loads ahead of everything else

    int acc = 0;
    if (Lr > 0) acc = min(max(n_accept[n], 0), Lr);

    // ---- stage the inputs: token u of the replay (u < acc) or the window
    const float ea = __expf(A[h]);
    float *rbase = lds, *wbase = lds + (size_t)Lr * RF;
    const int rgroups = acc * (DK / 4), wgroups = L * (DK / 4);
    for (int i = t; i < rgroups + wgroups; i += THREADS) {
        const bool win = i >= rgroups;
        const int u = win ? (i - rgroups) / (DK / 4) : i / (DK / 4);
        const int c0 = 4 * (win ? (i - rgroups) % (DK / 4) : i % (DK / 4));
        // token u of sequence n: row (n * len + u) of the [N][len][H][d] inputs
        const size_t kr = ((size_t)(n * (win ? L : Lr) + u) * H + h) * DK + c0;
        const f32x4 zv = *reinterpret_cast<const f32x4 *>((win ? z : rz) + kr);
        const f32x4 kv = load_io4<F32IO>(win ? k : rk, kr);
        f32x4 av;
#pragma unroll
        for (int j = 0; j < 4; ++j) av[j] = exp2f(gate_log2(ea, zv[j]));
        float *img = win ? wbase + (size_t)u * WF : rbase + (size_t)u * RF;
        *reinterpret_cast<f32x4 *>(img + c0) = av;
        *reinterpret_cast<f32x4 *>(img + DK + c0) = kv;
        if (win) *reinterpret_cast<f32x4 *>(img + 2 * DK + c0) = load_io4<F32IO>(q, kr);
    }
    for (int i = t; i < (acc + L) * (DV / 4); i += THREADS) {
        const bool win = i >= acc * (DV / 4);
        const int j4 = win ? i - acc * (DV / 4) : i;
        const int u = j4 / (DV / 4), c0 = 4 * (j4 % (DV / 4));
        const size_t vr = ((size_t)(n * (win ? L : Lr) + u) * H + h) * DV + c0;
        float *img = win ? wbase + (size_t)u * WF + 3 * DK : rbase + (size_t)u * RF + 2 * DK;
        *reinterpret_cast<f32x4 *>(img + c0) = load_io4<F32IO>(win ? v : rv, vr);
    }
    for (int u = t; u < acc + L; u += THREADS) {
        const bool win = u >= acc;
        const int uu = win ? u - acc : u;
        const float b = win ? beta[(size_t)(n * L + uu) * H + h] : rbeta[(size_t)(n * Lr + uu) * H + h];
        (win ? wbase + (size_t)uu * WF + 3 * DK + DV : rbase + (size_t)uu * RF + 2 * DK + DV)[0] = b;
    }
    __syncthreads();

    // one token: alpha at a, k at a + DK, v at vv, beta at vv + DV; returns e * beta
    auto advance = [&](const float *a, const float *kk, const float *vv, float b, const float *qq, float &pq) {
        float sb[16];
        float pk = 0.f;
        pq = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 av = *reinterpret_cast<const f32x4 *>(a + 4 * (cl + LPR * m));
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(kk + 4 * (cl + LPR * m));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sb[4 * m + j] = av[j] * s[m][j];
                pk += sb[4 * m + j] * kv[j];
            }
            if (qq) {
                const f32x4 qv = *reinterpret_cast<const f32x4 *>(qq + 4 * (cl + LPR * m));
#pragma unroll
                for (int j = 0; j < 4; ++j) pq += sb[4 * m + j] * qv[j];
            }
        }
        pk = lane_group_sum<LPR>(pk);
        const float be = b * (vv[row] - pk);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(kk + 4 * (cl + LPR * m));
#pragma unroll
            for (int j = 0; j < 4; ++j) s[m][j] = sb[4 * m + j] + be * kv[j];
        }
        return be;
    };

    for (int u = 0; u < acc; ++u) {
        const float *img = rbase + (size_t)u * RF;
        float unused;
        advance(img, img + DK, img + 2 * DK, img[2 * DK + DV], nullptr, unused);
    }
    auto write_state = [&]() {
#pragma unroll
        for (int m = 0; m < 4; ++m)
            __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4 *>(Sp + (size_t)row * DK + 4 * (cl + LPR * m)));
    };
    if (!commit_window && acc > 0) write_state();

    for (int u = 0; u < L; ++u) {
        const float *img = wbase + (size_t)u * WF;
        const float *qq = img + 2 * DK;
        // k . q over the full row
        float kq = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(img + DK + 4 * (cl + LPR * m));
            const f32x4 qv = *reinterpret_cast<const f32x4 *>(qq + 4 * (cl + LPR * m));
#pragma unroll
            for (int j = 0; j < 4; ++j) kq += kv[j] * qv[j];
        }
        float pq;
        const float be = advance(img, img + DK, img + 3 * DK, img[3 * DK + DV], qq, pq);
        kq = lane_group_sum<LPR>(kq);
        pq = lane_group_sum<LPR>(pq);
        if (cl == 0) store_io<F32IO>(o, ((size_t)(n * L + u) * H + h) * DV + row, pq + be * kq);
    }
    if (commit_window && acc + L > 0) write_state();
}

size_t decode_window_lds_bytes(int d, int Lr, int L) { return WindowLds{d, d}.bytes(Lr, L); }

template <int D, bool F32IO>
static int launch_window_t(const DecodeWindowArgs &a) {
    constexpr int THREADS = D * (D / 16);
    const size_t lds = decode_window_lds_bytes(D, a.Lr, a.L);
    if (!set_lds(&decode_window_kernel<D, D, F32IO>, lds)) return -1;
    hipLaunchKernelGGL((decode_window_kernel<D, D, F32IO>), dim3((unsigned)(a.N * a.H)), dim3(THREADS), lds, a.stream,
                       a.rk, a.rv, a.rz, a.rbeta, a.n_accept, a.Lr, a.q, a.k, a.v, a.z, a.beta, a.L, a.A, a.S, a.o,
                       a.H, a.commit_window ? 1 : 0);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_decode_window(const DecodeWindowArgs &a) {
    if (a.N == 0) return 0;
    switch (a.dk) {
        case 32: return a.f32io ? launch_window_t<32, true>(a) : launch_window_t<32, false>(a);
        case 64: return a.f32io ? launch_window_t<64, true>(a) : launch_window_t<64, false>(a);
        case 128: return a.f32io ? launch_window_t<128, true>(a) : launch_window_t<128, false>(a);
    }
    return -1;
}

}  // namespace kda
