// kda_backward.hip -- reverse-mode gradients of the chunkwise prefill for gfx950.
//
// The pages give the forward recurrence and its chunk form but no backward
// pass; this one differentiates the chunk form of the s1mplewind "kimi-k3"
// notes (section "Chunkwise 形式") as matrices.  Per chunk of C = 64 tokens,
// with S the state at the chunk's start, dS' the gradient of the state at its
// end, Gamma the inclusive cumulative decay inside the chunk, gamma_C its last
// row, T = (I + StrictTril(Diag(beta)(Gamma*K)(K/Gamma)^T))^{-1},
// M = T Diag(beta), W = M (Gamma*K), P = Tril((Gamma*Q)(K/Gamma)^T),
// K~ = (gamma_C/Gamma)*K and V~ = V - (Gamma*K) S (so V' = M V~):
//   dV' = P^T dO + K~ dS'
//   dS  = (Gamma*Q)^T dO + Diag(gamma_C) dS' - W^T dV'      (to the previous chunk)
//   dV  = M^T dV',  dM = dV' V~^T,  dbeta_j += sum_t dM_tj T_tj
//   dA_kk = -StrictTril(T^T (dM Diag(beta)) T^T),  dbeta_r += sum_i dA_kk,ri R_ri
//   dR = Diag(beta) dA_kk,  dP = Tril(dO V'^T)
//   dQ = Gamma*(dO S^T) + [dP (K/Gamma)]*Gamma
//   dK = -Gamma*(M^T dV' S^T) + [dR (K/Gamma)]*Gamma + [(dP^T (Gamma*Q) + dR^T (Gamma*K))]/Gamma
//        + (gamma_C/Gamma)*(V' dS'^T)
// and the gradient of the log-decay, which a reverse cumulative sum over the
// chunk turns into the gradient of every token's gate.
//
// Pipeline (one call):
//   1. the forward prefill again, saving the state at every chunk boundary
//      (kda_prefill's checkpoint path with a 64-token interval);
//   2. bwd_local_kernel, one workgroup per (chunk, head): R, P, T, W, K~,
//      gamma_C and the chain's dS-free terms X = P^T dO, Y = (Gamma*Q)^T dO;
//   3. bwd_chain_kernel, per (sequence, head, value columns): walks the
//      chunks backwards carrying dS in fp32 MFMA accumulators, stores dS'
//      (key-major) and dV' (both orientations) of every chunk, and dh0;
//   4. bwd_grad_kernel, persistent over (chunk, head) items: every input gradient;
//   5. bwd_dA_kernel: the per-head sum of the chunks' A gradients, in a fixed
//      order (the result does not depend on scheduling).
//
// Everything after the forward recompute accumulates in fp32.  fp32 inputs:
// fp32 16x16x4 MFMA throughout.  bf16 inputs: the products run on K32 pairs of
// 16x16x32 bf16 MFMAs with each fp32 operand split into bf16 hi + lo (three
// MFMAs, about 2^-16 relative per term; two when the other operand is the
// exact bf16 dO); the blocked inverse (T) and the decay-masked products of
// dP and dA_kk stay on fp32 MFMA.
// Decay factors: a 64-token chunk can decay by e^-320, so no Gamma or 1/Gamma
// over a chunk is formed where the quotient of two would be needed.  Log2
// decays are kept relative to the start of each 16-token block (Gb) with the
// block totals bt; a factor exp2(G_r - G_i), r >= i, is split at a reference
// point so that both halves are <= 1 when r and i lie in different blocks
// (the end of i's block or the start of r's), and at the block's middle row
// when they share one, so neither half exceeds e^40 (eight steps of the
// bounded gate; devpress K3 walk-through §3.2, Eq 5).  The middle reference
// keeps gradients as large as 1e20 within fp32 range in those products.
// ---------------------------------------------------------------------------
#include "kda_chunk.h"
#include "kda_device.h"
#include "kda_internal.h"

#include <algorithm>
#include <type_traits>

namespace kda {

namespace {

constexpr int kBwdWaves = 8, kBwdThreads = 64 * kBwdWaves;
constexpr int kPS = 68;   // pitch of 64 x 64 fp32 matrices in LDS

// Per-(chunk, head) fp32 record in the workspace; offsets in floats.
template <int D>
struct BwdItem {
    static constexpr size_t kt = 0;              // K~ = (gamma_C/Gamma)*K        [64][D]
    static constexpr size_t wt = kt + 64 * D;    // W^T                           [D][64]
    static constexpr size_t xv = wt + 64 * D;    // X^T, then dV'^T               [D][64]
    static constexpr size_t dvr = xv + 64 * D;   // dV'                           [64][D]
    static constexpr size_t ys = dvr + 64 * D;   // Y, then dS'                   [D][D] (key-major)
    static constexpr size_t gam = ys + D * D;    // gamma_C                       [D]
    static constexpr size_t r = gam + D;         // R, strictly lower             [64][64]
    static constexpr size_t t = r + 64 * 64;     // T                             [64][64]
    static constexpr size_t floats = (t + 64 * 64 + 63) / 64 * 64;
};

__device__ __forceinline__ f32x4 rd4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void wr4(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }
// p[0], p[ld], p[2 ld], p[3 ld]: four rows of one column
__device__ __forceinline__ f32x4 rdcol4(const float *p, int ld) {
    return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}
__device__ __forceinline__ f32x4 exp2x4(f32x4 x) {
    return f32x4{fast_exp2(x[0]), fast_exp2(x[1]), fast_exp2(x[2]), fast_exp2(x[3])};
}
__device__ __forceinline__ f32x4 splat4(float x) { return f32x4{x, x, x, x}; }

// acc + A B over two K16 tiles (a0, b0: tile 2p; a1, b1: tile 2p + 1) in the
// fp32 fragment layout.  fp32 path: four fp32 MFMAs per tile.  bf16 path: each
// operand split into bf16 hi + lo and three 16x16x32 bf16 MFMAs (hi hi, hi lo,
// lo hi), good to about 2^-16 relative per term.
template <bool F32>
__device__ __forceinline__ f32x4 mma_k32(f32x4 a0, f32x4 a1, f32x4 b0, f32x4 b1, f32x4 acc) {
    if constexpr (F32) {
        acc = mma_f32_k16(a0, b0, acc);
        return mma_f32_k16(a1, b1, acc);
    } else {
        u32x4 ah, al, bh, bl;
        quads_to_bf16_split(a0, a1, ah, al);
        quads_to_bf16_split(b0, b1, bh, bl);
        return mma3_bf16(ah, al, bh, bl, acc);
    }
}

// The same for a B operand that holds bf16 values exactly (dO on the bf16
// path): only A is split, two MFMAs.
__device__ __forceinline__ f32x4 mma_k32_exact_b(f32x4 a0, f32x4 a1, f32x4 b0, f32x4 b1, f32x4 acc) {
    u32x4 ah, al;
    quads_to_bf16_split(a0, a1, ah, al);
    const u32x4 bh = quads_to_bf16(b0, b1);
    acc = mma_bf16_k32(ah, bh, acc);
    return mma_bf16_k32(al, bh, acc);
}

// sum_{m = lo}^{hi - 1} bt[m][c] (zero when lo >= hi); bt is [4][D].
template <int D>
__device__ __forceinline__ f32x4 span4(const float *bt, int lo, int hi, int c) {
    f32x4 s = zero4();
    for (int m = lo; m < hi; ++m) s += rd4(bt + m * D + c);
    return s;
}
template <int D>
__device__ __forceinline__ float span1(const float *bt, int lo, int hi, int c) {
    float s = 0.f;
    for (int m = lo; m < hi; ++m) s += bt[m * D + c];
    return s;
}

// Rows [0, 64) of a chunk's [T][H][D] slice into LDS as fp32 (pitch D + 4);
// rows >= L are zero.
template <int D, bool F32IO>
__device__ __forceinline__ void stage_rows(float *dst, const void *src, int t0, int L, int h, int H,
                                           int tid) {
    constexpr int PB = D + 4, Q = D / 4;
    for (int i = tid; i < 64 * Q; i += kBwdThreads) {
        const int r = i / Q, c = 4 * (i % Q);
        f32x4 x = zero4();
        if (r < L) x = load_io4<F32IO>(src, ((size_t)(t0 + r) * H + h) * D + c);
        wr4(dst + r * PB + c, x);
    }
}

// Raw inputs of one (chunk, head) item for one thread of the local kernel:
// the quads of q, k and dO it stages (io dtype; rows past the chunk's end
// zero), the 16 gate logits of thread (c, I) = (tid % D, tid / D), and beta.
// The next item's are fetched into registers while the current one computes.
template <int D, bool F32IO>
struct LocalIn {
    static constexpr int Q = D / 4, NQ = 64 * Q / kBwdThreads;
    using Quad = typename std::conditional<F32IO, f32x4, u32x2>::type;
    Quad q[NQ], k[NQ], o[NQ];
    float z[16];
    float beta;
};

template <int D, bool F32IO>
__device__ __forceinline__ typename LocalIn<D, F32IO>::Quad load_quad(const void *p, size_t i) {
    if constexpr (F32IO)
        return *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(p) + i);
    else
        return *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(p) + i);
}

template <int D, bool F32IO>
__device__ __forceinline__ void load_local(LocalIn<D, F32IO> &R, const void *q, const void *k, const void *dO,
                                           const float *z, const float *beta, int t0, int L, int h, int H,
                                           int tid) {
    using LI = LocalIn<D, F32IO>;
#pragma unroll
    for (int s = 0; s < LI::NQ; ++s) {
        const int i = tid + s * kBwdThreads, r = i / LI::Q, c = 4 * (i % LI::Q);
        const size_t off = ((size_t)(t0 + r) * H + h) * D + c;
        R.q[s] = r < L ? load_quad<D, F32IO>(q, off) : typename LI::Quad{};
        R.k[s] = r < L ? load_quad<D, F32IO>(k, off) : typename LI::Quad{};
        R.o[s] = r < L ? load_quad<D, F32IO>(dO, off) : typename LI::Quad{};
    }
    if (tid < 4 * D) {
        const int c = tid % D, I = tid / D;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 16 * I + i;
            R.z[i] = r < L ? z[((size_t)(t0 + r) * H + h) * D + c] : 0.f;
        }
    }
    R.beta = (tid < 64 && tid < L) ? beta[(size_t)(t0 + tid) * H + h] : 0.f;
}

// A zero the compiler cannot see through.  Lane-dependent constants built
// from `lane + opaque_zero()` inside a persistent item loop are rebuilt per
// item instead of being hoisted out of the loop and kept live (or spilled)
// across it.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// Raw inputs of one (chunk, head) item for one thread of the grad kernel:
// quads of k and v (io dtype; rows past the chunk's end zero), the 16 gate
// logits of thread (c, I) = (tid % D, tid / D), beta, and two quads of the
// item's T.  The next item's are fetched into registers during the current
// item's last phase.
template <int D, bool F32IO>
struct GradIn {
    static constexpr int Q = D / 4, NQ = 64 * Q / kBwdThreads;
    using Quad = typename std::conditional<F32IO, f32x4, u32x2>::type;
    Quad k[NQ], v[NQ];
    float z[16];
    float beta;
    f32x4 t[64 * 16 / kBwdThreads];
    f32x4 s[D / 16];   // the state's rows 16 (wave % KT) + ln, all key quads: B operands of V~
};

template <int D, bool F32IO>
__device__ __forceinline__ void load_grad_rows(GradIn<D, F32IO> &R, const void *k, const void *v,
                                               const float *beta, const float *item_t, int t0, int L, int h, int H,
                                               int tid) {
    using GI = GradIn<D, F32IO>;
#pragma unroll
    for (int s = 0; s < GI::NQ; ++s) {
        const int i = tid + s * kBwdThreads, r = i / GI::Q, c = 4 * (i % GI::Q);
        const size_t off = ((size_t)(t0 + r) * H + h) * D + c;
        R.k[s] = r < L ? load_quad<D, F32IO>(k, off) : typename GI::Quad{};
        R.v[s] = r < L ? load_quad<D, F32IO>(v, off) : typename GI::Quad{};
    }
    R.beta = (tid < 64 && tid < L) ? beta[(size_t)(t0 + tid) * H + h] : 0.f;
#pragma unroll
    for (int s = 0; s < 64 * 16 / kBwdThreads; ++s) {
        const int i = tid + s * kBwdThreads;
        R.t[s] = rd4(item_t + (i >> 4) * 64 + 4 * (i & 15));
    }
}
template <int D, bool F32IO>
__device__ __forceinline__ void load_grad_state(GradIn<D, F32IO> &R, const float *Sg, int nt, int ln, int lg) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        R.s[kk] = Sg ? rd4(Sg + (size_t)(16 * nt + ln) * D + 16 * kk + 4 * lg) : zero4();
}
template <int D, bool F32IO>
__device__ __forceinline__ void load_grad_z(GradIn<D, F32IO> &R, const float *z, int t0, int L, int h, int H,
                                            int tid) {
    if (tid < 4 * D) {
        const int c = tid % D, I = tid / D;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 16 * I + i;
            R.z[i] = r < L ? z[((size_t)(t0 + r) * H + h) * D + c] : 0.f;
        }
    }
}

// Rows [0, 64) of staged quads into LDS as fp32 (pitch D + 4).
template <int D, bool F32IO>
__device__ __forceinline__ void stage_quads(float *dst, const typename LocalIn<D, F32IO>::Quad *x, int tid) {
    using LI = LocalIn<D, F32IO>;
#pragma unroll
    for (int s = 0; s < LI::NQ; ++s) {
        const int i = tid + s * kBwdThreads, r = i / LI::Q, c = 4 * (i % LI::Q);
        wr4(dst + r * (D + 4) + c, quad_f32<F32IO>(x[s]));
    }
}

// LDS carve-up of the two per-item kernels (floats).
// Local kernel: q, k and the block log-decays Gb are staged first, then
// turned into block-referenced operands in place (qA = q 2^Gb and kA = k 2^Gb
// over q and k, kB = k 2^(bt - Gb) over Gb), with per-channel factor vectors
// [I][D]: pre = 2^(sum_{m<I} bt_m), suf = 2^(sum_{m>I} bt_m), off[J][I] =
// 2^(sum_{J<m<I} bt_m), dgA = 2^-Gb_mid(I), dgB = 2^(Gb_mid(I) - bt_I), where
// mid(I) is block I's row 7.  Every decay factor of the products below is one
// operand times one of these vectors.
template <int D>
struct LocalLds {
    static constexpr int PB = D + 4;
    static constexpr int q = 0, k = q + 64 * PB, gb = k + 64 * PB, r = gb + 64 * PB, p = r + 64 * kPS;
    static constexpr int beta = p + 64 * kPS, bt = beta + 64, gmid = bt + 4 * D;
    static constexpr int pre = gmid + 4 * D, suf = pre + 4 * D, off = suf + 4 * D, dga = off + 16 * D;
    static constexpr int dgb = dga + 4 * D, floats = dgb + 4 * D;
};

// The bf16 path stores K~ and W^T as split bf16 A fragments of the chain's
// products: fragment f of a region is 2 KiB, 64 lanes x 16 B of bf16 hi
// parts, then 64 x 16 B of lo parts, each lane's 16 B holding K16 tiles 2p
// (bytes 0-7) and 2p + 1 (bytes 8-15) of its K32 pair in the layout of
// quads_to_bf16_split.  This writes one tile's half of a lane's slots.
__device__ __forceinline__ void store_split_half(float *region, int f, int half, int lane, f32x4 x) {
    const u32x2 hi = {f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3])};
    const f32x4 r = x - f32x4{bf16_lo_half(hi[0]), bf16_hi_half(hi[0]), bf16_lo_half(hi[1]), bf16_hi_half(hi[1])};
    const u32x2 lo = {f32x2_to_bf16x2(r[0], r[1]), f32x2_to_bf16x2(r[2], r[3])};
    unsigned char *p = reinterpret_cast<unsigned char *>(region) + (size_t)f * 2048 + lane * 16 + half * 8;
    *reinterpret_cast<u32x2 *>(p) = hi;
    *reinterpret_cast<u32x2 *>(p + 1024) = lo;
}

template <int D>
struct GradLds {
    static constexpr int PB = D + 4;
    static constexpr int k = 0, gb = k + 64 * PB, x = gb + 64 * PB, s0 = x + 64 * PB, s1 = s0 + 64 * kPS;
    static constexpr int beta = s1 + 64 * kPS, bt = beta + 64, pd = bt + 4 * D, dgc = pd + 64;
    static constexpr int red = dgc + D, part = red + (8 * D > 512 ? 8 * D : 512), floats = part + kBwdWaves;
    static_assert(64 * PB <= 2 * 64 * kPS, "the gradient of the log-decay fits the two small matrices");
};

// ---------------------------------------------------------------------------
// Stage 2: per (chunk, head), the terms of the chain that do not depend on dS.
// ---------------------------------------------------------------------------
template <int D, bool F32IO>
__global__ void __launch_bounds__(kBwdThreads) bwd_local_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const float *__restrict__ z,
    const float *__restrict__ A, const float *__restrict__ beta, const void *__restrict__ dO,
    const int32_t *__restrict__ meta, const int4 *__restrict__ table, int N, int H, int max_chunks,
    float *__restrict__ items) {
    using IT = BwdItem<D>;
    using SL = LocalLds<D>;
    constexpr int PB = D + 4, KT = D / 16;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float *Qs = lds + SL::q, *Ks = lds + SL::k, *Gb = lds + SL::gb, *Rs = lds + SL::r, *Ps = lds + SL::p;
    float *bet = lds + SL::beta, *bt = lds + SL::bt, *gmid = lds + SL::gmid;
    float *fpre = lds + SL::pre, *fsuf = lds + SL::suf, *foff = lds + SL::off, *fdga = lds + SL::dga,
          *fdgb = lds + SL::dgb;
    float *kB = Gb;   // after the operand pass
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    using LI = LocalIn<D, F32IO>;
    const int total = meta[N] * H;
    int it = blockIdx.x;
    if (it >= total) return;
    LI R;
    int4 ent = table[it / H];
    load_local<D, F32IO>(R, q, k, dO, z, beta, ent.y, ent.z, it % H, H, tid);

    // persistent: items blockIdx.x, + gridDim.x, ...; the next item's inputs
    // load into R while this one computes
    for (; it < total; it += gridDim.x) {
        const int chunk = it / H, h = it % H;
        const int L = ent.z;
        float *item = items + ((size_t)h * max_chunks + chunk) * IT::floats;
        const float ea = __expf(A[h]);

        stage_quads<D, F32IO>(Qs, R.q, tid);
        stage_quads<D, F32IO>(Ks, R.k, tid);
        typename LI::Quad ocur[LI::NQ];
#pragma unroll
        for (int s = 0; s < LI::NQ; ++s) ocur[s] = R.o[s];
        if (tid < 4 * D) {
            // Gb (inclusive block scans of the log2 gate) and the block totals bt
            const int c = tid % D, I = tid / D;
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * I + i;
                run += r < L ? gate_log2(ea, R.z[i]) : 0.f;
                Gb[r * (D + 4) + c] = run;
                if (i == 7) gmid[I * D + c] = run;
            }
            bt[I * D + c] = run;
        }
        if (tid < 64) bet[tid] = R.beta;
        {
            const int it_next = it + gridDim.x;
            if (it_next < total) {
                ent = table[it_next / H];
                load_local<D, F32IO>(R, q, k, dO, z, beta, ent.y, ent.z, it_next % H, H, tid);
            }
        }
        __syncthreads();

        // factor vectors, and the operands qA, kA (in place) and kB (over Gb)
        for (int c = tid; c < D; c += kBwdThreads) {
            const float b0 = bt[c], b1 = bt[D + c], b2 = bt[2 * D + c], b3 = bt[3 * D + c];
            fpre[c] = 1.f;
            fpre[D + c] = fast_exp2(b0);
            fpre[2 * D + c] = fast_exp2(b0 + b1);
            fpre[3 * D + c] = fast_exp2(b0 + b1 + b2);
            fsuf[c] = fast_exp2(b1 + b2 + b3);
            fsuf[D + c] = fast_exp2(b2 + b3);
            fsuf[2 * D + c] = fast_exp2(b3);
            fsuf[3 * D + c] = 1.f;
            foff[(0 * 4 + 1) * D + c] = 1.f;
            foff[(0 * 4 + 2) * D + c] = fast_exp2(b1);
            foff[(0 * 4 + 3) * D + c] = fast_exp2(b1 + b2);
            foff[(1 * 4 + 2) * D + c] = 1.f;
            foff[(1 * 4 + 3) * D + c] = fast_exp2(b2);
            foff[(2 * 4 + 3) * D + c] = 1.f;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const float gm = gmid[I * D + c];
                fdga[I * D + c] = fast_exp2(-gm);
                fdgb[I * D + c] = fast_exp2(gm - bt[I * D + c]);
            }
        }
        for (int i = tid; i < 64 * (D / 4); i += kBwdThreads) {
            const int r = i / (D / 4), c = 4 * (i % (D / 4));
            const f32x4 g = rd4(Gb + r * PB + c);
            const f32x4 ea4 = exp2x4(g), eb4 = exp2x4(rd4(bt + (r >> 4) * D + c) - g);
            const f32x4 kv = rd4(Ks + r * PB + c);
            wr4(Qs + r * PB + c, rd4(Qs + r * PB + c) * ea4);
            wr4(Ks + r * PB + c, kv * ea4);
            wr4(kB + r * PB + c, kv * eb4);
        }
        __syncthreads();

        // Decayed Gram tiles (I, J), J <= I: R = (K.K) and P = (Q.K) with the
        // per-channel factor exp2(G_r - G_i); R strictly lower, P lower.
        //   J < I:  qA/kA_r . kB_i off[J][I]
        //   J = I:  qA/kA_r dgA[I] . kB_i dgB[I]   (halves <= e^40)
        for (int u = wave; u < 32; u += kBwdWaves) {
            const bool isP = u >= 16;
            const int I = (u & 15) >> 2, J = u & 3;
            float *dst = isP ? Ps : Rs;
            f32x4 acc = zero4();
            if (J <= I) {
                const float *src = isP ? Qs : Ks;
                const int r = 16 * I + ln, i = 16 * J + ln;
                const float *fa = I == J ? fdga + I * D : nullptr;
                const float *fb = I == J ? fdgb + I * D : foff + (J * 4 + I) * D;
                auto av = [&](int c) { return I == J ? rd4(src + r * PB + c) * rd4(fa + c) : rd4(src + r * PB + c); };
                auto bv = [&](int c) { return rd4(kB + i * PB + c) * rd4(fb + c); };
                if constexpr (F32IO) {
#pragma unroll
                    for (int kk = 0; kk < KT; ++kk) acc = mma_f32_k16(av(16 * kk + 4 * lg), bv(16 * kk + 4 * lg), acc);
                } else {
#pragma unroll
                    for (int kp = 0; kp < KT / 2; ++kp) {
                        const int c0 = 32 * kp + 4 * lg, c1 = c0 + 16;
                        acc = mma_k32<false>(av(c0), av(c1), bv(c0), bv(c1), acc);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 16 * I + 4 * lg + j, ii = 16 * J + ln;
                const bool keep = isP ? ii <= rr : ii < rr;
                dst[rr * kPS + ii] = keep ? acc[j] : 0.f;
            }
        }
        __syncthreads();

        // R to the record; Diag(beta) R in place, then T = (I + Diag(beta) R)^{-1}
        for (int i = tid; i < 64 * 16; i += kBwdThreads) {
            const int r = i >> 4, c = 4 * (i & 15);
            const f32x4 x = rd4(Rs + r * kPS + c);
            wr4(item + IT::r + r * 64 + c, x);
            wr4(Rs + r * kPS + c, x * bet[r]);
        }
        __syncthreads();
        // diagonal 16 x 16 blocks by forward substitution, one lane per column
        if (wave < 4 && lane < 16) {
            const int b = 16 * wave;
            float col[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = (r == lane) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) x -= Rs[(b + r) * kPS + b + i] * col[i];
                col[r] = x;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Rs[(b + r) * kPS + b + lane] = col[r];
        }
        __syncthreads();
        // blocks below the diagonal: T_IJ = -T_II sum_{J <= m < I} A_Im T_mJ
        for (int I = 1; I < 4; ++I) {
            f32x4 y = zero4();
            if (wave < I) {
                const int J = wave;
                f32x4 x = zero4();
                for (int m = J; m < I; ++m)
                    x = mma_f32_k16(rd4(Rs + (16 * I + ln) * kPS + 16 * m + 4 * lg),
                                    rdcol4(Rs + (16 * m + 4 * lg) * kPS + 16 * J + ln, kPS), x);
                y = mma_f32_k16(rd4(Rs + (16 * I + ln) * kPS + 16 * I + 4 * lg), x, zero4());
            }
            __syncthreads();
            if (wave < I) {
#pragma unroll
                for (int j = 0; j < 4; ++j) Rs[(16 * I + 4 * lg + j) * kPS + 16 * wave + ln] = -y[j];
            }
            __syncthreads();
        }
        for (int i = tid; i < 64 * 16; i += kBwdThreads) {
            const int r = i >> 4, c = 4 * (i & 15);
            wr4(item + IT::t + r * 64 + c, rd4(Rs + r * kPS + c));
        }

        // W = M (Gamma*K), stored transposed: tile (t block mt, channel block nt)
        for (int u = wave; u < 4 * KT; u += kBwdWaves) {
            const int mt = u / KT, nt = u % KT;
            const int c = 16 * nt + ln;
            f32x4 acc = zero4();
            auto av = [&](int kk) {
                const int s = 16 * kk + 4 * lg;
                return rd4(Rs + (16 * mt + ln) * kPS + s) * rd4(bet + s);
            };
            auto bv = [&](int kk) { return rdcol4(Ks + (16 * kk + 4 * lg) * PB + c, PB) * fpre[kk * D + c]; };
            if constexpr (F32IO) {
                for (int kk = 0; kk <= mt; ++kk) acc = mma_f32_k16(av(kk), bv(kk), acc);
            } else {
                // K16 tile mt + 1 of the last pair, when there is one, is the
                // zero block of T above the diagonal
                for (int kp = 0; 2 * kp <= mt; ++kp)
                    acc = mma_k32<false>(av(2 * kp), av(2 * kp + 1), bv(2 * kp), bv(2 * kp + 1), acc);
            }
            if constexpr (F32IO)
                wr4(item + IT::wt + (size_t)c * 64 + 16 * mt + 4 * lg, acc);
            else   // lane (n, g) holds W^T[16 nt + n][16 mt + 4 g + j]: A operand of W^T (-dV')
                store_split_half(item + IT::wt, nt * 2 + (mt >> 1), mt & 1, lane, acc);
        }
        // K~ = (gamma_C/Gamma)*K and gamma_C
        for (int i = tid; i < 64 * (D / 4); i += kBwdThreads) {
            const int r = i / (D / 4), c = 4 * (i % (D / 4));
            const f32x4 x = rd4(kB + r * PB + c) * rd4(fsuf + (r >> 4) * D + c);
            if constexpr (F32IO)
                wr4(item + IT::kt + (size_t)r * D + c, x);
            else   // A operand of K~ dS: row r = 16 rt + m, key c = 32 kp + 16 half + 4 g
                store_split_half(item + IT::kt, (r >> 4) * (D / 32) + (c >> 5), (c >> 4) & 1,
                                 (r & 15) + 16 * ((c & 15) >> 2), x);
        }
        for (int c = tid; c < D; c += kBwdThreads) item[IT::gam + c] = fast_exp2(span1<D>(bt, 0, 4, c));
        __syncthreads();

        // dO replaces K
        float *DOs = Ks;
        stage_quads<D, F32IO>(DOs, ocur, tid);
        __syncthreads();

        // Y = (Gamma*Q)^T dO, key-major [c][v]: tile (key block mt, value block nt)
        for (int u = wave; u < KT * KT; u += kBwdWaves) {
            const int mt = u / KT, nt = u % KT;
            const int c = 16 * mt + ln;
            f32x4 acc = zero4();
            auto av = [&](int kk) { return rdcol4(Qs + (16 * kk + 4 * lg) * PB + c, PB) * fpre[kk * D + c]; };
            auto bv = [&](int kk) { return rdcol4(DOs + (16 * kk + 4 * lg) * PB + 16 * nt + ln, PB); };
            if constexpr (F32IO) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mma_f32_k16(av(kk), bv(kk), acc);
            } else {
#pragma unroll
                for (int kp = 0; kp < 2; ++kp)
                    acc = mma_k32_exact_b(av(2 * kp), av(2 * kp + 1), bv(2 * kp), bv(2 * kp + 1), acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) item[IT::ys + (size_t)(16 * mt + 4 * lg + j) * D + 16 * nt + ln] = acc[j];
        }
        // X = P^T dO, stored transposed: tile (row block mt, value block nt)
        for (int u = wave; u < 4 * KT; u += kBwdWaves) {
            const int mt = u / KT, nt = u % KT;
            f32x4 acc = zero4();
            auto av = [&](int kk) { return rdcol4(Ps + (16 * kk + 4 * lg) * kPS + 16 * mt + ln, kPS); };
            auto bv = [&](int kk) { return rdcol4(DOs + (16 * kk + 4 * lg) * PB + 16 * nt + ln, PB); };
            if constexpr (F32IO) {
                for (int kk = mt; kk < 4; ++kk) acc = mma_f32_k16(av(kk), bv(kk), acc);
            } else {
                // K16 tile mt - 1 of the first pair, when there is one, is the
                // zero block of P above the diagonal
                for (int kp = mt >> 1; kp < 2; ++kp)
                    acc = mma_k32_exact_b(av(2 * kp), av(2 * kp + 1), bv(2 * kp), bv(2 * kp + 1), acc);
            }
            wr4(item + IT::xv + (size_t)(16 * nt + ln) * 64 + 16 * mt + 4 * lg, acc);
        }
        __syncthreads();   // LDS is restaged for the next item
    }
}

// ---------------------------------------------------------------------------
// Stage 3: the reverse chain.  Wave w of a workgroup owns 16 value columns;
// its slice of dS (D x 16) lives in accumulators, so both products of a step
// are wave-local:
//   dV' = X + K~ dS'           (accumulator of K~ dS' = B operand of W^T dV')
//   dS  = Y + gamma_C * dS' - W^T dV'
// K~ and W^T of the next chunk are staged during a step into the other half
// of a double buffer (one barrier per step): fp32 path, global -> registers
// -> padded LDS rows; bf16 path, split bf16 fragments copied global -> LDS
// directly, both products on split-bf16 MFMA.
// ---------------------------------------------------------------------------
template <int D>
struct ChainShape {
    static constexpr int KT = D / 16;
    static constexpr int NW = KT < 4 ? KT : 4;     // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int PB = D + 4;
    static constexpr int buf = 64 * PB + D * kPS;  // floats per buffer: K~ then W^T
    static constexpr int NS = 2 * 64 * D / 4 / NT; // float4 per thread per stage (fp32 path)
    static constexpr int NF = 2 * 64 * D * 4 / 1024; // 1 KiB pieces of [K~ | W^T] (bf16 path)
    static constexpr size_t lds_bytes = 2 * (size_t)buf * 4;
};

template <int D, bool F32IO>
__global__ void __launch_bounds__(ChainShape<D>::NT) bwd_chain_kernel(const int32_t *__restrict__ meta,
                                                                       const float *__restrict__ dhT,
                                                                       float *__restrict__ items, int N, int H,
                                                                       int max_chunks, int groups,
                                                                       float *__restrict__ dh0) {
    using IT = BwdItem<D>;
    using SH = ChainShape<D>;
    constexpr int KT = SH::KT, PB = SH::PB, NS = SH::NS;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int unit = blockIdx.x / groups, grp = blockIdx.x % groups;
    const int n = unit / H, h = unit % H;
    if (n >= N) return;
    const int ct = grp * SH::NW + wave;  // value column tile of this wave
    const int v = 16 * ct + ln;
    const int c_begin = meta[n], c_end = meta[n + 1];
    auto rec = [&](int c) { return items + ((size_t)h * max_chunks + c) * IT::floats; };

    const size_t sb = ((size_t)n * H + h) * D * D + (size_t)v * D + 4 * lg;
    f32x4 dS[KT];
#pragma unroll
    for (int rc = 0; rc < KT; ++rc) dS[rc] = dhT ? rd4(dhT + sb + 16 * rc) : zero4();

    // fp32 path: [K~ | W^T] fp32 rows through registers into padded LDS rows.
    // bf16 path: split bf16 fragments, copied straight into LDS, 1 KiB per
    // wave instruction.
    f32x4 st[F32IO ? NS : 1];
    auto copy_stage = [&](const float *src, float *dst) {
        const unsigned char *s8 = reinterpret_cast<const unsigned char *>(src);
        unsigned char *d8 = reinterpret_cast<unsigned char *>(dst);
        for (int f = wave; f < SH::NF; f += SH::NW)
            __builtin_amdgcn_global_load_lds(s8 + (size_t)f * 1024 + lane * 16,
                                             (__attribute__((address_space(3))) void *)(d8 + f * 1024), 16, 0, 0);
    };
    auto load_stage = [&](const float *src) {
#pragma unroll
        for (int s = 0; s < NS; ++s) st[s] = rd4(src + 4 * (tid + s * SH::NT));
    };
    auto store_stage = [&](float *dst) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int i = tid + s * SH::NT;  // float4 index into [K~ | W^T]
            if (i < 16 * D) {
                const int r = i / (D / 4), c = 4 * (i % (D / 4));
                wr4(dst + r * PB + c, st[s]);
            } else {
                const int j = i - 16 * D, r = j >> 4, c = 4 * (j & 15);
                wr4(dst + 64 * PB + r * kPS + c, st[s]);
            }
        }
    };
    f32x4 X[4], Y[KT], G[KT];
    auto fetch = [&](const float *it) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) X[rt] = rd4(it + IT::xv + (size_t)v * 64 + 16 * rt + 4 * lg);
#pragma unroll
        for (int rc = 0; rc < KT; ++rc) {
            Y[rc] = rdcol4(it + IT::ys + (size_t)(16 * rc + 4 * lg) * D + v, D);
            G[rc] = rd4(it + IT::gam + 16 * rc + 4 * lg);
        }
    };

    if (c_end > c_begin) {
        if constexpr (F32IO) {
            load_stage(rec(c_end - 1) + IT::kt);
            store_stage(lds);
        } else {
            copy_stage(rec(c_end - 1) + IT::kt, lds);
        }
        fetch(rec(c_end - 1));
        __builtin_amdgcn_s_waitcnt(0);   // the direct copies have landed
        __syncthreads();
        int b = 0;
        for (int c = c_end - 1; c >= c_begin; --c, b ^= 1) {
            const bool more = c > c_begin;
            const float *Kt = lds + b * SH::buf, *Wt = Kt + 64 * PB;
            f32x4 Xc[4], Yc[KT], Gc[KT];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) Xc[rt] = X[rt];
#pragma unroll
            for (int rc = 0; rc < KT; ++rc) {
                Yc[rc] = Y[rc];
                Gc[rc] = G[rc];
            }
            if (more) {
                if constexpr (F32IO)
                    load_stage(rec(c - 1) + IT::kt);
                else
                    copy_stage(rec(c - 1) + IT::kt, lds + (b ^ 1) * SH::buf);
                fetch(rec(c - 1));
            }
            f32x4 dv[4], nd[KT];
            if constexpr (F32IO) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f32x4 acc = Xc[rt];
#pragma unroll
                    for (int kk = 0; kk < KT; ++kk)
                        acc = mma_f32_k16(rd4(Kt + (16 * rt + ln) * PB + 16 * kk + 4 * lg), dS[kk], acc);
                    dv[rt] = acc;
                }
#pragma unroll
                for (int rc = 0; rc < KT; ++rc) {
                    f32x4 acc = Yc[rc] + Gc[rc] * dS[rc];
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
                        acc = mma_f32_k16(rd4(Wt + (16 * rc + ln) * kPS + 16 * kt + 4 * lg), -dv[kt], acc);
                    nd[rc] = acc;
                }
            } else {
                // bf16 path: both operands of each product split into bf16
                // hi + lo (three 16x16x32 MFMAs per pair of K16 tiles); K~ and
                // W^T arrive split, as fragments f = 2 KiB pieces of the buffer
                const unsigned char *fb = reinterpret_cast<const unsigned char *>(Kt);
                auto afrag = [&](int f, u32x4 &hi, u32x4 &lo) {
                    hi = *reinterpret_cast<const u32x4 *>(fb + (size_t)f * 2048 + lane * 16);
                    lo = *reinterpret_cast<const u32x4 *>(fb + (size_t)f * 2048 + 1024 + lane * 16);
                };
                u32x4 sh[KT / 2], sl[KT / 2];
#pragma unroll
                for (int kp = 0; kp < KT / 2; ++kp) quads_to_bf16_split(dS[2 * kp], dS[2 * kp + 1], sh[kp], sl[kp]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f32x4 acc = Xc[rt];
#pragma unroll
                    for (int kp = 0; kp < KT / 2; ++kp) {
                        u32x4 ah, al;
                        afrag(rt * (KT / 2) + kp, ah, al);
                        acc = mma3_bf16(ah, al, sh[kp], sl[kp], acc);
                    }
                    dv[rt] = acc;
                }
                u32x4 vh[2], vl[2];
#pragma unroll
                for (int kp = 0; kp < 2; ++kp) quads_to_bf16_split(-dv[2 * kp], -dv[2 * kp + 1], vh[kp], vl[kp]);
#pragma unroll
                for (int rc = 0; rc < KT; ++rc) {
                    f32x4 acc = Yc[rc] + Gc[rc] * dS[rc];
#pragma unroll
                    for (int kp = 0; kp < 2; ++kp) {
                        u32x4 ah, al;
                        afrag(2 * KT + rc * 2 + kp, ah, al);
                        acc = mma3_bf16(ah, al, vh[kp], vl[kp], acc);
                    }
                    nd[rc] = acc;
                }
            }
            float *it = rec(c);
            // dS' over Y (the same lanes read and write the same addresses),
            // dV' over X^T and row-major beside it
#pragma unroll
            for (int rc = 0; rc < KT; ++rc) {
#pragma unroll
                for (int j = 0; j < 4; ++j) it[IT::ys + (size_t)(16 * rc + 4 * lg + j) * D + v] = dS[rc][j];
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                wr4(it + IT::xv + (size_t)v * 64 + 16 * rt + 4 * lg, dv[rt]);
#pragma unroll
                for (int j = 0; j < 4; ++j) it[IT::dvr + (size_t)(16 * rt + 4 * lg + j) * D + v] = dv[rt][j];
            }
#pragma unroll
            for (int rc = 0; rc < KT; ++rc) dS[rc] = nd[rc];
            if constexpr (F32IO) {
                if (more) store_stage(lds + (b ^ 1) * SH::buf);
            } else {
                __builtin_amdgcn_s_waitcnt(0);   // the next chunk's direct copies have landed
            }
            __syncthreads();
        }
    }
    if (dh0) {
#pragma unroll
        for (int rc = 0; rc < KT; ++rc) wr4(dh0 + sb + 16 * rc, dS[rc]);
    }
}

// ---------------------------------------------------------------------------
// Stage 4: per (chunk, head), every input gradient.
// ---------------------------------------------------------------------------
template <int D, bool F32IO>
__global__ void __launch_bounds__(kBwdThreads) bwd_grad_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ vin,
    const float *__restrict__ z, const float *__restrict__ A, const float *__restrict__ beta,
    const float *__restrict__ h0, const void *__restrict__ dO, const int32_t *__restrict__ meta,
    const int4 *__restrict__ table, const int32_t *__restrict__ ck_off, const float *__restrict__ ck, int ck_cap,
    int N, int H, int max_chunks, const float *__restrict__ items, float *__restrict__ gq,
    float *__restrict__ gk, float *gv, float *__restrict__ gz, float *__restrict__ gbeta,
    float *__restrict__ dA_part) {
    using IT = BwdItem<D>;
    using SL = GradLds<D>;
    constexpr int PB = D + 4, KT = D / 16;
    constexpr int NU = (4 * KT + kBwdWaves - 1) / kBwdWaves;  // [t][c] tiles per wave
    static_assert(kBwdWaves % KT == 0, "a wave's [t][c] tiles share one column block");
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float *Ks = lds + SL::k, *Gb = lds + SL::gb, *Xs = lds + SL::x, *S0 = lds + SL::s0, *S1 = lds + SL::s1;
    float *bet = lds + SL::beta, *bt = lds + SL::bt, *pd = lds + SL::pd, *dgc = lds + SL::dgc;
    float *red = lds + SL::red, *part = lds + SL::part;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave index in an SGPR
    const int total = meta[N] * H;
    int it = blockIdx.x;
    if (it >= total) return;
    auto rec = [&](int i) { return items + ((size_t)(i % H) * max_chunks + i / H) * IT::floats; };
    // state at the start of chunk `chunk` of sequence n, [v][c]; NULL = zero
    auto state_of = [&](int chunk, int h, int n) -> const float * {
        const int j = chunk - meta[n];
        if (j == 0) return h0 ? h0 + ((size_t)n * H + h) * D * D : nullptr;
        if (!ck) return nullptr;
        const int idx = ck_off[n] + j - 1;
        return (idx >= 0 && idx < ck_cap) ? ck + ((size_t)idx * H + h) * D * D : nullptr;
    };
    GradIn<D, F32IO> R;
    int4 ent = table[it / H];
    load_grad_rows<D, F32IO>(R, k, vin, beta, rec(it) + IT::t, ent.y, ent.z, it % H, H, threadIdx.x);
    load_grad_z<D, F32IO>(R, z, ent.y, ent.z, it % H, H, threadIdx.x);
    load_grad_state<D, F32IO>(R, state_of(it / H, it % H, ent.x), wave % KT, threadIdx.x & 15, (threadIdx.x >> 4) & 3);

    // persistent: items blockIdx.x, + gridDim.x, ...  Every LDS region but
    // `part` is last read before an item's final barrier, and `part` is next
    // written many barriers into the following item, so items need no barrier
    // between them.
    for (; it < total; it += gridDim.x) {
        // thread and lane coordinates, rebuilt per item (see opaque_zero)
        const int tid = (int)threadIdx.x + opaque_zero();
        const int lane = tid & 63, ln = lane & 15, lg = lane >> 4;
        const int chunk = it / H, h = it % H;
        const int n = ent.x, t0 = ent.y, L = ent.z;
        const float *item = rec(it);
        const float *dvp = item + IT::xv;   // dV'^T [v][t]
        const float *dvr = item + IT::dvr;  // dV' [t][v]
        const float *dsp = item + IT::ys;   // dS' [c][v]
        const float ea = __expf(A[h]);
        const float *Sg = state_of(chunk, h, n);   // the state at the chunk's start
        auto row_io = [&](const void *p, int r, int c) -> f32x4 {
            return r < L ? load_io4<F32IO>(p, ((size_t)(t0 + r) * H + h) * D + c) : zero4();
        };

        // ---- K, the block log-decays, V, beta, T (from the registers)
        stage_quads<D, F32IO>(Ks, R.k, tid);
        stage_quads<D, F32IO>(Xs, R.v, tid);
        if (tid < 4 * D) {
            const int c = tid % D, I = tid / D;
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * I + i;
                run += r < L ? gate_log2(ea, R.z[i]) : 0.f;
                Gb[r * PB + c] = run;
            }
            bt[I * D + c] = run;
        }
        if (tid < 64) bet[tid] = R.beta;
        f32x4 tq[64 * 16 / kBwdThreads];
#pragma unroll
        for (int s = 0; s < 64 * 16 / kBwdThreads; ++s) tq[s] = R.t[s];
        __syncthreads();

        // ---- V~ = V - (Gamma*K) S, in place
        for (int u = wave; u < 4 * KT; u += kBwdWaves) {
            const int mt = u / KT, nt = u % KT;
            f32x4 acc = zero4();
            if (Sg) {
                const int r = 16 * mt + ln;
                auto kg = [&](int kk) {
                    const int c = 16 * kk + 4 * lg;
                    return rd4(Ks + r * PB + c) * exp2x4(rd4(Gb + r * PB + c) + span4<D>(bt, 0, mt, c));
                };
                // B operands: the state's rows 16 nt + ln, fetched during the previous item
#pragma unroll
                for (int kp = 0; kp < KT / 2; ++kp)
                    acc = mma_k32<F32IO>(kg(2 * kp), kg(2 * kp + 1), R.s[2 * kp], R.s[2 * kp + 1], acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) Xs[(16 * mt + 4 * lg + j) * PB + 16 * nt + ln] -= acc[j];
        }
#pragma unroll
        for (int s = 0; s < 64 * 16 / kBwdThreads; ++s) {
            const int i = tid + s * kBwdThreads, r = i >> 4, c = 4 * (i & 15);
            wr4(S0 + r * kPS + c, tq[s]);
        }
        __syncthreads();

        // ---- dM = dV' V~^T -> S1;  V' = M V~ (registers, then over V~);
        //      dV = M^T dV' -> gv
        for (int u = wave; u < 16; u += kBwdWaves) {
            const int mt = u >> 2, nt = u & 3;
            f32x4 acc = zero4();
            {
                const float *ar = dvr + (size_t)(16 * mt + ln) * D + 4 * lg, *br = Xs + (16 * nt + ln) * PB + 4 * lg;
#pragma unroll
                for (int kp = 0; kp < KT / 2; ++kp)
                    acc = mma_k32<F32IO>(rd4(ar + 32 * kp), rd4(ar + 32 * kp + 16), rd4(br + 32 * kp),
                                         rd4(br + 32 * kp + 16), acc);
            }
            // dbeta_j partial over the tile's rows: sum_t dM_tj T_tj
            float p = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                S1[(16 * mt + 4 * lg + j) * kPS + 16 * nt + ln] = acc[j];
                p += acc[j] * S0[(16 * mt + 4 * lg + j) * kPS + 16 * nt + ln];
            }
            p += __shfl_xor(p, 16);
            p += __shfl_xor(p, 32);
            if (lg == 0) red[mt * 64 + 16 * nt + ln] = p;
        }
        f32x4 vp[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = wave + i * kBwdWaves;
            vp[i] = zero4();
            if (u < 4 * KT) {
                const int mt = u / KT, nt = u % KT;
                auto av = [&](int kk) {
                    const int s = 16 * kk + 4 * lg;
                    return rd4(S0 + (16 * mt + ln) * kPS + s) * rd4(bet + s);
                };
                auto bv = [&](int kk) { return rdcol4(Xs + (16 * kk + 4 * lg) * PB + 16 * nt + ln, PB); };
                if constexpr (F32IO) {
                    for (int kk = 0; kk <= mt; ++kk) vp[i] = mma_f32_k16(av(kk), bv(kk), vp[i]);
                } else {
                    // the pair's K16 tile mt + 1, when there is one, is a zero block of T
                    for (int kp = 0; 2 * kp <= mt; ++kp)
                        vp[i] = mma_k32<false>(av(2 * kp), av(2 * kp + 1), bv(2 * kp), bv(2 * kp + 1), vp[i]);
                }
            }
        }
        for (int u = wave; u < 4 * KT; u += kBwdWaves) {
            const int mt = u / KT, nt = u % KT;
            const int v = 16 * nt + ln;
            f32x4 acc = zero4();
            const float bm = bet[16 * mt + ln];
            auto av = [&](int kk) { return rdcol4(S0 + (16 * kk + 4 * lg) * kPS + 16 * mt + ln, kPS) * bm; };
            auto bv = [&](int kk) { return rd4(dvp + (size_t)v * 64 + 16 * kk + 4 * lg); };
            if constexpr (F32IO) {
                for (int kk = mt; kk < 4; ++kk) acc = mma_f32_k16(av(kk), bv(kk), acc);
            } else {
                // the pair's K16 tile mt - 1, when there is one, is a zero block of T
                for (int kp = mt >> 1; kp < 2; ++kp)
                    acc = mma_k32<false>(av(2 * kp), av(2 * kp + 1), bv(2 * kp), bv(2 * kp + 1), acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * mt + 4 * lg + j;
                if (r < L) gv[((size_t)(t0 + r) * H + h) * D + v] = acc[j];
            }
        }
        __threadfence_block();
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = wave + i * kBwdWaves;
            if (u < 4 * KT) {
                const int mt = u / KT, nt = u % KT;
                if constexpr (F32IO) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) Xs[(16 * mt + 4 * lg + j) * PB + 16 * nt + ln] = vp[i][j];
                } else {
                    // bf16 path: V' split once into bf16 hi + lo; each 16-byte row
                    // quad holds [4 hi | 4 lo] in place of its four floats, the
                    // order quads_to_bf16_split gives, so readers take the
                    // fragments as loaded
                    uint16_t *xb = reinterpret_cast<uint16_t *>(Xs);
                    const int c = 16 * nt + ln;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float x = vp[i][j];
                        const uint32_t hb = f32x2_to_bf16x2(x, 0.f) & 0xffffu;
                        const uint32_t lb = f32x2_to_bf16x2(x - bf16_bits_to_f32(hb), 0.f) & 0xffffu;
                        const size_t e = (size_t)(16 * mt + 4 * lg + j) * (2 * PB) + (c >> 2) * 8 + (c & 3);
                        xb[e] = (uint16_t)hb;
                        xb[e + 4] = (uint16_t)lb;
                    }
                }
            }
        }

        // ---- E = (dM Diag(beta)) T^T (registers)
        f32x4 e[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = wave + i * kBwdWaves, mt = u >> 2, nt = u & 3;
            e[i] = zero4();
            auto av = [&](int kk) {
                const int s = 16 * kk + 4 * lg;
                return rd4(S1 + (16 * mt + ln) * kPS + s) * rd4(bet + s);
            };
            auto bv = [&](int kk) { return rd4(S0 + (16 * nt + ln) * kPS + 16 * kk + 4 * lg); };
            if constexpr (F32IO) {
                for (int kk = 0; kk <= nt; ++kk) e[i] = mma_f32_k16(av(kk), bv(kk), e[i]);
            } else {
                // the pair's K16 tile nt + 1, when there is one, is a zero block of T
                for (int kp = 0; 2 * kp <= nt; ++kp)
                    e[i] = mma_k32<false>(av(2 * kp), av(2 * kp + 1), bv(2 * kp), bv(2 * kp + 1), e[i]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = wave + i * kBwdWaves, mt = u >> 2, nt = u & 3;
#pragma unroll
            for (int j = 0; j < 4; ++j) S1[(16 * mt + 4 * lg + j) * kPS + 16 * nt + ln] = e[i][j];
        }
        __syncthreads();
        // ---- dA_kk = -StrictTril(T^T E) (registers, then over T)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = wave + i * kBwdWaves, mt = u >> 2, nt = u & 3;
            e[i] = zero4();
            if (nt <= mt) {
                auto av = [&](int kk) { return rdcol4(S0 + (16 * kk + 4 * lg) * kPS + 16 * mt + ln, kPS); };
                auto bv = [&](int kk) { return rdcol4(S1 + (16 * kk + 4 * lg) * kPS + 16 * nt + ln, kPS); };
                if constexpr (F32IO) {
                    for (int kk = mt; kk < 4; ++kk) e[i] = mma_f32_k16(av(kk), bv(kk), e[i]);
                } else {
                    // the pair's K16 tile mt - 1, when there is one, is a zero block of T
                    for (int kp = mt >> 1; kp < 2; ++kp)
                        e[i] = mma_k32<false>(av(2 * kp), av(2 * kp + 1), bv(2 * kp), bv(2 * kp + 1), e[i]);
                }
            }
        }
        __syncthreads();
        // dA_kk over T;  dbeta_r partials sum_i dA_kk,ri R_ri over the tile's columns
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = wave + i * kBwdWaves, mt = u >> 2, nt = u & 3;
            f32x4 p = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * mt + 4 * lg + j, w = 16 * nt + ln;
                const float x = w < r ? -e[i][j] : 0.f;
                S0[r * kPS + w] = x;
                if (w < r) p[j] = x * item[IT::r + r * 64 + w];
            }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) p[j] += __shfl_xor(p[j], m);
            }
            if (ln == 0) wr4(red + 256 + nt * 64 + 16 * mt + 4 * lg, p);
        }
        __syncthreads();
        // ---- dbeta = column sums of dM o T + row sums of dA_kk o R
        if (tid < 64 && tid < L) {
            float s = 0.f;
            for (int m = 0; m < 4; ++m) s += red[m * 64 + tid];
            for (int m = 0; m < 4; ++m) s += red[256 + m * 64 + tid];
            gbeta[(size_t)(t0 + tid) * H + h] = s;
        }

        // ---- dP = Tril(dO V'^T): the strictly lower part -> S1 (E is dead), the
        //      diagonal -> pd.  A diagonal term dP_rr q_r k_r enters the log-decay
        //      gradient of row r twice with opposite signs (its decay factor is 1),
        //      so it is kept out of the decay-masked sums and added to dq and dk
        //      on its own;  the [t][c] products that
        //      read S, dS' or dV: dQ_S = Gamma*(dO S^T), dKg = -Gamma*(dV S^T),
        //      dKt = (gamma_C/Gamma)*(V' dS'^T)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = wave + i * kBwdWaves, mt = u >> 2, nt = u & 3;
            f32x4 acc = zero4();
            if (nt <= mt) {
                const float *br = Xs + (16 * nt + ln) * PB + 4 * lg;
#pragma unroll
                for (int kp = 0; kp < KT / 2; ++kp) {
                    const int c0 = 32 * kp + 4 * lg, c1 = c0 + 16;
                    if constexpr (F32IO)
                        acc = mma_k32<true>(row_io(dO, 16 * mt + ln, c0), row_io(dO, 16 * mt + ln, c1),
                                            rd4(br + 32 * kp), rd4(br + 32 * kp + 16), acc);
                    else {   // dO is exactly bf16; V' is stored split
                        const u32x4 q0 = *reinterpret_cast<const u32x4 *>(br + 32 * kp);
                        const u32x4 q1 = *reinterpret_cast<const u32x4 *>(br + 32 * kp + 16);
                        const u32x4 ah = quads_to_bf16(row_io(dO, 16 * mt + ln, c0), row_io(dO, 16 * mt + ln, c1));
                        acc = mma_bf16_k32(ah, u32x4{q0[0], q0[1], q1[0], q1[1]}, acc);
                        acc = mma_bf16_k32(ah, u32x4{q0[2], q0[3], q1[2], q1[3]}, acc);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * mt + 4 * lg + j, s = 16 * nt + ln;
                S1[r * kPS + s] = s < r ? acc[j] : 0.f;
                if (s == r) pd[r] = acc[j];
            }
        }
        static_assert((4 * KT) % kBwdWaves == 0, "every wave has NU tiles");
        f32x4 dq[NU], dkg[NU], dkt[NU], dki[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i) dq[i] = dkg[i] = dkt[i] = dki[i] = zero4();
        // Every tile of a wave has the same key-column block ct = wave % KT; its
        // row blocks are (wave + i kBwdWaves) / KT.  The loop runs over pairs of
        // value tiles (kp) outside the wave's tiles, so the S and dS' fragments of
        // a pair are loaded, and on the bf16 path split into bf16 hi + lo, once
        // for all of them.
        const int ct = wave % KT, c = 16 * ct + ln;
        // B fragments of S: S_cv for c = 16 ct + ln, v = 16 kk + 4 lg + j
        f32x4 sfr[KT];
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) sfr[kk] = Sg ? rdcol4(Sg + (size_t)(16 * kk + 4 * lg) * D + c, D) : zero4();
        float gc = 0.f;   // dgC_c = sum_v dS'_cv S_cv
        auto products = [&](auto has_state) {
            constexpr bool HS = decltype(has_state)::value;
#pragma unroll
            for (int kp = 0; kp < KT / 2; ++kp) {
                const int v0 = 32 * kp + 4 * lg, v1 = v0 + 16;
                const f32x4 ds0 = rd4(dsp + (size_t)c * D + v0), ds1 = rd4(dsp + (size_t)c * D + v1);
                const f32x4 s0 = sfr[2 * kp], s1 = sfr[2 * kp + 1];
                u32x4 dsh, dsl, sh, sl;
                if constexpr (!F32IO) {
                    quads_to_bf16_split(ds0, ds1, dsh, dsl);
                    if constexpr (HS) quads_to_bf16_split(s0, s1, sh, sl);
                }
                if constexpr (HS) {
                    gc += s0[0] * ds0[0] + s0[1] * ds0[1] + s0[2] * ds0[2] + s0[3] * ds0[3];
                    gc += s1[0] * ds1[0] + s1[1] * ds1[1] + s1[2] * ds1[2] + s1[3] * ds1[3];
                }
#pragma unroll
                for (int i = 0; i < NU; ++i) {
                    const int r = 16 * ((wave + i * kBwdWaves) / KT) + ln;
                    const bool rok = r < L;
                    const size_t orow = ((size_t)(t0 + r) * H + h) * D;
                    if constexpr (F32IO) {
                        dkt[i] = mma_k32<true>(rd4(Xs + r * PB + v0), rd4(Xs + r * PB + v1), ds0, ds1, dkt[i]);
                    } else {   // V' is stored split
                        const u32x4 q0 = *reinterpret_cast<const u32x4 *>(Xs + r * PB + v0);
                        const u32x4 q1 = *reinterpret_cast<const u32x4 *>(Xs + r * PB + v1);
                        dkt[i] = mma3_bf16(u32x4{q0[0], q0[1], q1[0], q1[1]}, u32x4{q0[2], q0[3], q1[2], q1[3]}, dsh,
                                           dsl, dkt[i]);
                    }
                    if constexpr (HS) {
                        const f32x4 z0 = rok ? rd4(gv + orow + v0) : zero4(), z1 = rok ? rd4(gv + orow + v1) : zero4();
                        if constexpr (F32IO) {
                            dq[i] = mma_k32<true>(row_io(dO, r, v0), row_io(dO, r, v1), s0, s1, dq[i]);
                            dkg[i] = mma_k32<true>(z0, z1, s0, s1, dkg[i]);
                        } else {
                            // dO is bf16 already: its hi part is exact and its lo part zero
                            u32x4 dh = u32x4{0u, 0u, 0u, 0u};
                            if (rok) {
                                const uint16_t *dp = reinterpret_cast<const uint16_t *>(dO) + orow;
                                const u32x2 w0 = *reinterpret_cast<const u32x2 *>(dp + v0);
                                const u32x2 w1 = *reinterpret_cast<const u32x2 *>(dp + v1);
                                dh = u32x4{w0[0], w0[1], w1[0], w1[1]};
                            }
                            dq[i] = mma_bf16_k32(dh, sh, dq[i]);
                            dq[i] = mma_bf16_k32(dh, sl, dq[i]);
                            u32x4 zh, zl;
                            quads_to_bf16_split(z0, z1, zh, zl);
                            dkg[i] = mma3_bf16(zh, zl, sh, sl, dkg[i]);
                        }
                    }
                }
            }
        };
        if (Sg)
            products(std::true_type{});
        else
            products(std::false_type{});
        // the wave that holds row block 0 of column block ct
        gc += __shfl_xor(gc, 16);
        gc += __shfl_xor(gc, 32);
        if (wave < KT && lg == 0) dgc[c] = gc;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int rb = (wave + i * kBwdWaves) / KT;
            // lane (n = c, g) holds rows 16 rb + 4 lg + j
            const f32x4 g = rdcol4(Gb + (16 * rb + 4 * lg) * PB + c, PB);
            dq[i] *= exp2x4(g + splat4(span1<D>(bt, 0, rb, c)));
            dkg[i] *= -exp2x4(g + splat4(span1<D>(bt, 0, rb, c)));
            dkt[i] *= exp2x4(splat4(span1<D>(bt, rb, 4, c)) - g);
        }
        __syncthreads();

        // ---- Q replaces V'
        float *Qs = Xs;
        stage_rows<D, F32IO>(Qs, q, t0, L, h, H, tid);
        __syncthreads();

        // ---- the decay-masked products of dP (S1) and dA_kk (S0, dR = Diag(beta) dA_kk)
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = wave + i * kBwdWaves;
            if (u >= 4 * KT) continue;
            const int rb = u / KT, ct = u % KT;
            const int c = 16 * ct + ln;
            const float gmid = Gb[(16 * rb + 7) * PB + c];
            const f32x4 grow = rdcol4(Gb + (16 * rb + 4 * lg) * PB + c, PB);
            // forward direction, rows r in block rb:
            //   sum_{i <= r} X_ri k_i exp2(G_r - G_i),  X = dP (to dQ) and dR (to dK)
            f32x4 qo = zero4(), ko = zero4(), qd = zero4(), kd = zero4();
            const float br = bet[16 * rb + ln];
            for (int J = 0; J <= rb; ++J) {
                const int i0 = 16 * J + 4 * lg;
                const f32x4 gi = rdcol4(Gb + i0 * PB + c, PB);
                const f32x4 fb = (J < rb) ? splat4(span1<D>(bt, J, rb, c)) - gi : splat4(gmid) - gi;
                const f32x4 bk = rdcol4(Ks + i0 * PB + c, PB) * exp2x4(fb);
                const f32x4 ap = rd4(S1 + (16 * rb + ln) * kPS + 16 * J + 4 * lg);
                const f32x4 ar = rd4(S0 + (16 * rb + ln) * kPS + 16 * J + 4 * lg) * br;
                if (J < rb) {
                    qo = mma_f32_k16(ap, bk, qo);
                    ko = mma_f32_k16(ar, bk, ko);
                } else {
                    qd = mma_f32_k16(ap, bk, qd);
                    kd = mma_f32_k16(ar, bk, kd);
                }
            }
            const f32x4 fo = exp2x4(grow), fd = exp2x4(grow - splat4(gmid));
            dq[i] += qo * fo + qd * fd;
            dkg[i] += ko * fo + kd * fd;
            // backward direction, rows i in block rb:
            //   sum_{r >= i} (dP_ri q_r + dR_ri k_r) exp2(G_r - G_i)
            f32x4 xo = zero4(), xd = zero4();
            for (int I = rb; I < 4; ++I) {
                const int r0 = 16 * I + 4 * lg;
                const f32x4 gr = rdcol4(Gb + r0 * PB + c, PB);
                const f32x4 fr = (I > rb) ? gr + splat4(span1<D>(bt, rb + 1, I, c)) : gr - splat4(gmid);
                const f32x4 ex = exp2x4(fr);
                const f32x4 bq = rdcol4(Qs + r0 * PB + c, PB) * ex;
                const f32x4 bk = rdcol4(Ks + r0 * PB + c, PB) * ex;
                const f32x4 ap = rdcol4(S1 + r0 * kPS + 16 * rb + ln, kPS);
                const f32x4 ar = rdcol4(S0 + r0 * kPS + 16 * rb + ln, kPS) * rd4(bet + r0);
                if (I > rb) {
                    xo = mma_f32_k16(ap, bq, xo);
                    xo = mma_f32_k16(ar, bk, xo);
                } else {
                    xd = mma_f32_k16(ap, bq, xd);
                    xd = mma_f32_k16(ar, bk, xd);
                }
            }
            dki[i] = xo * exp2x4(splat4(bt[rb * D + c]) - grow) + xd * exp2x4(splat4(gmid) - grow);
        }

        // ---- outputs dq, dk; the log-decay gradient terms (registers)
        f32x4 gG[NU], gKt[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = wave + i * kBwdWaves;
            gG[i] = gKt[i] = zero4();
            if (u >= 4 * KT) continue;
            const int rb = u / KT, ct = u % KT;
            const int c = 16 * ct + ln;
            const f32x4 kv = rdcol4(Ks + (16 * rb + 4 * lg) * PB + c, PB);
            const f32x4 qv = rdcol4(Qs + (16 * rb + 4 * lg) * PB + c, PB);
            gG[i] = kv * (dkg[i] - dki[i]) + qv * dq[i];
            gKt[i] = kv * dkt[i];
            const f32x4 pdr = rd4(pd + 16 * rb + 4 * lg);
            const f32x4 dqo = dq[i] + pdr * kv;
            const f32x4 dko = dkg[i] + dki[i] + dkt[i] + pdr * qv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rb + 4 * lg + j;
                if (r < L) {
                    const size_t o = ((size_t)(t0 + r) * H + h) * D + c;
                    gq[o] = dqo[j];
                    gk[o] = dko[j];
                }
            }
        }
        __syncthreads();
        // gradient of the log-decay over S0|S1, the K~ terms over K
        float *Gg = S0, *Gt = Ks;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = wave + i * kBwdWaves;
            if (u >= 4 * KT) continue;
            const int rb = u / KT, ct = u % KT;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rb + 4 * lg + j;
                Gg[r * PB + 16 * ct + ln] = gG[i][j];
                Gt[r * PB + 16 * ct + ln] = gKt[i][j];
            }
        }
        __syncthreads();
        // per channel: block sums, then the cumulative sums inside each block:
        //   dg_t = sum_{r >= t} gG_r + sum_{r < t} gKt_r + dgC * gamma_C
        // (gKt_r = k_r dK~_r: the factor gamma_C / Gamma_r depends on the gates of
        // rows r + 1 .. C only, so it is summed forward, not as total - suffix)
        // the next item's rows, beta and T, into registers while this one
        // finishes (its gate logits follow once the dz pass is done).  The
        // loads are issued on every pass, the last one reloading this item,
        // so that the registers are fully redefined and no old value stays
        // live across the item.
        const int it_next = it + gridDim.x < total ? it + gridDim.x : it;
        ent = table[it_next / H];
        load_grad_rows<D, F32IO>(R, k, vin, beta, rec(it_next) + IT::t, ent.y, ent.z, it_next % H, H, tid);
        load_grad_state<D, F32IO>(R, state_of(it_next / H, it_next % H, ent.x), wave % KT, ln, lg);
        float dA_acc = 0.f;
        float zr[16];   // this thread's gate logits, fetched before the block sums
        if (tid < 4 * D) {
            const int c = tid % D, I = tid / D;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * I + i;
                zr[i] = r < L ? z[((size_t)(t0 + r) * H + h) * D + c] : 0.f;
            }
            float s = 0.f, st = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s += Gg[(16 * I + i) * PB + c];
                st += Gt[(16 * I + i) * PB + c];
            }
            red[I * D + c] = s;
            red[(4 + I) * D + c] = st;
        }
        __syncthreads();
        if (tid < 4 * D) {
            const int c = tid % D, I = tid / D;
            float fw[16];
            float pre = 0.f;
            for (int m = 0; m < I; ++m) pre += red[(4 + m) * D + c];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                fw[i] = pre;
                pre += Gt[(16 * I + i) * PB + c];
            }
            const float base = dgc[c] * fast_exp2(span1<D>(bt, 0, 4, c));
            float run = 0.f;
            for (int m = I + 1; m < 4; ++m) run += red[m * D + c];
#pragma unroll
            for (int i = 15; i >= 0; --i) {
                const int r = 16 * I + i;
                run += Gg[r * PB + c];
                const float dg = run + fw[i] + base;
                if (r < L) {
                    const size_t o = ((size_t)(t0 + r) * H + h) * D + c;
                    // sigmoid'(x) = e / (1 + e)^2 with e = exp(-|x|): no cancellation
                    // where the gate saturates
                    const float x = ea * zr[i];
                    const float ex = fast_exp2(-fabsf(x) * kLog2e);
                    const float dx = dg * -5.0f * ex * __builtin_amdgcn_rcpf((1.f + ex) * (1.f + ex));
                    gz[o] = dx * ea;
                    dA_acc += dx * x;
                }
            }
        }
        load_grad_z<D, F32IO>(R, z, ent.y, ent.z, it_next % H, H, tid);
        // fixed-order block reduction of the A gradient
        for (int off = 32; off > 0; off >>= 1) dA_acc += __shfl_xor(dA_acc, off);
        if (lane == 0) part[wave] = dA_acc;
        __syncthreads();
        if (tid == 0) {
            float s = 0.f;
            for (int w = 0; w < kBwdWaves; ++w) s += part[w];
            dA_part[(size_t)chunk * H + h] = s;
        }
    }
}

// Stage 5: dA[h] = sum over chunks of the per-(chunk, head) parts.
__global__ void __launch_bounds__(256) bwd_dA_kernel(const int32_t *__restrict__ meta, int N, int H,
                                                     const float *__restrict__ part, float *__restrict__ dA) {
    __shared__ float red[256];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int total = meta[N];
    float s = 0.f;
    for (int c = tid; c < total; c += 256) s += part[(size_t)c * H + h];
    red[tid] = s;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) red[tid] += red[tid + off];
        __syncthreads();
    }
    if (tid == 0) dA[h] = red[0];
}

template <int D, bool F32IO>
int launch_backward_t(const BackwardArgs &a) {
    const BackwardPlan &p = a.plan;
    unsigned char *fws = a.ws + p.off_fwd;
    PrefillArgs fa;
    fa.f32io = F32IO;
    fa.q = a.q; fa.k = a.k; fa.v = a.v; fa.z = a.z; fa.A = a.A; fa.beta = a.beta; fa.h0 = a.h0;
    fa.cu = a.cu;
    fa.N = a.N; fa.T = a.T; fa.H = a.H; fa.dk = D; fa.dv = D;
    fa.o = a.ws + p.off_o;
    fa.hT = nullptr;
    float *ck = p.ck_cap > 0 ? reinterpret_cast<float *>(a.ws + p.off_ck) : nullptr;
    fa.ck = ck;
    fa.ck_offsets = nullptr;
    fa.ck_interval = ck ? kChunk : 0;
    fa.ws = fws;
    fa.plan = p.fwd;
    fa.stream = a.stream;
    if (launch_prefill(fa) != 0) return -1;

    const int32_t *meta = reinterpret_cast<const int32_t *>(fws + p.fwd.off_meta);
    const int4 *table = reinterpret_cast<const int4 *>(fws + p.fwd.off_table);
    const int32_t *ck_off = reinterpret_cast<const int32_t *>(fws + p.fwd.off_ckoff);
    float *items = reinterpret_cast<float *>(a.ws + p.off_items);
    float *part = reinterpret_cast<float *>(a.ws + p.off_dA);
    const int max_chunks = p.fwd.max_chunks;
    const long long blocks = (long long)max_chunks * a.H;

    if (blocks > 0) {
        const size_t lds = sizeof(float) * LocalLds<D>::floats;
        if (!set_lds(&bwd_local_kernel<D, F32IO>, lds)) return -1;
        const unsigned grid = (unsigned)std::min<long long>(blocks, (long long)device_cus());
        hipLaunchKernelGGL((bwd_local_kernel<D, F32IO>), dim3(grid), dim3(kBwdThreads), lds, a.stream,
                           a.q, a.k, a.z, a.A, a.beta, a.dO, meta, table, a.N, a.H, max_chunks, items);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    if (a.N > 0) {
        using SH = ChainShape<D>;
        const int groups = SH::KT / SH::NW;
        if (!set_lds(&bwd_chain_kernel<D, F32IO>, SH::lds_bytes)) return -1;
        hipLaunchKernelGGL((bwd_chain_kernel<D, F32IO>), dim3(a.N * a.H * groups), dim3(SH::NT), SH::lds_bytes,
                           a.stream, meta, a.dhT, items, a.N, a.H, max_chunks, groups, a.gh0);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    if (blocks > 0) {
        const size_t lds = sizeof(float) * GradLds<D>::floats;
        if (!set_lds(&bwd_grad_kernel<D, F32IO>, lds)) return -1;
        const unsigned grid = (unsigned)std::min<long long>(blocks, (long long)device_cus());
        hipLaunchKernelGGL((bwd_grad_kernel<D, F32IO>), dim3(grid), dim3(kBwdThreads), lds, a.stream,
                           a.q, a.k, a.v, a.z, a.A, a.beta, a.h0, a.dO, meta, table, ck_off, ck, p.ck_cap, a.N,
                           a.H, max_chunks, items, a.gq, a.gk, a.gv, a.gz, a.gbeta, part);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    hipLaunchKernelGGL(bwd_dA_kernel, dim3(a.H), dim3(256), 0, a.stream, meta, a.N, a.H, part, a.gA);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

size_t backward_item_bytes(int d) {
    switch (d) {
        case 32: return BwdItem<32>::floats * 4;
        case 64: return BwdItem<64>::floats * 4;
        case 128: return BwdItem<128>::floats * 4;
    }
    return 0;
}

static size_t align256b(size_t x) { return (x + 255) & ~(size_t)255; }

bool plan_backward(int N, int T, int H, int d, bool f32io, int P, BackwardPlan *p) {
    if (!plan_prefill(N, T, H, d, d, f32io, P, 1, &p->fwd)) return false;
    const size_t item = backward_item_bytes(d);
    if (item == 0) return false;
    p->ck_cap = T / kChunk;
    p->off_fwd = 0;
    // The forward's slabs and its o are dead once the forward has run (the
    // backward kernels read its chunk table and the stored states only), so
    // the per-(chunk, head) records start where the slabs do and run over o.
    // The states and the dA parts are live with the records and come after.
    p->off_o = align256b(p->fwd.total);
    const size_t o_end = p->off_o + align256b((size_t)T * H * d * (f32io ? 4 : 2));
    p->off_items = align256b(p->fwd.off_slabs);
    const size_t items_end = p->off_items + (size_t)H * p->fwd.max_chunks * item;
    p->off_ck = align256b(std::max(o_end, items_end));
    p->off_dA = p->off_ck + align256b((size_t)p->ck_cap * H * d * d * 4);
    p->total = p->off_dA + align256b((size_t)p->fwd.max_chunks * H * 4);
    return true;
}

int launch_prefill_backward(const BackwardArgs &a) {
    switch (a.d) {
        case 32: return a.f32io ? launch_backward_t<32, true>(a) : launch_backward_t<32, false>(a);
        case 64: return a.f32io ? launch_backward_t<64, true>(a) : launch_backward_t<64, false>(a);
        case 128: return a.f32io ? launch_backward_t<128, true>(a) : launch_backward_t<128, false>(a);
    }
    return -1;
}

}  // namespace kda
