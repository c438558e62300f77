// kda_prefill.hip -- chunkwise-parallel KDA prefill for gfx950.
//
// Three kernels on the caller's stream:
//   chunk_table_kernel  cu_seqlens -> first chunk of every sequence and a
//                       (sequence, first token, length) record per chunk;
//                       chunks of 64 tokens start at every sequence start.
//   intra_kernel        one workgroup per (chunk, head): the bounded gate,
//                       chunk-local log-decays, the decay-rescaled Gram
//                       matrices, the unit-lower-triangular solve and the
//                       W / U products.  Writes one "slab" of MFMA-ready
//                       fragments per (chunk, head).
//   inter_kernel        one wavefront per (sequence, head, 16 value columns):
//                       walks the sequence's chunks in order, carrying the
//                       fp32 state in MFMA accumulators.
//
// The algebra is the chunk form of the s1mplewind "kimi-k3" notes (section
// "Chunkwise 形式", derivation steps 1-6), in the d_k x d_v state
// orientation of "Kimi K3：架构、训练与推理系统研究" §3.1.  With Gamma_r the
// inclusive cumulative decay inside the chunk and gamma_C its last row:
//   M  = (I + StrictTril(Diag(beta)(Gamma*K)(K/Gamma)^T))^{-1} Diag(beta)
//   W  = M (Gamma*K),  U = M V,  V' = U - W S
//   O  = (Gamma*Q) S + Tril((Gamma*Q)(K/Gamma)^T) V'
//   S <- Diag(gamma_C) S + ((gamma_C/Gamma)*K)^T V'
// Gamma and 1/Gamma are never formed over a whole chunk: a 64-token chunk
// can decay by e^-320, which under- and overflows fp32.  Every decay factor
// is instead exp2 of a difference of log-decays measured from the start of
// the same 16-token block, so each factor is either <= 1 or, on a diagonal
// block, <= e^80.  That is the range argument of the devpress K3 walk-through
// (§3.2, Eq 5) and "Kimi K3：架构…" §3.2: sixteen steps of the bounded gate
// sum to at least -80.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------------------
// Slab layout (bytes from the slab start).  A "fragment" is 64 lanes x 16 B
// in the lane order of the MFMA operand it feeds (kda_device.h): a bf16
// fragment spans two K16 tiles (one 16x16x32 MFMA), an fp32 fragment one.
// ---------------------------------------------------------------------------
template <int D, bool F32>
struct Slab {
    static constexpr int KT = D / 16;                 // 16-wide key / value tiles
    static constexpr int NKF = F32 ? D / 16 : D / 32; // fragments over d per 16-row tile
    static constexpr int NCF = F32 ? 4 : 2;           // fragments over the 64 chunk rows
    static constexpr int SPL = F32 ? 1 : 2;           // bf16 operands are stored as hi, lo pairs
    static constexpr size_t FRAG = 1024;
    static constexpr size_t negW = 0;                           // -W      [I][NKF][SPL]
    static constexpr size_t qg = negW + 4 * NKF * SPL * FRAG;   // Gamma*Q [I][NKF][SPL]
    static constexpr size_t kdT = qg + 4 * NKF * SPL * FRAG;    // ((gamma_C/Gamma)*K)^T [t][NCF][SPL]
    static constexpr size_t aqk = kdT + KT * NCF * SPL * FRAG;  // A_qk    [I][NCF][SPL]
    static constexpr size_t u = aqk + 4 * NCF * SPL * FRAG;     // U (fp32 accumulator layout) [I][KT]
    static constexpr size_t gamma = u + 4 * KT * FRAG;          // gamma_C [D] fp32
    static constexpr size_t bytes = ((gamma + D * 4 + 255) / 256) * 256;
};

// Store an accumulator-pair as a split bf16 fragment (hi at `dst`, lo one
// fragment later) or an fp32 quad as an fp32 fragment.
__device__ __forceinline__ void store_split(unsigned char *dst, f32x4 x0, f32x4 x1) {
    u32x4 hi, lo;
    quads_to_bf16_split(x0, x1, hi, lo);
    *reinterpret_cast<u32x4 *>(dst) = hi;
    *reinterpret_cast<u32x4 *>(dst + 1024) = lo;
}

size_t slab_bytes(int dk, int dv, bool f32io) {
    if (dk != dv) return 0;
    switch (dk) {
        case 32: return f32io ? Slab<32, true>::bytes : Slab<32, false>::bytes;
        case 64: return f32io ? Slab<64, true>::bytes : Slab<64, false>::bytes;
        case 128: return f32io ? Slab<128, true>::bytes : Slab<128, false>::bytes;
    }
    return 0;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool plan_prefill(int N, int T, int H, int dk, int dv, bool f32io, PrefillPlan *p) {
    size_t sb = slab_bytes(dk, dv, f32io);
    if (sb == 0 || N < 0 || T < 0 || H <= 0) return false;
    p->max_chunks = (int)(((long long)T + kChunk - 1) / kChunk + N);
    p->slab_bytes = sb;
    p->off_meta = 0;
    p->off_table = align256((size_t)(N + 2) * 4);
    p->off_slabs = p->off_table + align256((size_t)p->max_chunks * 16);
    p->total = p->off_slabs + (size_t)H * p->max_chunks * sb;
    return true;
}

// ---------------------------------------------------------------------------
// Chunk table.  One workgroup.  meta[n] = first chunk of sequence n,
// meta[N] = number of chunks; table[c] = {n, first token, length, 0}.
// Sequence bounds are clamped to [0, T] and the chunk count to max_chunks,
// so a malformed cu_seqlens can give wrong results but no stray access.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) chunk_table_kernel(const int32_t *__restrict__ cu, int N,
                                                          int T, int max_chunks,
                                                          int32_t *__restrict__ meta,
                                                          int4 *__restrict__ table) {
    __shared__ int32_t scan[256];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + tid;
        int cnt = 0;
        if (n < N) {
            int s = min(max(cu[n], 0), T), e = min(max(cu[n + 1], 0), T);
            cnt = e > s ? (e - s + kChunk - 1) / kChunk : 0;
        }
        scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            int x = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += x;
            __syncthreads();
        }
        if (n < N) meta[n] = min(carry + scan[tid] - cnt, max_chunks);
        __syncthreads();
        if (tid == 255) carry += scan[255];
        __syncthreads();
    }
    if (tid == 0) meta[N] = min(carry, max_chunks);
    __syncthreads();
    const int total = min(carry, max_chunks);
    for (int c = tid; c < total; c += 256) {
        int lo = 0, hi = N - 1;  // last n with meta[n] <= c
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (meta[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const int n = lo;
        const int s = min(max(cu[n], 0), T), e = min(max(cu[n + 1], 0), T);
        const int first = s + (c - meta[n]) * kChunk;
        table[c] = make_int4(n, first, min(kChunk, e - first), 0);
    }
}

// ---------------------------------------------------------------------------
// Intra-chunk kernel.
// ---------------------------------------------------------------------------
template <int D>
struct IntraLds {
    static constexpr int P = D + 4;  // row pitch (floats) of the [64][D] arrays
    float kr[64][P];   // k_r * exp2(Gl_r): row operand of A_kk; Gamma*K after a block prefix
    float qr[64][P];   // q_r * exp2(Gl_r): row operand of A_qk; reused for V
    float ke[64][P];   // k_i * exp2(bt_J - Gl_i): decay from i to the end of its block
    float a[64][68];   // A_kk (beta and the strict lower mask applied)
    float tm[64][68];  // T = (I + A_kk)^{-1}
    float beta[64];
    float bt[4][D];    // block log2-decay totals
    float pfx[4][D];   // exp2(sum_{m<I} bt_m)       decay from the chunk start to block I
    float sfx[4][D];   // exp2(sum_{m>J} bt_m)       decay from block J+1 to the chunk end
    float dg[4][D];    // exp2(-bt_J)                undo one block: diagonal column factor
    float off[6][D];   // exp2(sum_{J<m<I} bt_m)     blocks strictly between J and I
};

__device__ __forceinline__ int off_index(int J, int I) {
    // (J, I) with J < I -> 0..5 : (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
    return J == 0 ? I - 1 : (J == 1 ? I + 1 : 5);
}

template <int P>
__device__ __forceinline__ f32x4 lds_quad(const float (*a)[P], int row, int col) {
    return *reinterpret_cast<const f32x4 *>(&a[row][col]);
}
template <int P>
__device__ __forceinline__ f32x4 lds_col4(const float (*a)[P], int row0, int col) {
    return f32x4{a[row0][col], a[row0 + 1][col], a[row0 + 2][col], a[row0 + 3][col]};
}

template <int D, bool F32IO>
__global__ void __launch_bounds__(256) intra_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ z, const float *__restrict__ A, const float *__restrict__ beta,
    const int32_t *__restrict__ meta, const int4 *__restrict__ table, int N, int H,
    int max_chunks, unsigned char *__restrict__ slabs, size_t slab_stride) {
    using SL = Slab<D, F32IO>;
    constexpr int KT = D / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    IntraLds<D> &s = *reinterpret_cast<IntraLds<D> *>(lds_raw);

    const int chunk = blockIdx.x;
    const int h = blockIdx.y;
    if (chunk >= meta[N]) return;
    const int4 ent = table[chunk];
    const int t0 = ent.y, L = ent.z;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int ln = lane & 15, lg = lane >> 4;
    unsigned char *slab = slabs + ((size_t)h * max_chunks + chunk) * slab_stride;

    // ---- phase 1: gate, block-local cumulative log2-decay, scaled operands
    for (int i = tid; i < 64 * 68; i += 256) {
        (&s.a[0][0])[i] = 0.f;
        (&s.tm[0][0])[i] = 0.f;
    }
    if (tid < 64) s.beta[tid] = tid < L ? beta[(size_t)(t0 + tid) * H + h] : 0.f;
    const float ea = __expf(A[h]);
    for (int task = tid; task < 4 * D; task += 256) {
        const int c = task % D, I = task / D;
        float gl[16], kk[16];
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 16 * I + r;
            const bool ok = row < L;
            const size_t idx = ((size_t)(t0 + row) * H + h) * D + c;
            const float zz = ok ? z[idx] : 0.f;
            kk[r] = ok ? load_io<F32IO>(k, idx) : 0.f;
            const float qq = ok ? load_io<F32IO>(q, idx) : 0.f;
            run += ok ? gate_log2(ea, zz) : 0.f;
            gl[r] = run;
            const float rf = exp2f(run);
            s.kr[row][c] = kk[r] * rf;
            s.qr[row][c] = qq * rf;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s.ke[16 * I + r][c] = kk[r] * exp2f(run - gl[r]);
        s.bt[I][c] = run;
    }
    __syncthreads();
    for (int c = tid; c < D; c += 256) {
        const float b0 = s.bt[0][c], b1 = s.bt[1][c], b2 = s.bt[2][c], b3 = s.bt[3][c];
        s.pfx[0][c] = 1.f;
        s.pfx[1][c] = exp2f(b0);
        s.pfx[2][c] = exp2f(b0 + b1);
        s.pfx[3][c] = exp2f(b0 + b1 + b2);
        s.sfx[0][c] = exp2f(b1 + b2 + b3);
        s.sfx[1][c] = exp2f(b2 + b3);
        s.sfx[2][c] = exp2f(b3);
        s.sfx[3][c] = 1.f;
        s.dg[0][c] = exp2f(-b0);
        s.dg[1][c] = exp2f(-b1);
        s.dg[2][c] = exp2f(-b2);
        s.dg[3][c] = exp2f(-b3);
        s.off[0][c] = 1.f;            // (0,1)
        s.off[1][c] = exp2f(b1);      // (0,2)
        s.off[2][c] = exp2f(b1 + b2); // (0,3)
        s.off[3][c] = 1.f;            // (1,2)
        s.off[4][c] = exp2f(b2);      // (1,3)
        s.off[5][c] = 1.f;            // (2,3)
        reinterpret_cast<float *>(slab + SL::gamma)[c] = exp2f(b0 + b1 + b2 + b3);
    }
    __syncthreads();

    // ---- phase 2: decayed Gram tiles A_kk (I, J) and A_qk^T, J <= I
    // A_kk[r][i] = beta_r sum_c k_rc k_ic e^{G_rc - G_ic} is formed as
    // (kr row of block I) x (ke row of block J) * factor, where the factor is
    // exp2(-bt_J) on the diagonal block (the <= e^80 case) and the decay of the
    // blocks strictly between J and I otherwise (<= 1).
    for (int tile = wave; tile < 10; tile += 4) {
        const int I = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
        const int J = tile - (I * (I + 1)) / 2;
        const float *fac = (I == J) ? s.dg[J] : s.off[off_index(J, I)];
        f32x4 akk = zero4(), aqt = zero4();
        if constexpr (F32IO) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int c0 = 16 * kt + 4 * lg;
                const f32x4 kr = lds_quad(s.kr, 16 * I + ln, c0);
                const f32x4 qr = lds_quad(s.qr, 16 * I + ln, c0);
                const f32x4 kc = lds_quad(s.ke, 16 * J + ln, c0) * *reinterpret_cast<const f32x4 *>(fac + c0);
                akk = mma_f32_k16(kr, kc, akk);
                aqt = mma_f32_k16(kc, qr, aqt);
            }
        } else {
#pragma unroll
            for (int p = 0; p < KT / 2; ++p) {
                const int c0 = 32 * p + 4 * lg, c1 = c0 + 16;
                const f32x4 kr0 = lds_quad(s.kr, 16 * I + ln, c0), kr1 = lds_quad(s.kr, 16 * I + ln, c1);
                const f32x4 qr0 = lds_quad(s.qr, 16 * I + ln, c0), qr1 = lds_quad(s.qr, 16 * I + ln, c1);
                const f32x4 kc0 = lds_quad(s.ke, 16 * J + ln, c0) * *reinterpret_cast<const f32x4 *>(fac + c0);
                const f32x4 kc1 = lds_quad(s.ke, 16 * J + ln, c1) * *reinterpret_cast<const f32x4 *>(fac + c1);
                u32x4 krh, krl, kch, kcl, qrh, qrl;
                quads_to_bf16_split(kr0, kr1, krh, krl);
                quads_to_bf16_split(kc0, kc1, kch, kcl);
                quads_to_bf16_split(qr0, qr1, qrh, qrl);
                akk = mma3_bf16(krh, krl, kch, kcl, akk);
                aqt = mma3_bf16(kch, kcl, qrh, qrl, aqt);
            }
        }
        // A_kk: lane (n = i, g) holds rows r = 4g + j of the tile
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rl = 4 * lg + j;
            float x = akk[j] * s.beta[16 * I + rl];
            if (I == J && ln >= rl) x = 0.f;
            s.a[16 * I + rl][16 * J + ln] = x;
        }
        // A_qk^T: lane (n = r, g) holds i = 4g + j, i.e. the A_qk operand
        // fragment of row tile I; keep i <= r on the diagonal tile.
        f32x4 aq;
#pragma unroll
        for (int j = 0; j < 4; ++j) aq[j] = (I == J && 4 * lg + j > ln) ? 0.f : aqt[j];
        if constexpr (F32IO) {
            *reinterpret_cast<f32x4 *>(slab + SL::aqk + ((size_t)(I * 4 + J) * 64 + lane) * 16) = aq;
        } else {
            uint32_t hb[4], lb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split_bf16(aq[j], hb[j], lb[j]);
            const int qf = J >> 1, half = J & 1;
            u32x2 hv = {pack2(hb[0], hb[1]), pack2(hb[2], hb[3])};
            u32x2 lv = {pack2(lb[0], lb[1]), pack2(lb[2], lb[3])};
            unsigned char *base = slab + SL::aqk + ((size_t)((I * 2 + qf) * 2) * 64 + lane) * 16 + half * 8;
            *reinterpret_cast<u32x2 *>(base) = hv;
            *reinterpret_cast<u32x2 *>(base + 64 * 16) = lv;
            if (I == J && (I & 1) == 0) {  // the tile right of an even diagonal shares its fragment
                *reinterpret_cast<u32x2 *>(base + 8) = u32x2{0u, 0u};
                *reinterpret_cast<u32x2 *>(base + 64 * 16 + 8) = u32x2{0u, 0u};
            }
        }
    }

    // Gamma*Q fragments (row tile I, key fragment f) and the transposed,
    // end-of-chunk-decayed keys ((gamma_C/Gamma)*K)^T (key tile t, row fragment f).
    for (int fr = wave; fr < 4 * SL::NKF; fr += 4) {
        const int I = fr / SL::NKF, f = fr % SL::NKF;
        unsigned char *dst = slab + SL::qg + ((size_t)fr * SL::SPL * 64 + lane) * 16;
        if constexpr (F32IO) {
            const int c0 = 16 * f + 4 * lg;
            *reinterpret_cast<f32x4 *>(dst) =
                lds_quad(s.qr, 16 * I + ln, c0) * *reinterpret_cast<const f32x4 *>(&s.pfx[I][c0]);
        } else {
            const int c0 = 32 * f + 4 * lg, c1 = c0 + 16;
            store_split(dst,
                        lds_quad(s.qr, 16 * I + ln, c0) * *reinterpret_cast<const f32x4 *>(&s.pfx[I][c0]),
                        lds_quad(s.qr, 16 * I + ln, c1) * *reinterpret_cast<const f32x4 *>(&s.pfx[I][c1]));
        }
    }
    for (int fr = wave; fr < KT * SL::NCF; fr += 4) {
        const int t = fr / SL::NCF, f = fr % SL::NCF;
        const int c = 16 * t + ln;
        unsigned char *dst = slab + SL::kdT + ((size_t)fr * SL::SPL * 64 + lane) * 16;
        if constexpr (F32IO) {
            const int J = f;
            *reinterpret_cast<f32x4 *>(dst) = lds_col4(s.ke, 16 * J + 4 * lg, c) * s.sfx[J][c];
        } else {
            const int J0 = 2 * f, J1 = 2 * f + 1;
            store_split(dst, lds_col4(s.ke, 16 * J0 + 4 * lg, c) * s.sfx[J0][c],
                        lds_col4(s.ke, 16 * J1 + 4 * lg, c) * s.sfx[J1][c]);
        }
    }
    __syncthreads();

    // ---- phase 3: V into LDS (over q's rows) and the diagonal 16x16 inverses
    for (int i = tid; i < 64 * D; i += 256) {
        const int row = i / D, c = i % D;
        s.qr[row][c] = row < L ? load_io<F32IO>(v, ((size_t)(t0 + row) * H + h) * D + c) : 0.f;
    }
    if (lane < 16) {
        // forward substitution for column `lane` of (I + A_ww)^{-1}
        const int b = 16 * wave;
        float col[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = (r == lane) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) x -= s.a[b + r][b + i] * col[i];
            col[r] = x;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s.tm[b + r][b + lane] = col[r];
    }
    __syncthreads();

    // ---- phase 4: off-diagonal blocks, T_IJ = -T_II sum_{J<=m<I} A_Im T_mJ (fp32 MFMA)
    for (int I = 1; I < 4; ++I) {
        if (wave < I) {
            const int J = wave;
            f32x4 x = zero4();
            for (int m = J; m < I; ++m)
                x = mma_f32_k16(lds_quad(s.a, 16 * I + ln, 16 * m + 4 * lg),
                                lds_col4(s.tm, 16 * m + 4 * lg, 16 * J + ln), x);
            f32x4 y = mma_f32_k16(lds_quad(s.tm, 16 * I + ln, 16 * I + 4 * lg), x, zero4());
#pragma unroll
            for (int j = 0; j < 4; ++j) s.tm[16 * I + 4 * lg + j][16 * J + ln] = -y[j];
        }
        __syncthreads();
    }

    // ---- phase 5: -W fragments (from W^T tiles) and U tiles.  M = T Diag(beta).
    // W^T tile (t, I) = sum_J (Gamma*K)^T_{tJ} M^T_{JI}: the accumulator lane
    // (n = r, g) holds W[16I + r][16t + 4g + j], which is the A-operand
    // fragment of -W in the state-propagation product.
    for (int I = 0; I < 4; ++I) {
        const int nJ = I + 1;
        // M row quads of row tile I (B operand of W^T, A operand of U)
        for (int tp = wave; tp < SL::NKF; tp += 4) {
            if constexpr (F32IO) {
                const int t = tp;
                f32x4 acc = zero4();
                for (int J = 0; J < nJ; ++J) {
                    const int cJ = 16 * J + 4 * lg;
                    const f32x4 mq = lds_quad(s.tm, 16 * I + ln, cJ) * *reinterpret_cast<const f32x4 *>(&s.beta[cJ]);
                    const f32x4 gk = lds_col4(s.kr, 16 * J + 4 * lg, 16 * t + ln) * s.pfx[J][16 * t + ln];
                    acc = mma_f32_k16(gk, mq, acc);
                }
                *reinterpret_cast<f32x4 *>(slab + SL::negW + ((size_t)(I * SL::NKF + tp) * 64 + lane) * 16) = -acc;
            } else {
                const int t0_ = 2 * tp, t1_ = 2 * tp + 1;
                f32x4 acc0 = zero4(), acc1 = zero4();
                for (int pj = 0; pj < (nJ + 1) / 2; ++pj) {
                    const int J0 = 2 * pj, J1 = 2 * pj + 1;
                    const int cJ0 = 16 * J0 + 4 * lg, cJ1 = 16 * J1 + 4 * lg;
                    const f32x4 m0 = lds_quad(s.tm, 16 * I + ln, cJ0) * *reinterpret_cast<const f32x4 *>(&s.beta[cJ0]);
                    const f32x4 m1 = lds_quad(s.tm, 16 * I + ln, cJ1) * *reinterpret_cast<const f32x4 *>(&s.beta[cJ1]);
                    u32x4 mh, ml, gah, gal, gbh, gbl;
                    quads_to_bf16_split(m0, m1, mh, ml);
                    const int ca = 16 * t0_ + ln, cb = 16 * t1_ + ln;
                    quads_to_bf16_split(lds_col4(s.kr, 16 * J0 + 4 * lg, ca) * s.pfx[J0][ca],
                                        lds_col4(s.kr, 16 * J1 + 4 * lg, ca) * s.pfx[J1][ca], gah, gal);
                    quads_to_bf16_split(lds_col4(s.kr, 16 * J0 + 4 * lg, cb) * s.pfx[J0][cb],
                                        lds_col4(s.kr, 16 * J1 + 4 * lg, cb) * s.pfx[J1][cb], gbh, gbl);
                    acc0 = mma3_bf16(gah, gal, mh, ml, acc0);
                    acc1 = mma3_bf16(gbh, gbl, mh, ml, acc1);
                }
                store_split(slab + SL::negW + ((size_t)(I * SL::NKF + tp) * 2 * 64 + lane) * 16, -acc0, -acc1);
            }
        }
        // U tile (I, w) = sum_J M_{IJ} V_{Jw}; accumulator layout is what the
        // state-propagation kernel starts V' from.
        for (int w = wave; w < KT; w += 4) {
            f32x4 acc = zero4();
            if constexpr (F32IO) {
                for (int J = 0; J < nJ; ++J) {
                    const int cJ = 16 * J + 4 * lg;
                    const f32x4 mq = lds_quad(s.tm, 16 * I + ln, cJ) * *reinterpret_cast<const f32x4 *>(&s.beta[cJ]);
                    acc = mma_f32_k16(mq, lds_col4(s.qr, 16 * J + 4 * lg, 16 * w + ln), acc);
                }
            } else {
                for (int pj = 0; pj < (nJ + 1) / 2; ++pj) {
                    const int J0 = 2 * pj, J1 = 2 * pj + 1;
                    const int cJ0 = 16 * J0 + 4 * lg, cJ1 = 16 * J1 + 4 * lg;
                    const f32x4 m0 = lds_quad(s.tm, 16 * I + ln, cJ0) * *reinterpret_cast<const f32x4 *>(&s.beta[cJ0]);
                    const f32x4 m1 = lds_quad(s.tm, 16 * I + ln, cJ1) * *reinterpret_cast<const f32x4 *>(&s.beta[cJ1]);
                    u32x4 mh, ml;
                    quads_to_bf16_split(m0, m1, mh, ml);
                    const u32x4 vb = quads_to_bf16(lds_col4(s.qr, 16 * J0 + 4 * lg, 16 * w + ln),
                                                   lds_col4(s.qr, 16 * J1 + 4 * lg, 16 * w + ln));
                    acc = mma_bf16_k32(mh, vb, acc);
                    acc = mma_bf16_k32(ml, vb, acc);
                }
            }
            *reinterpret_cast<f32x4 *>(slab + SL::u + ((size_t)(I * KT + w) * 64 + lane) * 16) = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// Inter-chunk kernel.  Wave w of a workgroup owns value columns
// [16 vt, 16 vt + 16) of one (sequence, head); its state slice S[:, cols]
// lives in DK/16 accumulator tiles (lane (n, g) holds S[16t + 4g + j][16vt + n]).
// Per chunk, in the order of the chunk form:
//   V' = U - W S                 (U is the initial accumulator, -W the A operand)
//   O  = (Gamma*Q) S + A_qk V'
//   S  = Diag(gamma_C) S + ((gamma_C/Gamma)*K)^T V'
// Every bf16 operand (stored fragments and the S, V' accumulators) enters
// the MFMAs split into hi + lo parts; each product is hi*hi + hi*lo + lo*hi.
// ---------------------------------------------------------------------------
template <int D, bool F32IO>
__global__ void __launch_bounds__(256) inter_kernel(
    const float *__restrict__ h0, const int32_t *__restrict__ meta, const int4 *__restrict__ table,
    int N, int H, int max_chunks, const unsigned char *__restrict__ slabs, size_t slab_stride,
    void *__restrict__ o, float *__restrict__ hT, int groups) {
    using SL = Slab<D, F32IO>;
    constexpr int KT = D / 16;
    constexpr int WPG = KT < 4 ? KT : 4;  // waves per workgroup
    // blockIdx -> (pair, column group) with every group of a pair on the same XCD
    const int b = blockIdx.x;
    const int xcd = b & 7, rest = b >> 3;
    const int cg = rest % groups;
    const int pair = (rest / groups) * 8 + xcd;
    if (pair >= N * H) return;
    const int n = pair / H, h = pair % H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ln = lane & 15, lg = lane >> 4;
    const int vt = cg * WPG + wave;
    const int col = 16 * vt + ln;

    f32x4 S[KT];
    const size_t srow = ((size_t)pair * D + col) * D;
#pragma unroll
    for (int t = 0; t < KT; ++t)
        S[t] = h0 ? *reinterpret_cast<const f32x4 *>(h0 + srow + 16 * t + 4 * lg) : zero4();

    const int c_begin = meta[n], c_end = meta[n + 1];
    for (int c = c_begin; c < c_end; ++c) {
        const int4 ent = table[c];
        const int t0 = ent.y, L = ent.z;
        const unsigned char *slab = slabs + ((size_t)h * max_chunks + c) * slab_stride;
        auto frag = [&](size_t off, int idx) -> const void * {
            return slab + off + ((size_t)idx * 64 + lane) * 16;
        };
        f32x4 vp[4], acc_o[4];
        if constexpr (F32IO) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                vp[I] = *reinterpret_cast<const f32x4 *>(frag(SL::u, I * KT + vt));
                acc_o[I] = zero4();
#pragma unroll
                for (int t = 0; t < KT; ++t) {
                    vp[I] = mma_f32_k16(*reinterpret_cast<const f32x4 *>(frag(SL::negW, I * KT + t)), S[t], vp[I]);
                    acc_o[I] = mma_f32_k16(*reinterpret_cast<const f32x4 *>(frag(SL::qg, I * KT + t)), S[t], acc_o[I]);
                }
            }
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int J = 0; J <= I; ++J)
                    acc_o[I] = mma_f32_k16(*reinterpret_cast<const f32x4 *>(frag(SL::aqk, I * 4 + J)), vp[J], acc_o[I]);
            const f32x4 *gam = reinterpret_cast<const f32x4 *>(slab + SL::gamma);
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                S[t] = S[t] * gam[4 * t + lg];
#pragma unroll
                for (int J = 0; J < 4; ++J)
                    S[t] = mma_f32_k16(*reinterpret_cast<const f32x4 *>(frag(SL::kdT, t * 4 + J)), vp[J], S[t]);
            }
        } else {
            u32x4 sh[KT / 2], sl[KT / 2];
#pragma unroll
            for (int p = 0; p < KT / 2; ++p) quads_to_bf16_split(S[2 * p], S[2 * p + 1], sh[p], sl[p]);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                vp[I] = *reinterpret_cast<const f32x4 *>(frag(SL::u, I * KT + vt));
                acc_o[I] = zero4();
#pragma unroll
                for (int p = 0; p < KT / 2; ++p) {
                    const int fi = (I * (KT / 2) + p) * 2;
                    const u32x4 wh = *reinterpret_cast<const u32x4 *>(frag(SL::negW, fi));
                    const u32x4 wl = *reinterpret_cast<const u32x4 *>(frag(SL::negW, fi + 1));
                    const u32x4 gh = *reinterpret_cast<const u32x4 *>(frag(SL::qg, fi));
                    const u32x4 gl = *reinterpret_cast<const u32x4 *>(frag(SL::qg, fi + 1));
                    vp[I] = mma3_bf16(wh, wl, sh[p], sl[p], vp[I]);
                    acc_o[I] = mma3_bf16(gh, gl, sh[p], sl[p], acc_o[I]);
                }
            }
            u32x4 vh[2], vl[2];
            quads_to_bf16_split(vp[0], vp[1], vh[0], vl[0]);
            quads_to_bf16_split(vp[2], vp[3], vh[1], vl[1]);
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int qf = 0; qf <= I / 2; ++qf) {
                    const u32x4 ah = *reinterpret_cast<const u32x4 *>(frag(SL::aqk, (I * 2 + qf) * 2));
                    const u32x4 al = *reinterpret_cast<const u32x4 *>(frag(SL::aqk, (I * 2 + qf) * 2 + 1));
                    acc_o[I] = mma3_bf16(ah, al, vh[qf], vl[qf], acc_o[I]);
                }
            const f32x4 *gam = reinterpret_cast<const f32x4 *>(slab + SL::gamma);
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                S[t] = S[t] * gam[4 * t + lg];
#pragma unroll
                for (int qf = 0; qf < 2; ++qf) {
                    const u32x4 ah = *reinterpret_cast<const u32x4 *>(frag(SL::kdT, (t * 2 + qf) * 2));
                    const u32x4 al = *reinterpret_cast<const u32x4 *>(frag(SL::kdT, (t * 2 + qf) * 2 + 1));
                    S[t] = mma3_bf16(ah, al, vh[qf], vl[qf], S[t]);
                }
            }
        }
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * I + 4 * lg + j;
                if (r < L) store_io<F32IO>(o, ((size_t)(t0 + r) * H + h) * D + col, acc_o[I][j]);
            }
    }
    if (hT) {
#pragma unroll
        for (int t = 0; t < KT; ++t) *reinterpret_cast<f32x4 *>(hT + srow + 16 * t + 4 * lg) = S[t];
    }
}

// ---------------------------------------------------------------------------
template <int D, bool F32IO>
static int launch_prefill_t(const PrefillArgs &a) {
    const PrefillPlan &p = a.plan;
    int32_t *meta = reinterpret_cast<int32_t *>(a.ws + p.off_meta);
    int4 *table = reinterpret_cast<int4 *>(a.ws + p.off_table);
    unsigned char *slabs = a.ws + p.off_slabs;

    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, a.stream, a.cu, a.N, a.T,
                       p.max_chunks, meta, table);
    if (hipGetLastError() != hipSuccess) return -1;

    if (p.max_chunks > 0) {
        const size_t lds = sizeof(IntraLds<D>);
        static bool attr_set = false;
        if (!attr_set) {
            if (hipFuncSetAttribute(reinterpret_cast<const void *>(&intra_kernel<D, F32IO>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
                return -1;
            attr_set = true;
        }
        hipLaunchKernelGGL((intra_kernel<D, F32IO>), dim3(p.max_chunks, a.H), dim3(256), lds, a.stream,
                           a.q, a.k, a.v, a.z, a.A, a.beta, meta, table, a.N, a.H, p.max_chunks, slabs,
                           p.slab_bytes);
        if (hipGetLastError() != hipSuccess) return -1;
    }

    constexpr int KT = D / 16;
    constexpr int WPG = KT < 4 ? KT : 4;
    const int groups = KT / WPG;
    const int pairs = a.N * a.H;
    if (pairs > 0) {
        const int pair_blocks = (pairs + 7) / 8 * 8;
        hipLaunchKernelGGL((inter_kernel<D, F32IO>), dim3(pair_blocks * groups), dim3(64 * WPG), 0,
                           a.stream, a.h0, meta, table, a.N, a.H, p.max_chunks, slabs, p.slab_bytes,
                           a.o, a.hT, groups);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

int launch_prefill(const PrefillArgs &a) {
    switch (a.dk) {
        case 32: return a.f32io ? launch_prefill_t<32, true>(a) : launch_prefill_t<32, false>(a);
        case 64: return a.f32io ? launch_prefill_t<64, true>(a) : launch_prefill_t<64, false>(a);
        case 128: return a.f32io ? launch_prefill_t<128, true>(a) : launch_prefill_t<128, false>(a);
    }
    return -1;
}

}  // namespace kda
