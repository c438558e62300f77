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
#include "kda_chunk.h"
#include "kda_device.h"
#include "kda_internal.h"

#include <algorithm>
#include <type_traits>

namespace kda {

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
    p->off_null = p->off_table + align256((size_t)p->max_chunks * 16);
    p->off_slabs = p->off_null + align256((size_t)dk * 4 + (size_t)dk * 4 + 4);
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
                                                          int4 *__restrict__ table,
                                                          float *__restrict__ null_row, int d) {
    __shared__ int32_t scan[256];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    // The null row that rows past a chunk's end read instead of real inputs:
    // z = -inf gives a zero gate (no decay), and k = q = v = 0, beta = 0.
    for (int c = tid; c < 2 * d + 1; c += 256)
        null_row[c] = c < d ? -__builtin_inff() : 0.f;
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
// Intra-chunk kernel.  Persistent: each workgroup walks (chunk, head) items
// with a stride of the grid size and prefetches the next item's raw inputs
// into registers while it computes the current one.
//
// In phase 1 wave w owns the 16-row block I = w; lane (ln, lg) = (l % 16,
// l / 16) holds row 16w + ln and key channels 16kt + 4lg + {0..3}.  That is
// the MFMA A-operand layout, and a scan over the 16 lanes of a row group
// gives the block-local cumulative log-decay of every channel.
// ---------------------------------------------------------------------------
template <int D>
struct IntraLds {
    static constexpr int P = D + 4;          // fp32 row pitch (floats)
    static constexpr int RB = 4 * P;         // row pitch (bytes) of the row-operand arrays
    static constexpr int TP = 64 + 4;        // row pitch (elements) of the transposed bf16 arrays
    // Row operands k_r exp2(Gl_r) and q_r exp2(Gl_r).  bf16 path: per row,
    // [pair p][hi, lo][lane group][8 bf16], so one 16-byte read is one MFMA
    // fragment slot; fp32 path: [64][P] floats.  After the Gram phase the
    // bf16 path reuses both arrays for (Gamma*K)^T split into hi and lo, and
    // ke's array for M = T Diag(beta) split in the same fragment-row layout.
    unsigned char krs[64 * RB];
    unsigned char qrs[64 * RB];
    float ke[64][P];      // k_i exp2(bt_J - Gl_i); fp32 path: V after the Gram phase
    float a[64][68];      // A_kk, then T = (I + A_kk)^{-1} in place
    uint16_t vt[D][TP];   // bf16 path: V^T (bf16 bits)
    float beta[64];
    float bt[4][D];       // block log2-decay totals
    float pfx[4][D];      // exp2(sum_{m<I} bt_m)       chunk start -> start of block I
    float sfx[4][D];      // exp2(sum_{m>J} bt_m)       end of block J -> chunk end
    float dg[4][D];       // exp2(-bt_J)                undo one block: diagonal column factor
    float off[6][D];      // exp2(sum_{J<m<I} bt_m)     blocks strictly between J and I
};

constexpr int kIntraWaves = 8;
// Row pitch (bytes) of the split M array: 2 pairs x (hi, lo) x 64 B plus 16 B
// so that the 16 rows a wave reads at once fall on different LDS banks.
constexpr int kMsRow = 2 * 128 + 16;

// Raw inputs of one (chunk, head) item for one lane of an 8-wave group:
// wave w loads row block (w & 3), key-channel half (w >> 2).  Lanes whose
// row lies past the chunk's end load the chunk's first row instead; the
// consumer masks them.  Every load is unconditional and issued in the order
// of use, so a wait for one prefetched register never has to cover the
// stores issued after the prefetch.
template <int D, bool F32IO>
struct IntraRegs {
    static constexpr int KH = D / 32;  // K16 tiles per channel half
    using Q = typename std::conditional<F32IO, f32x4, u32x2>::type;
    float beta;
    f32x4 z[KH];
    Q k[KH], q[KH], v[KH];
};

template <int D, bool F32IO>
__device__ __forceinline__ void intra_load(IntraRegs<D, F32IO> &R, const void *q, const void *k,
                                           const void *v, const float *z, const float *beta,
                                           int4 ent, int h, int H, int lane, int wave) {
    constexpr int KH = D / 32;
    constexpr int ES = F32IO ? 4 : 2;
    using Q = typename IntraRegs<D, F32IO>::Q;
    const int ln = lane & 15, lg = lane >> 4;
    const int row = 16 * (wave & 3) + ln;
    const size_t trow = (size_t)(ent.y + (row < ent.z ? row : 0)) * H + h;
    const size_t base = trow * D + (D / 2) * (wave >> 2) + 4 * lg;
    const unsigned char *kb = reinterpret_cast<const unsigned char *>(k);
    const unsigned char *qb = reinterpret_cast<const unsigned char *>(q);
    const unsigned char *vb = reinterpret_cast<const unsigned char *>(v);
    R.beta = beta[trow];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
        const size_t idx = base + 16 * kk;
        R.z[kk] = ld4(z + idx);
        R.k[kk] = *reinterpret_cast<const Q *>(kb + idx * ES);
        R.q[kk] = *reinterpret_cast<const Q *>(qb + idx * ES);
        R.v[kk] = *reinterpret_cast<const Q *>(vb + idx * ES);
    }
}

// Split bf16 row operand in the fragment-row layout: row r, K16 tile kt,
// lane group g -> 8 bytes of hi at [kt/2][0][g][kt%2], 8 bytes of lo at [kt/2][1][g][kt%2].
template <int RB>
__device__ __forceinline__ void store_row_split(unsigned char *arr, int row, int kt, int g, f32x4 x) {
    const u32x2 hv = {f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3])};
    const f32x4 hq = f32x4{bf16_lo_half(hv[0]), bf16_hi_half(hv[0]), bf16_lo_half(hv[1]), bf16_hi_half(hv[1])};
    const f32x4 r4 = x - hq;
    const u32x2 lv = {f32x2_to_bf16x2(r4[0], r4[1]), f32x2_to_bf16x2(r4[2], r4[3])};
    unsigned char *b = arr + row * RB + (kt >> 1) * 128 + g * 16 + (kt & 1) * 8;
    *reinterpret_cast<u32x2 *>(b) = hv;
    *reinterpret_cast<u32x2 *>(b + 64) = lv;
}

template <int D, bool F32IO>
__global__ void __launch_bounds__(64 * kIntraWaves) intra_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ z, const float *__restrict__ A, const float *__restrict__ beta,
    const int32_t *__restrict__ meta, const int4 *__restrict__ table, int N, int H,
    int max_chunks, unsigned char *__restrict__ slabs, size_t slab_stride) {
    using SL = Slab<D, F32IO>;
    using LDS = IntraLds<D>;
    constexpr int KT = D / 16, KH = D / 32;
    constexpr int NW = kIntraWaves, NTH = 64 * NW;
    constexpr int P = LDS::P, RB = LDS::RB, TP = LDS::TP;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    LDS &s = *reinterpret_cast<LDS *>(lds_raw);
    float (*krf)[P] = reinterpret_cast<float (*)[P]>(s.krs);   // fp32 path views
    float (*qrf)[P] = reinterpret_cast<float (*)[P]>(s.qrs);
    uint16_t (*gkh)[TP] = reinterpret_cast<uint16_t (*)[TP]>(s.krs);               // bf16 path:
    uint16_t (*gkl)[TP] = reinterpret_cast<uint16_t (*)[TP]>(s.krs + D * TP * 2);  // (Gamma*K)^T
    unsigned char *msp = reinterpret_cast<unsigned char *>(&s.ke[0][0]);          // bf16 path: M split

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index in an SGPR
    const int ln = lane & 15, lg = lane >> 4;
    const int blk = wave & 3, half = wave >> 2;   // phase-1 ownership: row block, channel half
    const int total = meta[N] * H;
    const int stride = gridDim.x;

    int it = blockIdx.x;
    if (it >= total) return;
    IntraRegs<D, F32IO> R;
    int4 ent = table[it / H];
    intra_load<D, F32IO>(R, q, k, v, z, beta, ent, it % H, H, lane, wave);
    // Nothing else is in flight here: settle these loads so that the waits at
    // the loop head are set by the loop body alone, where the previous item's
    // stores stay in flight behind the prefetched loads.
    __builtin_amdgcn_s_waitcnt(0);
    // Chunk-table entries and A_h are read through the scalar cache, whose
    // loads every barrier waits for: fetch them one item ahead of their use.
    int4 ent_next = (it + stride < total) ? table[(it + stride) / H] : make_int4(0, 0, 0, 0);
    float a_cur = A[it % H];

    for (; it < total; it += stride) {
        const int chunk = it / H, h = it % H;
        const int L = ent.z;
        unsigned char *slab = slabs + ((size_t)h * max_chunks + chunk) * slab_stride;
        const float ea = __expf(a_cur);
        const int it_next = it + stride;
        const int4 ent_after = (it_next + stride < total) ? table[(it_next + stride) / H] : make_int4(0, 0, 0, 0);
        const float a_next = it_next < total ? A[it_next % H] : 0.f;
        const int row = 16 * blk + ln;
        const bool ok = row < L;

        // ---- phase 1: gate, block-local cumulative log2-decay, row operands
        for (int i = tid; i < 64 * 68; i += NTH) (&s.a[0][0])[i] = 0.f;
        if (lg == 0 && wave < 4) s.beta[row] = ok ? R.beta : 0.f;
        f32x4 krv[KH], qrv[KH], vreg[KH];
#pragma unroll
        for (int kk = 0; kk < KH; ++kk) {
            const int kt = half * KH + kk;
            const int c0 = 16 * kt + 4 * lg;
            const f32x4 kq = ok ? quad_f32<F32IO>(R.k[kk]) : zero4();
            const f32x4 qq = ok ? quad_f32<F32IO>(R.q[kk]) : zero4();
            vreg[kk] = ok ? quad_f32<F32IO>(R.v[kk]) : zero4();
            f32x4 gl, bt, rf, kev;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gl[j] = row16_inclusive_scan(ok ? gate_log2(ea, R.z[kk][j]) : 0.f);
                bt[j] = row16_last(gl[j]);
                rf[j] = fast_exp2(gl[j]);
                kev[j] = kq[j] * fast_exp2(bt[j] - gl[j]);
            }
            krv[kk] = kq * rf;
            qrv[kk] = qq * rf;
            *reinterpret_cast<f32x4 *>(&s.ke[row][c0]) = kev;
            if (ln == 15) *reinterpret_cast<f32x4 *>(&s.bt[blk][c0]) = bt;
            if constexpr (F32IO) {
                *reinterpret_cast<f32x4 *>(&krf[row][c0]) = krv[kk];
                *reinterpret_cast<f32x4 *>(&qrf[row][c0]) = qrv[kk];
            } else {
                store_row_split<RB>(s.krs, row, kt, lg, krv[kk]);
                store_row_split<RB>(s.qrs, row, kt, lg, qrv[kk]);
                const u32x2 vv = ok ? R.v[kk] : u32x2{0u, 0u};
                s.vt[c0 + 0][row] = (uint16_t)(vv[0] & 0xffffu);
                s.vt[c0 + 1][row] = (uint16_t)(vv[0] >> 16);
                s.vt[c0 + 2][row] = (uint16_t)(vv[1] & 0xffffu);
                s.vt[c0 + 3][row] = (uint16_t)(vv[1] >> 16);
            }
        }
        // The raw inputs are consumed: fetch the next item (bf16 path; the
        // fp32 path keeps V in registers until phase 3 and fetches there).
        if constexpr (!F32IO) {
            if (it_next < total) intra_load<D, F32IO>(R, q, k, v, z, beta, ent_next, it_next % H, H, lane, wave);
        }
        __syncthreads();

        for (int c = tid; c < D; c += NTH) {
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
            s.off[0][c] = 1.f;             // (0,1)
            s.off[1][c] = exp2f(b1);       // (0,2)
            s.off[2][c] = exp2f(b1 + b2);  // (0,3)
            s.off[3][c] = 1.f;             // (1,2)
            s.off[4][c] = exp2f(b2);       // (1,3)
            s.off[5][c] = 1.f;             // (2,3)
            reinterpret_cast<float *>(slab + SL::gamma)[c] = exp2f(b0 + b1 + b2 + b3);
        }
        __syncthreads();

        // ---- phase 2: decayed Gram tiles A_kk (I, J) and A_qk^T, J <= I.
        // A_kk[r][i] = beta_r sum_c k_rc k_ic e^{G_rc - G_ic} is (row operand of
        // block I) x (ke of block J) x factor: exp2(-bt_J) on the diagonal block
        // (the <= e^80 case), the decay of the blocks strictly between J and I
        // otherwise (<= 1).
        for_wave_units<10, NW>(wave, [&](int tile) {
            const int I = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J = tile - (I * (I + 1)) / 2;
            const float *fac = (I == J) ? s.dg[J] : s.off[off_index(J, I)];
            f32x4 akk = zero4(), aqt = zero4();
            if constexpr (F32IO) {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    const int c0 = 16 * kt + 4 * lg;
                    const f32x4 kc = lds_quad(s.ke, 16 * J + ln, c0) * ld4(fac + c0);
                    akk = mma_f32_k16(lds_quad(krf, 16 * I + ln, c0), kc, akk);
                    aqt = mma_f32_k16(kc, lds_quad(qrf, 16 * I + ln, c0), aqt);
                }
            } else {
                const unsigned char *kr_row = s.krs + (16 * I + ln) * RB + lg * 16;
                const unsigned char *qr_row = s.qrs + (16 * I + ln) * RB + lg * 16;
#pragma unroll
                for (int p = 0; p < KT / 2; ++p) {
                    const int c0 = 32 * p + 4 * lg, c1 = c0 + 16;
                    const u32x4 krh = *reinterpret_cast<const u32x4 *>(kr_row + p * 128);
                    const u32x4 krl = *reinterpret_cast<const u32x4 *>(kr_row + p * 128 + 64);
                    const u32x4 qrh = *reinterpret_cast<const u32x4 *>(qr_row + p * 128);
                    const u32x4 qrl = *reinterpret_cast<const u32x4 *>(qr_row + p * 128 + 64);
                    u32x4 kch, kcl;
                    quads_to_bf16_split(lds_quad(s.ke, 16 * J + ln, c0) * ld4(fac + c0),
                                        lds_quad(s.ke, 16 * J + ln, c1) * ld4(fac + c1), kch, kcl);
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
                const int qf = J >> 1, hh = J & 1;
                unsigned char *base = slab + SL::aqk + ((size_t)aqk_frag(I, qf) * 64 + lane) * 16 + hh * 8;
                *reinterpret_cast<u32x2 *>(base) = quad_to_f16(aq);
                if (I == J && (I & 1) == 0)  // the tile right of an even diagonal shares its fragment
                    *reinterpret_cast<u32x2 *>(base + 8) = u32x2{0u, 0u};
            }
        });

        // Gamma*Q fragments (row tile I, key fragment f) and the transposed,
        // end-of-chunk-decayed keys ((gamma_C/Gamma)*K)^T (key tile t, row fragment f).
        for_wave_units<4 * SL::NKF, NW>(wave, [&](int fr) {
            const int I = fr / SL::NKF, f = fr % SL::NKF;
            unsigned char *dst = slab + SL::qg + ((size_t)fr * SL::SPL * 64 + lane) * 16;
            if constexpr (F32IO) {
                const int c0 = 16 * f + 4 * lg;
                *reinterpret_cast<f32x4 *>(dst) = lds_quad(qrf, 16 * I + ln, c0) * ld4(&s.pfx[I][c0]);
            } else {
                const unsigned char *qr_row = s.qrs + (16 * I + ln) * RB + lg * 16;
                f32x4 h0, h1, l0, l1;
                bf16_to_quads(*reinterpret_cast<const u32x4 *>(qr_row + f * 128), h0, h1);
                bf16_to_quads(*reinterpret_cast<const u32x4 *>(qr_row + f * 128 + 64), l0, l1);
                const int c0 = 32 * f + 4 * lg, c1 = c0 + 16;
                store_f16(dst, (h0 + l0) * ld4(&s.pfx[I][c0]), (h1 + l1) * ld4(&s.pfx[I][c1]));
            }
        });
        for_wave_units<KT * SL::NCF, NW>(wave, [&](int fr) {
            const int t = fr / SL::NCF, f = fr % SL::NCF;
            const int c = 16 * t + ln;
            unsigned char *dst = slab + SL::kdT + ((size_t)fr * SL::SPL * 64 + lane) * 16;
            if constexpr (F32IO) {
                const int J = f;
                *reinterpret_cast<f32x4 *>(dst) = lds_col4(s.ke, 16 * J + 4 * lg, c) * s.sfx[J][c];
            } else {
                const int J0 = 2 * f, J1 = 2 * f + 1;
                store_f16(dst, lds_col4(s.ke, 16 * J0 + 4 * lg, c) * s.sfx[J0][c],
                          lds_col4(s.ke, 16 * J1 + 4 * lg, c) * s.sfx[J1][c]);
            }
        });
        __syncthreads();

        // ---- phase 3: (Gamma*K)^T (bf16) or V (fp32 path) into the freed
        // arrays, and the diagonal 16x16 inverses, in place.
        if constexpr (F32IO) {
#pragma unroll
            for (int kk = 0; kk < KH; ++kk)
                *reinterpret_cast<f32x4 *>(&s.ke[row][16 * (half * KH + kk) + 4 * lg]) = vreg[kk];
            if (it_next < total) intra_load<D, F32IO>(R, q, k, v, z, beta, ent_next, it_next % H, H, lane, wave);
        } else {
#pragma unroll
            for (int kk = 0; kk < KH; ++kk) {
                const int c0 = 16 * (half * KH + kk) + 4 * lg;
                const f32x4 gk = krv[kk] * ld4(&s.pfx[blk][c0]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t hb, lb;
                    split_bf16(gk[j], hb, lb);
                    gkh[c0 + j][row] = (uint16_t)hb;
                    gkl[c0 + j][row] = (uint16_t)lb;
                }
            }
        }
        if (wave < 4 && lane < 16) {
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
            for (int r = 0; r < 16; ++r) s.a[b + r][b + lane] = col[r];
        }
        __syncthreads();

        // ---- phase 4: off-diagonal blocks, T_IJ = -T_II sum_{J<=m<I} A_Im T_mJ
        // (fp32 MFMA), written over A_IJ once every wave has read row block I.
        for (int I = 1; I < 4; ++I) {
            f32x4 y = zero4();
            if (wave < I) {
                const int J = wave;
                f32x4 x = zero4();
                for (int m = J; m < I; ++m)
                    x = mma_f32_k16(lds_quad(s.a, 16 * I + ln, 16 * m + 4 * lg),
                                    lds_col4(s.a, 16 * m + 4 * lg, 16 * J + ln), x);
                y = mma_f32_k16(lds_quad(s.a, 16 * I + ln, 16 * I + 4 * lg), x, zero4());
            }
            __syncthreads();
            if (wave < I) {
#pragma unroll
                for (int j = 0; j < 4; ++j) s.a[16 * I + 4 * lg + j][16 * wave + ln] = -y[j];
            }
            __syncthreads();
        }

        // ---- phase 4b (bf16 path): M = T Diag(beta), split once, in the
        // fragment-row layout [row][J pair][hi, lo][lane group][8 bf16] with
        // rows kMsRow bytes apart.
        if constexpr (!F32IO) {
            const int pj = half;
            const int c0 = 32 * pj + 4 * lg, c1 = c0 + 16;
            u32x4 mh, ml;
            quads_to_bf16_split(lds_quad(s.a, row, c0) * ld4(&s.beta[c0]),
                                lds_quad(s.a, row, c1) * ld4(&s.beta[c1]), mh, ml);
            unsigned char *b = msp + row * kMsRow + pj * 128 + lg * 16;
            *reinterpret_cast<u32x4 *>(b) = mh;
            *reinterpret_cast<u32x4 *>(b + 64) = ml;
            __syncthreads();
        }

        // ---- phase 5: -W fragments (from W^T tiles) and U tiles; M = T Diag(beta).
        // W^T tile (t, I) = sum_J (Gamma*K)^T_{tJ} M^T_{JI}: the accumulator
        // lane (n = r, g) holds W[16I + r][16t + 4g + j], the A-operand
        // fragment of -W in the state-propagation product.
        for_wave_units<4 * SL::NKF, NW>(wave, [&](int unit) {
            const int I = unit / SL::NKF, tp = unit % SL::NKF;
            const int nJ = I + 1;
            if constexpr (F32IO) {
                const int t = tp;
                f32x4 acc = zero4();
                for (int J = 0; J < nJ; ++J) {
                    const int cJ = 16 * J + 4 * lg;
                    const f32x4 mq = lds_quad(s.a, 16 * I + ln, cJ) * ld4(&s.beta[cJ]);
                    const f32x4 gk = lds_col4(krf, 16 * J + 4 * lg, 16 * t + ln) * s.pfx[J][16 * t + ln];
                    acc = mma_f32_k16(gk, mq, acc);
                }
                *reinterpret_cast<f32x4 *>(slab + SL::negW + ((size_t)(I * SL::NKF + tp) * 64 + lane) * 16) = -acc;
            } else {
                const int ca = 32 * tp + ln, cb = ca + 16;
                f32x4 acc0 = zero4(), acc1 = zero4();
                for (int pj = 0; pj < (nJ + 1) / 2; ++pj) {
                    const int cJ0 = 32 * pj + 4 * lg, cJ1 = cJ0 + 16;
                    const unsigned char *mb = msp + (16 * I + ln) * kMsRow + pj * 128 + lg * 16;
                    const u32x4 mh = *reinterpret_cast<const u32x4 *>(mb);
                    const u32x4 ml = *reinterpret_cast<const u32x4 *>(mb + 64);
                    const u32x4 gah = cat2(lds_bf16x4(gkh, ca, cJ0), lds_bf16x4(gkh, ca, cJ1));
                    const u32x4 gal = cat2(lds_bf16x4(gkl, ca, cJ0), lds_bf16x4(gkl, ca, cJ1));
                    const u32x4 gbh = cat2(lds_bf16x4(gkh, cb, cJ0), lds_bf16x4(gkh, cb, cJ1));
                    const u32x4 gbl = cat2(lds_bf16x4(gkl, cb, cJ0), lds_bf16x4(gkl, cb, cJ1));
                    acc0 = mma3_bf16(gah, gal, mh, ml, acc0);
                    acc1 = mma3_bf16(gbh, gbl, mh, ml, acc1);
                }
                store_f16(slab + SL::negW + ((size_t)(I * SL::NKF + tp) * 64 + lane) * 16, -acc0, -acc1);
            }
        });
        // U tile (I, w) = sum_J M_{IJ} V_{Jw}, in the accumulator layout the
        // state-propagation kernel starts V' from.
        for_wave_units<4 * KT, NW>(wave, [&](int unit) {
            const int I = unit / KT, w = unit % KT;
            const int nJ = I + 1;
            f32x4 acc = zero4();
            if constexpr (F32IO) {
                for (int J = 0; J < nJ; ++J) {
                    const int cJ = 16 * J + 4 * lg;
                    const f32x4 mq = lds_quad(s.a, 16 * I + ln, cJ) * ld4(&s.beta[cJ]);
                    acc = mma_f32_k16(mq, lds_col4(s.ke, 16 * J + 4 * lg, 16 * w + ln), acc);
                }
            } else {
                for (int pj = 0; pj < (nJ + 1) / 2; ++pj) {
                    const int cJ0 = 32 * pj + 4 * lg, cJ1 = cJ0 + 16;
                    const unsigned char *mb = msp + (16 * I + ln) * kMsRow + pj * 128 + lg * 16;
                    const u32x4 vb = cat2(lds_bf16x4(s.vt, 16 * w + ln, cJ0), lds_bf16x4(s.vt, 16 * w + ln, cJ1));
                    acc = mma_bf16_k32(*reinterpret_cast<const u32x4 *>(mb), vb, acc);
                    acc = mma_bf16_k32(*reinterpret_cast<const u32x4 *>(mb + 64), vb, acc);
                }
            }
            if constexpr (F32IO) {
                *reinterpret_cast<f32x4 *>(slab + SL::u + ((size_t)(I * KT + w) * 64 + lane) * 16) = acc;
            } else {
                float m = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(acc[j]));
                const int e = scale_exp(wave_max_nonneg(m));
                *reinterpret_cast<u32x2 *>(slab + SL::u + ((size_t)(I * KT + w) * 64 + lane) * 8) =
                    quad_to_f16(acc * exp2i(-e));
                if (lane == 0) reinterpret_cast<int *>(slab + SL::uexp)[I * KT + w] = e;
            }
        });
        ent = ent_next;
        ent_next = ent_after;
        a_cur = a_next;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Inter-chunk kernel.  Wave w of a workgroup owns value columns
// [16 vt, 16 vt + 16) of one (sequence, head); its state slice S[:, cols]
// lives in DK/16 fp32 accumulator tiles (lane (n, g) holds S[16t + 4g + j][16vt + n]).
// Per chunk, in the order of the chunk form:
//   V' = U - W S,   O = (Gamma*Q) S + A_qk V',   S = Diag(gamma_C) S + K~^T V'
// Value columns are independent, so each wave may scale its own S and V'
// slices: bf16 path, S and V' are multiplied by a power of two chosen from
// the wave's largest magnitude, rounded to fp16 for the MFMAs (fp16 stored
// operands, fp32 accumulation), and the products are scaled back exactly.
// The fp32 path uses fp32 MFMA and no scaling.
//
// Staging: the operands every wave shares (-W, Gamma*Q, K~^T, A_qk, gamma)
// reach LDS by direct global->LDS copies (global_load_lds_dwordx4, one 1 KiB
// fragment per wave instruction).  bf16 path: region A (-W, Gamma*Q: needed
// first in a step) rotates through three buffers and is fetched two chunks
// ahead, region B through two, fetched one chunk ahead; a step ends by
// waiting for everything except the A copies it issued last.  fp32 path
// (larger fragments): region B of this chunk streams during phase A, region
// A of the next chunk during phase B.
// ---------------------------------------------------------------------------
template <int D, bool F32IO>
struct InterShape {
    using SL = Slab<D, F32IO>;
    static constexpr int KT = D / 16;
    static constexpr int WPG = KT < 4 ? KT : 4;          // waves per workgroup
    static constexpr int NT = 64 * WPG;
    // bf16 path: region A ring of 3, region B ring of 2, and two output
    // staging tiles of 64 rows x (16 * WPG) bf16 columns
    static constexpr size_t ABYTES = (size_t)SL::FA * SL::FRAG, BBYTES = (size_t)SL::FB * SL::FRAG;
    static constexpr int OPITCH = 16 * WPG + 8;                  // bf16 elements per staged row
    static constexpr size_t obuf_bytes = F32IO ? 0 : (size_t)64 * OPITCH * 2;
    static constexpr size_t ring_bytes = 3 * ABYTES + 2 * BBYTES;
    static constexpr size_t lds_bytes = F32IO ? (size_t)(SL::FA + SL::FB) * SL::FRAG : ring_bytes + 2 * obuf_bytes;
};

// Copy `nfrag` consecutive 1 KiB fragments from global `src` to LDS `dst`,
// spread over the workgroup's waves.  Asynchronous: wait on vmcnt before use.
__device__ __forceinline__ void copy_frags_to_lds(const unsigned char *src, unsigned char *dst, int nfrag,
                                                  int wave, int nwaves, int lane) {
    for (int f = wave; f < nfrag; f += nwaves)
        __builtin_amdgcn_global_load_lds(src + (size_t)f * 1024 + lane * 16,
                                         (__attribute__((address_space(3))) void *)(dst + f * 1024), 16, 0, 0);
}

__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Store a finished 64 x 16 output tile (accumulator layout) for rows < L.
template <bool F32IO>
__device__ __forceinline__ void store_o_tile(void *o, const f32x4 (&acc)[4], int t0, int L, int H, int h,
                                             int D, int col, int lg) {
    const size_t rstride = (size_t)H * D;
    const size_t base = ((size_t)t0 * H + h) * D + col;
    if (L >= 64) {
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                store_io<F32IO>(o, base + (size_t)(16 * I + 4 * lg + j) * rstride, acc[I][j]);
    } else {
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * I + 4 * lg + j;
                if (r < L) store_io<F32IO>(o, base + (size_t)r * rstride, acc[I][j]);
            }
    }
}

template <int D, bool F32IO>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) inter_kernel(
    const float *__restrict__ h0, const int32_t *__restrict__ meta, const int4 *__restrict__ table,
    int N, int H, int max_chunks, const unsigned char *__restrict__ slabs, size_t slab_stride,
    void *__restrict__ o, float *__restrict__ hT, int groups) {
    using SL = Slab<D, F32IO>;
    using SHP = InterShape<D, F32IO>;
    constexpr int KT = D / 16;
    constexpr int WPG = SHP::WPG;
    constexpr size_t BUF = (size_t)(SL::FA + SL::FB) * SL::FRAG;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];

    // blockIdx -> (pair, column group) with every group of a pair on the same XCD
    const int b = blockIdx.x;
    const int xcd = b & 7, rest = b >> 3;
    const int cg = rest % groups;
    const int pair = (rest / groups) * 8 + xcd;
    if (pair >= N * H) return;
    const int n = pair / H, h = pair % H;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index in an SGPR
    const int ln = lane & 15, lg = lane >> 4;
    const int vt = cg * WPG + wave;
    const int col = 16 * vt + ln;

    f32x4 S[KT];
    const size_t srow = ((size_t)pair * D + col) * D;
#pragma unroll
    for (int t = 0; t < KT; ++t)
        S[t] = h0 ? *reinterpret_cast<const f32x4 *>(h0 + srow + 16 * t + 4 * lg) : zero4();

    const int c_begin = meta[n], c_end = meta[n + 1];
    auto slab_of = [&](int c) { return slabs + ((size_t)h * max_chunks + c) * slab_stride; };
    // U: fp32 tiles (fp32 path) or fp16 tiles with a per-tile exponent (bf16 path)
    using UReg = typename std::conditional<F32IO, f32x4, u32x2>::type;
    auto load_u = [&](int c, UReg *dst) {
        const UReg *us = reinterpret_cast<const UReg *>(slab_of(c) + SL::u);
#pragma unroll
        for (int I = 0; I < 4; ++I) dst[I] = us[(I * KT + vt) * 64 + lane];
    };
    // region A = [-W | Gamma*Q], region B = [K~^T | A_qk | gamma] of a buffer
    auto copy_A = [&](int c, unsigned char *buf) { copy_frags_to_lds(slab_of(c), buf, SL::FA, wave, WPG, lane); };
    auto copy_B = [&](int c, unsigned char *buf) {
        copy_frags_to_lds(slab_of(c) + SL::kdT, buf + SL::kdT, SL::FB, wave, WPG, lane);
    };
    // this lane's 16 bytes of fragment idx of the region at slab offset `off`
    auto frag = [&](const unsigned char *buf, size_t off, int idx) -> u32x4 {
        return *reinterpret_cast<const u32x4 *>(buf + off + ((size_t)idx * 64 + lane) * 16);
    };
    auto gamma_of = [&](const unsigned char *buf) { return reinterpret_cast<const f32x4 *>(buf + SL::gamma); };

    UReg u[4], un[4];
    f32x4 acc_o[4];
    int o_t0 = 0, o_L = 0;     // pending output of the previous chunk

    if constexpr (!F32IO) {
        // ------------------------------------------------------------- bf16 path
        // Output rows go out as whole 16 * WPG-column segments: each wave
        // computes its 64 x 16 tile row-major (O^T products), stages it in LDS,
        // and after the next barrier every lane stores 16-byte pieces of full rows.
        constexpr int OP = SHP::OPITCH;
        constexpr size_t AB = SHP::ABYTES, BB = SHP::BBYTES;
        unsigned char *aring = lds_raw, *bring = lds_raw + 3 * AB;
        uint16_t *obuf = reinterpret_cast<uint16_t *>(lds_raw + SHP::ring_bytes);
        auto flush_o = [&](int par, int t0, int L) {
            const uint16_t *ob = obuf + par * 64 * OP;
            constexpr int SEG = 16 * WPG / 8;                   // 16-byte pieces per row
            for (int i = tid; i < 64 * SEG; i += SHP::NT) {
                const int r = i / SEG, sgm = i % SEG;
                if (r < L)
                    *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(o) +
                                               ((size_t)(t0 + r) * H + h) * D + 16 * WPG * cg + 8 * sgm) =
                        *reinterpret_cast<const u32x4 *>(ob + r * OP + 8 * sgm);
            }
        };
        auto copyA = [&](int c, unsigned char *dst) { copy_frags_to_lds(slab_of(c), dst, SL::FA, wave, WPG, lane); };
        auto copyB = [&](int c, unsigned char *dst) {
            copy_frags_to_lds(slab_of(c) + SL::kdT, dst, SL::FB, wave, WPG, lane);
        };
        // A copies per wave: the last of a step's memory operations, and the
        // only ones still allowed in flight at its end
        constexpr int NA = SL::FA / WPG;
        static_assert(SL::FA % WPG == 0 && NA < 16 && NA % 4 == 0, "A fragments per wave");
        // token range of the sequence, from its first and last chunk records:
        // chunk c starts at t_first + 64 (c - c_begin), with at most t_end - start rows
        int t_first = 0, t_end = 0;
        if (c_begin < c_end) {
            const int4 e0 = table[c_begin], e1 = table[c_end - 1];
            t_first = e0.y;
            t_end = e1.y + e1.z;
        }
        if (c_begin < c_end) {
            copyA(c_begin, aring);
            copyB(c_begin, bring);
            load_u(c_begin, u);
            if (c_begin + 1 < c_end) copyA(c_begin + 1, aring + AB);
        }
        wait_all_memory();
        __syncthreads();
        for (int c = c_begin; c < c_end; ++c) {
            const int i = c - c_begin;
            const int par = i & 1;
            const unsigned char *abuf = aring + (i % 3) * AB;
            const unsigned char *bbuf = bring + par * BB;
            // a region-B offset of the slab, seen in the B buffer
            auto fragB = [&](size_t off, int idx) -> u32x4 {
                return *reinterpret_cast<const u32x4 *>(bbuf + (off - SL::kdT) + ((size_t)idx * 64 + lane) * 16);
            };
            auto fragA = [&](size_t off, int idx) -> u32x4 {
                return *reinterpret_cast<const u32x4 *>(abuf + off + ((size_t)idx * 64 + lane) * 16);
            };
            const int *uexp = reinterpret_cast<const int *>(bbuf + (SL::uexp - SL::kdT));
            if (o_L > 0) flush_o(par ^ 1, o_t0, o_L);   // the previous chunk's rows
            if (c + 1 < c_end) {
                load_u(c + 1, un);
                copyB(c + 1, bring + (par ^ 1) * BB);
            }
            // A copies of chunk c + 2, issued a few at a time between this
            // step's products so that the memory pipeline works under the math
            const bool fetch_a = c + 2 < c_end;
            const unsigned char *a_src = slab_of(fetch_a ? c + 2 : c);
            unsigned char *a_dst = aring + ((i + 2) % 3) * AB;
            auto copyA_part = [&](int r) {
                const int f = wave + r * WPG;
                __builtin_amdgcn_global_load_lds(a_src + (size_t)f * 1024 + lane * 16,
                                                 (__attribute__((address_space(3))) void *)(a_dst + f * 1024), 16, 0,
                                                 0);
            };

            // S -> fp16 with a per-wave power-of-two scale
            float m = 0.f;
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(S[t][j]));
            const int eS = scale_exp(wave_max_nonneg(m));
            const float dS = exp2i(-eS), uS = exp2i(eS);
            u32x4 sf[KT / 2];
#pragma unroll
            for (int p = 0; p < KT / 2; ++p) sf[p] = quads_to_f16(S[2 * p] * dS, S[2 * p + 1] * dS);

            f32x4 vp[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (fetch_a) {
#pragma unroll
                    for (int r = 0; r < NA / 4; ++r) copyA_part(I * (NA / 4) + r);
                }
                f32x4 ws = zero4(), qs = zero4();
#pragma unroll
                for (int p = 0; p < KT / 2; ++p) {
                    ws = mma_f16_k32(fragA(SL::negW, I * (KT / 2) + p), sf[p], ws);
                    // O^T = S^T (Gamma*Q)^T: the same fragments with the operands
                    // swapped, so the accumulator holds O row-major (lane (n, g):
                    // row n, columns 4g..4g+3) and o needs no transpose
                    qs = mma_f16_k32(sf[p], fragA(SL::qg, I * (KT / 2) + p), qs);
                }
                vp[I] = f16x4_to_quad(u[I]) * exp2i(uexp[I * KT + vt]) + ws * uS;
                acc_o[I] = qs * uS;
            }

            // V' -> fp16 with its own per-wave scale
            m = 0.f;
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(vp[I][j]));
            const int eV = scale_exp(wave_max_nonneg(m));
            const float dV = exp2i(-eV), uV = exp2i(eV);
            const u32x4 vf0 = quads_to_f16(vp[0] * dV, vp[1] * dV);
            const u32x4 vf1 = quads_to_f16(vp[2] * dV, vp[3] * dV);

            uint16_t *ob = obuf + par * 64 * OP;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                // (A_qk V')^T = V'^T A_qk^T, row-major like O above
                f32x4 a = mma_f16_k32(vf0, fragB(SL::aqk, aqk_frag(I, 0)), zero4());
                if (I >= 2) a = mma_f16_k32(vf1, fragB(SL::aqk, aqk_frag(I, 1)), a);
                acc_o[I] += a * uV;
                *reinterpret_cast<u32x2 *>(ob + (16 * I + ln) * OP + 16 * wave + 4 * lg) =
                    u32x2{f32x2_to_bf16x2(acc_o[I][0], acc_o[I][1]), f32x2_to_bf16x2(acc_o[I][2], acc_o[I][3])};
            }
            const f32x4 *gam = reinterpret_cast<const f32x4 *>(bbuf + (SL::gamma - SL::kdT));
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                f32x4 a = mma_f16_k32(fragB(SL::kdT, t * 2), vf0, zero4());
                a = mma_f16_k32(fragB(SL::kdT, t * 2 + 1), vf1, a);
                S[t] = S[t] * gam[4 * t + lg] + a * uV;
            }
            o_t0 = t_first + kChunk * i;
            o_L = min(kChunk, t_end - o_t0);
            // everything but this step's A copies must have landed (memory
            // operations complete in issue order)
            if (c + 2 < c_end)
                __builtin_amdgcn_s_waitcnt((NA & 15) | (0x7 << 4) | (0xf << 8) | ((NA >> 4) << 14));
            else
                wait_all_memory();
            __syncthreads();
#pragma unroll
            for (int I = 0; I < 4; ++I) u[I] = un[I];
        }
        if (o_L > 0) flush_o((c_end - c_begin - 1) & 1, o_t0, o_L);
        o_L = 0;
    } else {
        // ------------------------------------------------------------- fp32 path
        unsigned char *buf = lds_raw;
        if (c_begin < c_end) {
            copy_A(c_begin, buf);
            load_u(c_begin, u);
        }
        wait_all_memory();
        __syncthreads();
        for (int c = c_begin; c < c_end; ++c) {
            copy_B(c, buf);
            if (c + 1 < c_end) load_u(c + 1, un);
            if (o_L > 0) store_o_tile<F32IO>(o, acc_o, o_t0, o_L, H, h, D, col, lg);
            const int4 ent = table[c];
            f32x4 vp[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                vp[I] = u[I];
                acc_o[I] = zero4();
#pragma unroll
                for (int t = 0; t < KT; ++t) {
                    vp[I] = mma_f32_k16(__builtin_bit_cast(f32x4, frag(buf, SL::negW, I * KT + t)), S[t], vp[I]);
                    acc_o[I] = mma_f32_k16(__builtin_bit_cast(f32x4, frag(buf, SL::qg, I * KT + t)), S[t], acc_o[I]);
                }
            }
            wait_all_memory();
            __syncthreads();
            if (c + 1 < c_end) copy_A(c + 1, buf);
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int J = 0; J <= I; ++J)
                    acc_o[I] = mma_f32_k16(__builtin_bit_cast(f32x4, frag(buf, SL::aqk, I * 4 + J)), vp[J], acc_o[I]);
            const f32x4 *gam = gamma_of(buf);
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                S[t] = S[t] * gam[4 * t + lg];
#pragma unroll
                for (int J = 0; J < 4; ++J)
                    S[t] = mma_f32_k16(__builtin_bit_cast(f32x4, frag(buf, SL::kdT, t * 4 + J)), vp[J], S[t]);
            }
            o_t0 = ent.y;
            o_L = ent.z;
            wait_all_memory();
            __syncthreads();
#pragma unroll
            for (int I = 0; I < 4; ++I) u[I] = un[I];
        }
    }
    if (o_L > 0) store_o_tile<F32IO>(o, acc_o, o_t0, o_L, H, h, D, col, lg);
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
                       p.max_chunks, meta, table, reinterpret_cast<float *>(a.ws + p.off_null), D);
    if (hipGetLastError() != hipSuccess) return -1;

    const long long items = (long long)p.max_chunks * a.H;
    if constexpr (!F32IO) {
        if (launch_intra_bf16<D>(a, meta, table, reinterpret_cast<const float *>(a.ws + p.off_null), slabs) != 0)
            return -1;
    } else if (items > 0) {
        const size_t lds = sizeof(IntraLds<D>);
        if (!set_lds(&intra_kernel<D, F32IO>, lds)) return -1;
        const int grid = (int)std::min<long long>(items, (long long)device_cus());
        hipLaunchKernelGGL((intra_kernel<D, F32IO>), dim3(grid), dim3(64 * kIntraWaves), lds, a.stream, a.q, a.k,
                           a.v, a.z, a.A, a.beta, meta, table, a.N, a.H, p.max_chunks, slabs,
                           p.slab_bytes);
        if (hipGetLastError() != hipSuccess) return -1;
    }

    using SHP = InterShape<D, F32IO>;
    const int groups = SHP::KT / SHP::WPG;
    const int pairs = a.N * a.H;
    if (pairs > 0) {
        if (!set_lds(&inter_kernel<D, F32IO>, SHP::lds_bytes)) return -1;
        const int pair_blocks = (pairs + 7) / 8 * 8;
        hipLaunchKernelGGL((inter_kernel<D, F32IO>), dim3(pair_blocks * groups), dim3(SHP::NT),
                           SHP::lds_bytes, a.stream, a.h0, meta, table, a.N, a.H, p.max_chunks, slabs,
                           p.slab_bytes, a.o, a.hT, groups);
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
