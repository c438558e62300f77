// kda_prefill.hip -- chunkwise-parallel KDA prefill for gfx950.
//
// The kernels, on the caller's stream unless pipelined (below):
//   chunk_table_kernel  cu_seqlens -> first chunk of every sequence and a
//                       (sequence, first token, length) record per chunk;
//                       chunks of 64 tokens start at every sequence start.
//   intra kernels       (kda_intra.hip for bf16 inputs, kda_intra_f32.hip for
//                       fp32) parallel over (chunk, head): the bounded gate,
//                       chunk-local log-decays, the decay-rescaled Gram
//                       matrices, the unit-lower-triangular solve and the
//                       W / U products.  Write one "slab" of MFMA-ready
//                       fragments per (chunk, head).
//   inter_kernel        one wavefront per (segment, head, 16 value columns):
//                       walks the segment's chunks in order, carrying the
//                       fp32 state in MFMA accumulators.  A segment is a whole
//                       sequence unless long sequences are split (below).
//   combine_kernel      only for split sequences: composes the segments'
//                       affine state maps into every segment's incoming state.
//
// Chunk-block pipeline (long sequences, bf16): the chunk table is cut into
// runs, and the intra kernel of run j + 1 (caller's stream) runs beside the
// inter kernel of run j (a helper stream of the calling thread, ordered by
// events); the state crosses run boundaries through the workspace.  The
// fused call runs the same pipeline with a feature pass before each intra
// kernel and the inter kernel in its gated output mode.
//
// Split sequences (intra-device context parallelism, "Kimi K3：架构…" §11.1
// and the KCP merge of the devpress K3 walk-through §8.1, Eq 17): inter_kernel
// first runs in its transition mode over every segment but a sequence's last,
// producing the map
// S_in -> M S_in + S~ of its chunks; combine_kernel chains the maps from h0;
// inter_kernel then runs every segment's outputs in parallel.
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
#include <climits>
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

bool plan_prefill(int N, int T, int H, int dk, int dv, bool f32io, int P, int blocks, PrefillPlan *p, bool fused) {
    size_t sb = slab_bytes(dk, dv, f32io);
    if (sb == 0 || N < 0 || T < 0 || H <= 0 || P < 1 || P > kMaxSegments) return false;
    p->max_chunks = (int)(((long long)T + kChunk - 1) / kChunk + N);
    p->slab_bytes = sb;
    p->P = P;
    p->off_meta = 0;
    p->off_table = align256((size_t)(N + 2) * 4);
    p->off_null = p->off_table + align256((size_t)p->max_chunks * 16);
    p->off_ckoff = p->off_null + align256((size_t)dk * 4 + (size_t)dk * 4 + 4);
    p->off_segs = p->off_ckoff + align256((size_t)(N + 1) * 4);
    const size_t units = (size_t)N * P * H, dd = (size_t)dk * dk * 4;
    p->off_trans = p->off_segs + align256((size_t)N * P * 16);
    p->off_sin = p->off_trans + (P > 1 ? units * 2 * dd : 0);
    p->off_slabs = p->off_sin + (P > 1 ? units * dd : 0);
    p->blocks = P == 1 && !f32io && blocks > 1 ? blocks : 1;
    p->off_claims = p->off_slabs + (size_t)H * p->max_chunks * sb;
    p->off_carry = p->off_claims + (p->blocks > 1 ? align256((size_t)p->blocks * 4) : 0);
    p->staged = fused && p->blocks > 1;
    p->off_qkv = p->off_carry + (p->blocks > 1 ? align256((size_t)N * H * dv * dk * 4) : 0);
    p->total = p->off_qkv + (p->staged ? 3 * align256((size_t)T * H * dk * (f32io ? 4 : 2)) : 0);
    return true;
}

// Segment flags: a sequence's chunks are split into runs ("segments") that
// the inter kernel walks independently once each segment's incoming state is
// known (intra-device context parallelism).
constexpr int kSegValid = 1, kSegFirst = 2, kSegLast = 4;
// inter_kernel modes: the outputs and final states; or the segment's
// transition, two states carried side by side over the same chunk operands:
// the matrix M (run from the identity with U = 0) and the offset S~ (run from zero)
// the outputs with the output gate applied (fused prefill): y = Sigmoid(g) *
// RMSNorm(o), one workgroup per head so that a row's RMS covers its dv channels
constexpr int kModeOutput = 0, kModeTrans = 1, kModeGate = 2;

// ---------------------------------------------------------------------------
// Chunk table.  One workgroup.  meta[n] = first chunk of sequence n,
// meta[N] = number of chunks; table[c] = {n, first token, length, first chunk of n};
// segs[n P + k] = {n, first chunk, end chunk, flags} of segment k of sequence n;
// with checkpoints, ck_off[n] = index of sequence n's first checkpoint.
// Sequence bounds are clamped to [0, T] and the chunk count to max_chunks,
// so a malformed cu_seqlens can give wrong results but no stray access.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) chunk_table_kernel(const int32_t *__restrict__ cu, int N,
                                                          int T, int max_chunks,
                                                          int32_t *__restrict__ meta,
                                                          int4 *__restrict__ table,
                                                          float *__restrict__ null_row, int d, int P,
                                                          int4 *__restrict__ segs, int ck_chunks, int ck_cap,
                                                          int32_t *__restrict__ ck_off,
                                                          int32_t *__restrict__ ck_off_user,
                                                          int32_t *__restrict__ claims, int nclaims) {
    __shared__ int32_t scan[256];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    // the item counters of a pipelined prefill's blocks
    if (tid < nclaims) claims[tid] = 0;
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
        // .w marks a sequence's first chunk (the fused prefill's feature path
        // reads the carried conv window there)
        table[c] = make_int4(n, first, min(kChunk, e - first), c == meta[n] ? 1 : 0);
    }
    // segments: sequence n is cut into Pn = clamp(chunks, 1, P) runs of
    // consecutive chunks of near-equal length; slots past Pn are invalid
    for (int i = tid; i < N * P; i += 256) {
        const int n = i / P, k = i % P;
        const int c0 = meta[n], nc = meta[n + 1] - c0;
        const int pn = max(1, min(P, nc));
        int4 r = make_int4(n, 0, 0, 0);
        if (k < pn) {
            r.y = c0 + (int)((long long)k * nc / pn);
            r.z = c0 + (int)((long long)(k + 1) * nc / pn);
            r.w = kSegValid | (k == 0 ? kSegFirst : 0) | (k == pn - 1 ? kSegLast : 0);
        }
        segs[i] = r;
    }
    // checkpoints: sequence n has floor(len / (64 ck_chunks)) of them, the
    // first at index ck_off[n]; indices are clamped to the caller's ck_cap
    if (ck_chunks > 0) {
        __syncthreads();
        if (tid == 0) carry = 0;
        __syncthreads();
        for (int base = 0; base < N; base += 256) {
            const int n = base + tid;
            int cnt = 0;
            if (n < N) {
                const int s = min(max(cu[n], 0), T), e = min(max(cu[n + 1], 0), T);
                cnt = e > s ? (e - s) / (kChunk * ck_chunks) : 0;
            }
            scan[tid] = cnt;
            __syncthreads();
            for (int off = 1; off < 256; off <<= 1) {
                int x = tid >= off ? scan[tid - off] : 0;
                __syncthreads();
                scan[tid] += x;
                __syncthreads();
            }
            if (n < N) {
                const int first = min(carry + scan[tid] - cnt, ck_cap);
                ck_off[n] = first;
                if (ck_off_user) ck_off_user[n] = first;
            }
            __syncthreads();
            if (tid == 255) carry += scan[255];
            __syncthreads();
        }
        if (tid == 0) {
            ck_off[N] = min(carry, ck_cap);
            if (ck_off_user) ck_off_user[N] = min(carry, ck_cap);
        }
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
template <int D, bool F32IO, int MODE>
struct InterShape {
    using SL = Slab<D, F32IO>;
    static constexpr bool GATE = MODE == kModeGate;
    static constexpr int KT = D / 16;
    // waves per workgroup, 16 value columns each; the gate mode needs whole
    // rows in one workgroup
    static constexpr int WPG = GATE ? KT : (KT < 4 ? KT : 4);
    static constexpr int NT = 64 * WPG;
    static constexpr int GROUPS = KT / WPG;              // workgroups per (segment, head)
    static constexpr int WAVES_PER_SIMD = (NT + 255) / 256;
    // bf16 path: region A ring of 3, region B ring of 2, and output staging
    // tiles of 64 rows x (16 * WPG) columns: two in bf16; in the gate mode one
    // in fp16 with a power-of-two exponent per wave
    static constexpr size_t ABYTES = (size_t)SL::FA * SL::FRAG, BBYTES = (size_t)SL::FB * SL::FRAG;
    static constexpr int OPITCH = 16 * WPG + 8;                  // elements per staged row
    static constexpr size_t obuf_bytes = F32IO ? 0 : (size_t)64 * OPITCH * 2;
    static constexpr size_t ring_bytes = 3 * ABYTES + 2 * BBYTES;
    static constexpr size_t lds_bytes =
        F32IO ? (size_t)(SL::FA + SL::FB) * SL::FRAG : ring_bytes + (GATE ? obuf_bytes + 64 : 2 * obuf_bytes);
    static_assert(!(GATE && F32IO), "the gate mode is a bf16-path mode");
    static_assert(lds_bytes <= 160 * 1024, "LDS per workgroup");
};

// Copy one 1 KiB fragment from global `src` to LDS `dst` (16 bytes per lane).
// Asynchronous: wait on vmcnt before use.
__device__ __forceinline__ void copy_frag_to_lds(const unsigned char *src, unsigned char *dst, int lane) {
    __builtin_amdgcn_global_load_lds(src + lane * 16, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

// Copy `nfrag` consecutive 1 KiB fragments from global `src` to LDS `dst`,
// spread over the workgroup's waves.  Asynchronous: wait on vmcnt before use.
__device__ __forceinline__ void copy_frags_to_lds(const unsigned char *src, unsigned char *dst, int nfrag,
                                                  int wave, int nwaves, int lane) {
    for (int f = wave; f < nfrag; f += nwaves) copy_frag_to_lds(src + (size_t)f * 1024, dst + f * 1024, lane);
}

__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// A global load the compiler does not track.  The compiler counts vmcnt for
// its own loads only up to the first direct global->LDS copy issued after
// them, and waits for everything (vmcnt(0)) at their use.  Loads issued with
// this helper before a step's copies are instead covered by the step's
// explicit in-order wait; `settle` then marks the register as written at
// that point, so that no use of it can move above the wait.
__device__ __forceinline__ u32x2 load_untracked(const u32x2 *p) {
    u32x2 r;
    asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    return r;
}
__device__ __forceinline__ u32x4 load_untracked4(const u32x4 *p) {
    u32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    return r;
}
__device__ __forceinline__ void settle(u32x2 &r) { asm volatile("" : "+v"(r)); }
__device__ __forceinline__ void settle(u32x4 &r) { asm volatile("" : "+v"(r)); }

// Workgroup barrier for LDS written by ds instructions.  __syncthreads (and
// any release fence covering LDS) also waits for every direct global->LDS
// copy still in flight, since those are LDS writes counted by vmcnt --
// including copies meant for a later step.  Here the caller waits for the
// copies it needs with an explicit vmcnt; the barrier waits for the wave's
// own ds operations only.  The asm's memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

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

// x (n f32x4 tiles, n even) -> fp16 K32 fragments scaled by the power of two
// that the wave's largest magnitude asks for; returns the factor that undoes it
template <int n>
__device__ __forceinline__ float to_f16_scaled(const f32x4 *x, u32x4 *out) {
    float m = 0.f;
#pragma unroll
    for (int t = 0; t < n; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(x[t][j]));
    const int e = scale_exp(wave_max_nonneg(m));
    const float d = exp2i(-e);
#pragma unroll
    for (int p = 0; p < n / 2; ++p) out[p] = quads_to_f16(x[2 * p] * d, x[2 * p + 1] * d);
    return exp2i(e);
}

// S <- Diag(gamma_C) S + K~^T V' for one accumulator quad: a = K~^T V' at the
// scale of V''s fp16 copy and u the power of two that undoes it, so a * u is
// exact and one fused multiply-add rounds the new state once.  Written out
// rather than left to the compiler's contraction choice, which can differ
// between instantiations (output, gated-output and transition modes) and
// between compiler versions; either choice is within the error bound, but
// only a fixed one keeps the modes' states bit-identical.
__device__ __forceinline__ f32x4 decay_add(f32x4 s, f32x4 g, f32x4 a, float u) {
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = __builtin_fmaf(s[j], g[j], a[j] * u);
    return r;
}

template <int D, bool F32IO, int MODE>
__global__ void __launch_bounds__((InterShape<D, F32IO, MODE>::NT))
    __attribute__((amdgpu_waves_per_eu((InterShape<D, F32IO, MODE>::WAVES_PER_SIMD),
                                       (InterShape<D, F32IO, MODE>::WAVES_PER_SIMD)))) inter_kernel(
    const float *__restrict__ h0, const float *__restrict__ s_in, const int4 *__restrict__ segs,
    const int4 *__restrict__ table, int nseg, int H, int max_chunks, const unsigned char *__restrict__ slabs,
    size_t slab_stride, void *__restrict__ o, float *__restrict__ hT, float *__restrict__ trans, int groups,
    const int32_t *__restrict__ meta, const int32_t *__restrict__ ck_off, float *__restrict__ ck, int ck_chunks,
    const uint16_t *__restrict__ gate, const float *__restrict__ norm_w, float eps, int blk_lo, int blk_hi,
    float *__restrict__ carry) {
    static_assert(MODE == kModeOutput || MODE == kModeTrans || MODE == kModeGate, "mode");
    constexpr bool TR = MODE == kModeTrans;
    constexpr bool OUT = !TR;                       // the mode writes outputs and the final state
    constexpr bool GATE = MODE == kModeGate;
    using SL = Slab<D, F32IO>;
    using SHP = InterShape<D, F32IO, MODE>;
    constexpr int KT = D / 16;
    constexpr int WPG = SHP::WPG;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];

    // blockIdx -> (segment and head, column group) with every group of a
    // (segment, head) on the same XCD
    const int b = blockIdx.x;
    const int xcd = b & 7, rest = b >> 3;
    const int cg = rest % groups;
    const int unit = (rest / groups) * 8 + xcd;
    if (unit >= nseg * H) return;
    const int sg = unit / H, h = unit % H;
    const int4 rec = segs[sg];
    if (!(rec.w & kSegValid)) return;
    if (TR && (rec.w & kSegLast)) return;   // no transition after the last segment
    const int n = rec.x;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index in an SGPR
    const int ln = lane & 15, lg = lane >> 4;
    const int vt = cg * WPG + wave;
    const int col = 16 * vt + ln;

    // The chunks this launch walks: the segment's, or (block pipeline, bf16
    // output and gated-output modes) their part in [blk_lo, blk_hi) of the chunk table.  A
    // sequence that began in an earlier block starts from `carry`, one that
    // goes on into a later block leaves its state there.  An empty sequence
    // belongs to the block holding its position.
    int c_begin = rec.y, c_end = rec.z;
    bool from_carry = false, to_carry = false;
    if (OUT && !F32IO && carry) {
        const int lo_c = max(c_begin, blk_lo), hi_c = min(c_end, blk_hi);
        const bool here = c_begin < c_end ? lo_c < hi_c : (c_begin >= blk_lo && c_begin < blk_hi);
        if (!here) return;
        from_carry = lo_c > c_begin;
        to_carry = hi_c < c_end;
        c_begin = lo_c;
        c_end = hi_c;
    }

    // initial state: h0 (or zero) for a sequence in one segment, otherwise
    // the incoming state the combine kernel wrote (for the first segment a
    // copy of h0, so that h0 is never read here when hT may overwrite it);
    // a transition starts M from the identity (in S) and S~ from zero (in S2)
    f32x4 S[KT], S2[TR ? KT : 1];
    {
        const float *src = nullptr;
        if constexpr (!TR)
            src = from_carry ? carry + ((size_t)(n * H + h) * D + col) * D
                  : (rec.w & kSegFirst) && (rec.w & kSegLast)
                      ? (h0 ? h0 + ((size_t)(n * H + h) * D + col) * D : nullptr)
                      : s_in + ((size_t)(sg * H + h) * D + col) * D;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            if constexpr (TR) {
#pragma unroll
                for (int j = 0; j < 4; ++j) S[t][j] = (16 * t + 4 * lg + j == col) ? 1.f : 0.f;
                S2[t] = zero4();
            } else {
                S[t] = src ? *reinterpret_cast<const f32x4 *>(src + 16 * t + 4 * lg) : zero4();
            }
        }
    }

    // state checkpoints (output mode): after every chunk that ends 64 ck_chunks
    // tokens into the sequence, up to the sequence's count
    int ck_c0 = 0, ck_first = 0, ck_count = 0;
    if (OUT && ck) {
        ck_c0 = meta[n];
        ck_first = ck_off[n];
        ck_count = ck_off[n + 1] - ck_first;
    }
    auto checkpoint = [&](int c) {   // S holds the state after chunk c
        if (!OUT || !ck) return;
        const int pos = c - ck_c0 + 1;
        if (pos % ck_chunks != 0 || pos / ck_chunks > ck_count) return;
        float *dst = ck + (((size_t)(ck_first + pos / ck_chunks - 1) * H + h) * D + col) * D;
#pragma unroll
        for (int t = 0; t < KT; ++t) *reinterpret_cast<f32x4 *>(dst + 16 * t + 4 * lg) = S[t];
    };
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
        int *oexp = reinterpret_cast<int *>(lds_raw + SHP::ring_bytes + SHP::obuf_bytes);   // gate mode
        constexpr int SEG = 16 * WPG / 8;                       // 16-byte pieces per row
        constexpr int PPT = 64 * SEG / SHP::NT;                 // pieces per thread (2)
        static_assert(64 * SEG % SHP::NT == 0, "pieces per thread");
        auto flush_o = [&](int par, int t0, int L) {
            const uint16_t *ob = obuf + par * 64 * OP;
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                const int i = tid + SHP::NT * k;
                const int r = i / SEG, sgm = i % SEG;
                if (r < L)
                    *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(o) +
                                               ((size_t)(t0 + r) * H + h) * D + 16 * WPG * cg + 8 * sgm) =
                        *reinterpret_cast<const u32x4 *>(ob + r * OP + 8 * sgm);
            }
        };
        // Gate mode.  The SEG threads of a row are consecutive lanes holding
        // 8 channels each: the row's sum of squares is a lane-group
        // reduction, then y = o / sqrt(mean(o^2) + eps) * w * Sigmoid(g), in
        // the order of the standalone gate kernel, rounded once to bf16.
        // g of the flushed chunk's rows was loaded during the step before.
        f32x4 nw[2];
        u32x4 gcur[PPT], gnext[PPT];
        if constexpr (GATE) {
            const int c0 = 8 * (tid % SEG);
            nw[0] = *reinterpret_cast<const f32x4 *>(norm_w + c0);
            nw[1] = *reinterpret_cast<const f32x4 *>(norm_w + c0 + 4);
        }
        auto flush_gate = [&](int t0, int L) {
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                const int i = tid + SHP::NT * k;
                const int r = i / SEG, sgm = i % SEG;
                const u32x4 raw = *reinterpret_cast<const u32x4 *>(obuf + r * OP + 8 * sgm);
                const float sc = exp2i(oexp[sgm >> 1]);        // the wave that wrote these 8 columns
                f32x4 ov[2] = {f16x4_to_quad(u32x2{raw[0], raw[1]}), f16x4_to_quad(u32x2{raw[2], raw[3]})};
                ov[0] *= sc;
                ov[1] *= sc;
                float ss = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) ss += ov[0][j] * ov[0][j] + ov[1][j] * ov[1][j];
                ss = lane_group_sum<SEG>(ss);
                const float inv = fast_rsq(ss * (1.f / D) + eps);
                f32x4 gv[2];
                bf16_to_quads(gcur[k], gv[0], gv[1]);
                f32x4 y[2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        y[hf][j] = ov[hf][j] * inv * nw[hf][j] * fast_rcp(1.f + __expf(-gv[hf][j]));
                if (r < L)
                    *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(o) + ((size_t)(t0 + r) * H + h) * D +
                                               8 * sgm) = quads_to_bf16(y[0], y[1]);
            }
        };
        auto copyA = [&](int c, unsigned char *dst) { copy_frags_to_lds(slab_of(c), dst, SL::FA, wave, WPG, lane); };
        auto copyB = [&](int c, unsigned char *dst) {
            copy_frags_to_lds(slab_of(c) + SL::kdT, dst, SL::FB, wave, WPG, lane);
        };
        // region B of the slab at `src`, unrolled: wave w copies fragments w,
        // w + WPG, ...; only the last round depends on the (uniform) wave index
        auto copyB_from = [&](const unsigned char *src, unsigned char *dst) {
            constexpr int NB = (SL::FB + WPG - 1) / WPG;
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                const int f = wave + r * WPG;
                if (r < NB - 1 || f < SL::FB) copy_frag_to_lds(src + SL::kdT + (size_t)f * 1024, dst + f * 1024, lane);
            }
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
        // the slab of chunk c, and the A ring slot that holds it (the slot
        // two chunks ahead is the one before it): advanced step by step
        const unsigned char *slab_c = slab_of(c_begin);
        int aslot = 0;
        for (int c = c_begin; c < c_end; ++c) {
            const int i = c - c_begin;
            const int par = i & 1;
            const unsigned char *abuf = aring + aslot * AB;
            const unsigned char *bbuf = bring + par * BB;
            // chunks c + 1 and c + 2, clamped to the sequence's last chunk
            const unsigned char *slab_n1 = c + 1 < c_end ? slab_c + slab_stride : slab_c;
            const unsigned char *slab_n2 = c + 2 < c_end ? slab_c + 2 * slab_stride : slab_c;
            // a region-B offset of the slab, seen in the B buffer
            auto fragB = [&](size_t off, int idx) -> u32x4 {
                return *reinterpret_cast<const u32x4 *>(bbuf + (off - SL::kdT) + ((size_t)idx * 64 + lane) * 16);
            };
            auto fragA = [&](size_t off, int idx) -> u32x4 {
                return *reinterpret_cast<const u32x4 *>(abuf + off + ((size_t)idx * 64 + lane) * 16);
            };
            const int *uexp = reinterpret_cast<const int *>(bbuf + (SL::uexp - SL::kdT));
            if constexpr (GATE) {
                if (o_L > 0) flush_gate(o_t0, o_L);            // the previous chunk's rows
            } else if constexpr (OUT) {
                if (i > 0) checkpoint(c - 1);
            }
            // The next chunk's U and region B, and the region-A copies of chunk
            // c + 2 issued a few at a time between this step's products.  They
            // are issued on every step (chunk indices clamped, into ring slots
            // that are free) so that the same number of memory operations is in
            // flight on every path: the compiler can then wait for U by count
            // instead of draining every copy.
            {
                const u32x2 *us = reinterpret_cast<const u32x2 *>(slab_n1 + SL::u);
#pragma unroll
                for (int I = 0; I < 4; ++I) un[I] = load_untracked(us + (I * KT + vt) * 64 + lane);
            }
            if constexpr (GATE) {
                // this chunk's g rows, flushed at the next step (rows past the
                // chunk's end read its first row, and are not stored)
                const int t0 = t_first + kChunk * i, L = min(kChunk, t_end - t0);
#pragma unroll
                for (int k = 0; k < PPT; ++k) {
                    const int pi = tid + SHP::NT * k;
                    const int r = pi / SEG, sgm = pi % SEG;
                    gnext[k] = load_untracked4(reinterpret_cast<const u32x4 *>(
                        gate + ((size_t)(t0 + (r < L ? r : 0)) * H + h) * D + 8 * sgm));
                }
            }
            copyB_from(slab_n1, bring + (par ^ 1) * BB);
            const unsigned char *a_src = slab_n2;
            unsigned char *a_dst = aring + (aslot == 0 ? 2 : aslot - 1) * AB;
            auto copyA_part = [&](int r) {
                const int f = wave + r * WPG;
                __builtin_amdgcn_global_load_lds(a_src + (size_t)f * 1024 + lane * 16,
                                                 (__attribute__((address_space(3))) void *)(a_dst + f * 1024), 16, 0,
                                                 0);
            };

            // LDS reads are issued a phase ahead of their use, so their latency
            // hides behind VALU and MFMA work instead of stalling each product:
            // the -W and Gamma*Q fragments of row tile 0 and the U exponents
            // before the S conversion, those of row tile I + 1 during tile I,
            // and K~^T, A_qk and gamma_C during the last tile.
            u32x4 fwc[KT / 2], fqc[KT / 2];
            auto read_tile = [&](int I, u32x4 *fw, u32x4 *fq) {
#pragma unroll
                for (int p = 0; p < KT / 2; ++p) {
                    fw[p] = fragA(SL::negW, I * (KT / 2) + p);
                    if constexpr (!TR) fq[p] = fragA(SL::qg, I * (KT / 2) + p);
                }
            };
            read_tile(0, fwc, fqc);
            int uex[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) uex[I] = uexp[I * KT + vt];
            // S -> fp16 with a per-wave power-of-two scale (and S2 with its own)
            u32x4 sf[KT / 2], sf2[TR ? KT / 2 : 1];
            const float uS = to_f16_scaled<KT>(S, sf);
            float uS2 = 0.f;
            if constexpr (TR) uS2 = to_f16_scaled<KT>(S2, sf2);

            f32x4 vp[4], vp2[TR ? 4 : 1];
            u32x4 kfr[2 * KT], afr[OUT ? SL::NAQ : 1];
            f32x4 gmr[KT];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
#pragma unroll
                for (int r = 0; r < NA / 4; ++r) copyA_part(I * (NA / 4) + r);
                u32x4 fwn[KT / 2], fqn[KT / 2];
                if (I < 3) read_tile(I + 1, fwn, fqn);
                if (I == 3) {
#pragma unroll
                    for (int t = 0; t < 2 * KT; ++t) kfr[t] = fragB(SL::kdT, t);
                    const f32x4 *gp = reinterpret_cast<const f32x4 *>(bbuf + (SL::gamma - SL::kdT));
#pragma unroll
                    for (int t = 0; t < KT; ++t) gmr[t] = gp[4 * t + lg];
                    if constexpr (OUT) {
#pragma unroll
                        for (int f = 0; f < SL::NAQ; ++f) afr[f] = fragB(SL::aqk, f);
                    }
                }
                f32x4 ws = zero4(), qs = zero4(), ws2 = zero4();
#pragma unroll
                for (int p = 0; p < KT / 2; ++p) {
                    const u32x4 fw = fwc[p];
                    ws = mma_f16_k32(fw, sf[p], ws);
                    if constexpr (TR) {
                        ws2 = mma_f16_k32(fw, sf2[p], ws2);
                    } else {
                        // O^T = S^T (Gamma*Q)^T: the same fragments with the operands
                        // swapped, so the accumulator holds O row-major (lane (n, g):
                        // row n, columns 4g..4g+3) and o needs no transpose
                        qs = mma_f16_k32(sf[p], fqc[p], qs);
                    }
                }
                if (I < 3) {
#pragma unroll
                    for (int p = 0; p < KT / 2; ++p) {
                        fwc[p] = fwn[p];
                        fqc[p] = fqn[p];
                    }
                }
                const f32x4 uu = f16x4_to_quad(u[I]) * exp2i(uex[I]);
                if constexpr (TR) {
                    vp[I] = ws * uS;
                    vp2[I] = uu + ws2 * uS2;
                } else {
                    vp[I] = uu + ws * uS;
                    acc_o[I] = qs * uS;
                }
            }

            // V' -> fp16 with its own per-wave scale
            u32x4 vf[2], vf2[2];
            const float uV = to_f16_scaled<4>(vp, vf);
            float uV2 = 0.f;
            if constexpr (TR) uV2 = to_f16_scaled<4>(vp2, vf2);
            const u32x4 vf0 = vf[0], vf1 = vf[1];
            // the previous chunk's rows, stored once this step's chain products
            // are issued.  The stores follow this step's A copies in issue
            // order, so the counted wait at the end of the step also waits for
            // the oldest A copies (harmless) and still covers U and region B.
            if constexpr (OUT && !GATE) {
                if (o_L > 0) flush_o(par ^ 1, o_t0, o_L);
            }

            if constexpr (OUT) {
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    // (A_qk V')^T = V'^T A_qk^T, row-major like O above
                    f32x4 a = mma_f16_k32(vf0, afr[aqk_frag(I, 0)], zero4());
                    if (I >= 2) a = mma_f16_k32(vf1, afr[aqk_frag(I, 1)], a);
                    acc_o[I] += a * uV;
                }
                if constexpr (GATE) {
                    // o stays fp32 up to the gate: staged as fp16 with a
                    // power-of-two exponent per wave, the single staging tile
                    // is rewritten only once every wave has flushed it
                    float m = 0.f;
#pragma unroll
                    for (int I = 0; I < 4; ++I)
#pragma unroll
                        for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(acc_o[I][j]));
                    const int e = scale_exp(wave_max_nonneg(m));
                    const float d = exp2i(-e);
                    barrier_lds();
#pragma unroll
                    for (int I = 0; I < 4; ++I)
                        *reinterpret_cast<u32x2 *>(obuf + (16 * I + ln) * OP + 16 * wave + 4 * lg) =
                            quad_to_f16(acc_o[I] * d);
                    if (lane == 0) oexp[wave] = e;
                } else {
                    uint16_t *ob = obuf + par * 64 * OP;
#pragma unroll
                    for (int I = 0; I < 4; ++I)
                        *reinterpret_cast<u32x2 *>(ob + (16 * I + ln) * OP + 16 * wave + 4 * lg) =
                            u32x2{f32x2_to_bf16x2(acc_o[I][0], acc_o[I][1]),
                                  f32x2_to_bf16x2(acc_o[I][2], acc_o[I][3])};
                }
            }
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const u32x4 k0 = kfr[t * 2], k1 = kfr[t * 2 + 1];
                const f32x4 g = gmr[t];
                f32x4 a = mma_f16_k32(k0, vf0, zero4());
                a = mma_f16_k32(k1, vf1, a);
                S[t] = decay_add(S[t], g, a, uV);
                if constexpr (TR) {
                    f32x4 a2 = mma_f16_k32(k0, vf2[0], zero4());
                    a2 = mma_f16_k32(k1, vf2[1], a2);
                    S2[t] = decay_add(S2[t], g, a2, uV2);
                }
            }
            o_t0 = t_first + kChunk * i;
            o_L = min(kChunk, t_end - o_t0);
            // everything but this step's A copies must have landed (memory
            // operations complete in issue order)
            if (c + 2 < c_end)
                __builtin_amdgcn_s_waitcnt((NA & 15) | (0x7 << 4) | (0xf << 8) | ((NA >> 4) << 14));
            else
                wait_all_memory();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int I = 0; I < 4; ++I) settle(un[I]);   // issued before every copy: landed
            if constexpr (GATE) {
#pragma unroll
                for (int k = 0; k < PPT; ++k) settle(gnext[k]);
            }
            barrier_lds();
#pragma unroll
            for (int I = 0; I < 4; ++I) u[I] = un[I];
            if constexpr (GATE) {
#pragma unroll
                for (int k = 0; k < PPT; ++k) gcur[k] = gnext[k];
            }
            slab_c = slab_n1;
            aslot = aslot == 2 ? 0 : aslot + 1;
        }
        if constexpr (GATE) {
            if (o_L > 0) flush_gate(o_t0, o_L);
        } else if constexpr (OUT) {
            if (o_L > 0) flush_o((c_end - c_begin - 1) & 1, o_t0, o_L);
            if (c_begin < c_end) checkpoint(c_end - 1);
        }
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
            if constexpr (OUT) {
                if (o_L > 0) store_o_tile<F32IO>(o, acc_o, o_t0, o_L, H, h, D, col, lg);
                if (c > c_begin) checkpoint(c - 1);
            }
            const int4 ent = table[c];
            f32x4 vp[4], vp2[TR ? 4 : 1];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                vp[I] = TR ? zero4() : u[I];
                if constexpr (TR) vp2[I] = u[I];
                acc_o[I] = zero4();
#pragma unroll
                for (int t = 0; t < KT; ++t) {
                    const f32x4 fw = __builtin_bit_cast(f32x4, frag(buf, SL::negW, I * KT + t));
                    vp[I] = mma_f32_k16(fw, S[t], vp[I]);
                    if constexpr (TR)
                        vp2[I] = mma_f32_k16(fw, S2[t], vp2[I]);
                    else
                        acc_o[I] =
                            mma_f32_k16(__builtin_bit_cast(f32x4, frag(buf, SL::qg, I * KT + t)), S[t], acc_o[I]);
                }
            }
            wait_all_memory();
            __syncthreads();
            if (c + 1 < c_end) copy_A(c + 1, buf);
            if constexpr (OUT) {
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int J = 0; J <= I; ++J)
                        acc_o[I] =
                            mma_f32_k16(__builtin_bit_cast(f32x4, frag(buf, SL::aqk, I * 4 + J)), vp[J], acc_o[I]);
            }
            const f32x4 *gam = gamma_of(buf);
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const f32x4 g = gam[4 * t + lg];
                S[t] = S[t] * g;
                if constexpr (TR) S2[t] = S2[t] * g;
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    const f32x4 fk = __builtin_bit_cast(f32x4, frag(buf, SL::kdT, t * 4 + J));
                    S[t] = mma_f32_k16(fk, vp[J], S[t]);
                    if constexpr (TR) S2[t] = mma_f32_k16(fk, vp2[J], S2[t]);
                }
            }
            o_t0 = ent.y;
            o_L = ent.z;
            wait_all_memory();
            __syncthreads();
#pragma unroll
            for (int I = 0; I < 4; ++I) u[I] = un[I];
        }
    }
    if constexpr (OUT) {
        if (F32IO && o_L > 0) store_o_tile<F32IO>(o, acc_o, o_t0, o_L, H, h, D, col, lg);
        if (F32IO && c_begin < c_end) checkpoint(c_end - 1);
        if (to_carry || (hT && (rec.w & kSegLast))) {
            float *dst = (to_carry ? carry : hT) + ((size_t)(n * H + h) * D + col) * D;
#pragma unroll
            for (int t = 0; t < KT; ++t) *reinterpret_cast<f32x4 *>(dst + 16 * t + 4 * lg) = S[t];
        }
    } else {
        // the transition matrix M (dk x dk), row-major: M[i][j] at i * D + j;
        // this lane holds M[16t + 4g + j][col]
        float *dst = trans + ((size_t)(sg * H + h) * 2) * D * D;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[(size_t)(16 * t + 4 * lg + j) * D + col] = S[t][j];
        // the offset S~, in the state layout [value column][key]
        float *dst2 = trans + (((size_t)(sg * H + h) * 2 + 1) * D + col) * D;
#pragma unroll
        for (int t = 0; t < KT; ++t) *reinterpret_cast<f32x4 *>(dst2 + 16 * t + 4 * lg) = S2[t];
    }
}

// ---------------------------------------------------------------------------
// Segment combine.  The per-chunk update S <- (Diag(gamma_C) - K~^T W) S + K~^T U
// is affine in S, so a segment maps its incoming state S_in to M S_in + S~
// (the cross-device merge of "Kimi K3：架构…" §9.3 and the KCP recurrence of
// the devpress K3 walk-through §8.1, Eq 17, applied here to segments on one device).  For a sequence in
// Pn > 1 segments: S_in(0) = h0 (or zero), S_in(k + 1) = M_k S_in(k) + S~_k,
// each written to the segment's slot of s_in.
//
// One workgroup per (sequence, head, 16 value columns); wave I owns rows
// [16 I, 16 I + 16) of the d_k x 16 slice.  The slice lives in LDS between
// steps (column-major, padded); each step is a 16 x 16 x d_k fp32 MFMA
// product per wave.  M_k and S~_k do not depend on the chain, so each
// step's rows are loaded two steps ahead.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(D * 4) combine_kernel(const float *__restrict__ h0, const int4 *__restrict__ segs,
                                                        int N, int H, int P, const float *__restrict__ trans,
                                                        float *__restrict__ s_in) {
    constexpr int KT = D / 16;
    constexpr int PITCH = D + 4;                 // floats per column in LDS
    __shared__ __attribute__((aligned(16))) float sS[16 * PITCH];
    const int vt = blockIdx.x % KT, unit = blockIdx.x / KT;
    if (unit >= N * H) return;
    const int n = unit / H, h = unit % H;
    const int tid = threadIdx.x;
    const int I = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int ln = lane & 15, lg = lane >> 4;
    const int col = 16 * vt + ln;
    const int row = 16 * I + 4 * lg;             // this lane's 4 accumulator rows (and S~ rows)
    float *slot = sS + ln * PITCH;               // column ln of the slice

    auto out_ptr = [&](int sg) { return s_in + ((size_t)(sg * H + h) * D + col) * D + row; };
    auto m_rows = [&](int sg) { return trans + (size_t)(sg * H + h) * 2 * D * D + (size_t)(16 * I + ln) * D + 4 * lg; };
    auto st_ptr = [&](int sg) { return trans + ((size_t)(sg * H + h) * 2 + 1) * D * D + (size_t)col * D + row; };

    // Operands of step k are loaded two steps ahead.  The first two steps'
    // loads go out together with h0 and the segment records (indices 0 and 1
    // are in bounds for every sequence: P >= 2 here).  Later fetches are
    // issued on every path, indices clamped to the last step, so that the
    // compiler can count the loads in flight and waits only for the ones a
    // step uses.
    f32x4 mA[KT], sA, mB[KT], sB;
    auto fetch = [&](int k, f32x4(&mm)[KT], f32x4 &ss) {
#pragma unroll
        for (int t = 0; t < KT; ++t) mm[t] = *reinterpret_cast<const f32x4 *>(m_rows(n * P + k) + 16 * t);
        ss = *reinterpret_cast<const f32x4 *>(st_ptr(n * P + k));
    };
    const f32x4 S0 = h0 ? *reinterpret_cast<const f32x4 *>(h0 + ((size_t)(n * H + h) * D + col) * D + row) : zero4();
    // steps = segments - 1 = index of the last segment (one record per lane, P <= 64)
    const unsigned long long lasts = __ballot(lane < P && (segs[n * P + lane].w & kSegLast));
    fetch(0, mA, sA);
    fetch(1, mB, sB);
    if (lasts == 0) return;
    const int steps = __builtin_ctzll(lasts);
    if (steps == 0) return;   // one segment: its pass reads h0 itself
    *reinterpret_cast<f32x4 *>(slot + row) = S0;
    *reinterpret_cast<f32x4 *>(out_ptr(n * P)) = S0;

    auto step = [&](int k, const f32x4(&mm)[KT], const f32x4 &ss) {
        f32x4 b[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) b[t] = *reinterpret_cast<const f32x4 *>(slot + 16 * t + 4 * lg);
        // two independent accumulation chains
        f32x4 acc0 = ss, acc1 = zero4();
#pragma unroll
        for (int t = 0; t < KT; t += 2) {
            acc0 = mma_f32_k16(mm[t], b[t], acc0);
            acc1 = mma_f32_k16(mm[t + 1], b[t + 1], acc1);
        }
        const f32x4 acc = acc0 + acc1;
        __syncthreads();                          // every wave has read S_in(k)
        *reinterpret_cast<f32x4 *>(slot + row) = acc;
        *reinterpret_cast<f32x4 *>(out_ptr(n * P + k + 1)) = acc;
        __syncthreads();
    };
    const int kl = steps - 1;
    __syncthreads();
    for (int k = 0; k < steps; k += 2) {
        step(k, mA, sA);
        fetch(min(k + 2, kl), mA, sA);
        if (k + 1 < steps) step(k + 1, mB, sB);
        fetch(min(k + 3, kl), mB, sB);
    }
}

// Segments per sequence when the caller leaves the choice to the library:
// a sequence is split only when the (sequence, head, column group)
// workgroups of one pass fill less than half the device, into as many
// segments as fill it once, each of at least 4 chunks.  A function of the
// sizes and the current device's compute-unit count only.
// Pipelined prefill, two cases.  When the chain's workgroups (N H of them per
// 64 value columns) leave at least 32 CUs to the intra kernel, and the
// sequences are long enough that every run keeps the chain busy for far
// longer than the per-run launch and delay costs (tens of microseconds): three
// runs for the plain call; six for the fused one, whose intra kernel pass
// (with the feature path) and chain (with the gate) are both longer, so
// shorter runs start the chain earlier.  When the chain fills the device
// several times over, runs still help where many long sequences finish at
// different times: the next run's intra kernel fills the CUs that the last
// chain workgroups (the longest sequences) leave idle.  Measured at H = 96,
// d = 128: 32 lognormal lengths averaging 128 chunks 20.2 -> 19.3 ms (fused
// 32.9 -> 29.3), 32 equal ones 20.1 -> 19.9; 8 sequences of 256 chunks or 16
// of 96 gained nothing (+0.2 to +2 %), so four runs from 16 sequences of 128
// chunks up.  Whether to pipeline does not depend on `fused`.
int choose_blocks(int N, int T, int H, int d, bool fused) {
    if (N <= 0 || T <= 0 || H <= 0) return 1;
    const long long chain_wgs = (long long)N * H * (d == 128 ? 2 : 1);
    const long long chunks_per_seq = (long long)T / kChunk / N;
    if (chain_wgs <= device_cus() - 32) return chunks_per_seq >= 192 ? (fused ? 6 : 3) : 1;
    return N >= 16 && chunks_per_seq >= 128 ? 4 : 1;
}

int choose_segments(int N, int T, int H, int d) {
    if (N <= 0 || T <= 0 || H <= 0) return 1;
    const long long blocks = (long long)N * H * (d == 128 ? 2 : 1);
    const int cus = device_cus();
    if (2 * blocks >= cus) return 1;
    const long long avg_chunks = (long long)T / kChunk / N;
    const long long p = std::min<long long>({(long long)kMaxSegments, cus / blocks, avg_chunks / 4});
    return p > 1 ? (int)p : 1;
}

// ---------------------------------------------------------------------------
// Block pipeline helpers.  Each host thread gets, per device, one helper
// stream (default priority, created on its first pipelined call and kept
// until the process ends) and the events that order it against the caller's
// stream; a thread's calls run one after another on the host, so they can
// reuse them.
constexpr int kMaxBlocks = 16;
constexpr int kPipeDelayTicks = 800;   // 8 us of the 100 MHz real-time clock

struct PipeStreams {
    hipStream_t s1 = nullptr;
    hipEvent_t ev[kMaxBlocks + 1] = {};
};

static PipeStreams *pipe_streams() {
    constexpr int kMaxDevices = 64;
    thread_local PipeStreams *per_device[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    if (!per_device[dev]) {
        PipeStreams *ps = new PipeStreams;
        if (hipStreamCreateWithFlags(&ps->s1, hipStreamNonBlocking) != hipSuccess) return nullptr;
        for (auto &e : ps->ev)
            if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
        per_device[dev] = ps;
    }
    return per_device[dev];
}

// A bounded pause on the caller's stream (one wave sleeping on the 100 MHz
// real-time clock), between the intra kernel of block j and that of block
// j + 1, so that block j's inter kernel, released by the same event, claims
// its CUs first.
__global__ void __launch_bounds__(64) pipeline_delay_kernel(int ticks) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < (unsigned long long)ticks) __builtin_amdgcn_s_sleep(8);
}

template <int D, bool F32IO>
static int launch_prefill_t(const PrefillArgs &a) {
    const PrefillPlan &p = a.plan;
    int32_t *meta = reinterpret_cast<int32_t *>(a.ws + p.off_meta);
    int4 *table = reinterpret_cast<int4 *>(a.ws + p.off_table);
    unsigned char *slabs = a.ws + p.off_slabs;

    int4 *segs = reinterpret_cast<int4 *>(a.ws + p.off_segs);
    int32_t *ck_off = reinterpret_cast<int32_t *>(a.ws + p.off_ckoff);
    // block pipeline: the intra kernel of chunk block j + 1 runs beside the
    // inter kernel of block j (bf16 path without segments or checkpoints; in
    // the fused call, each intra kernel after a feature pass that stages its
    // run's q, k, v, and the inter kernel in its gated output mode)
    const bool pipe = !F32IO && p.blocks > 1 && p.P == 1 && !a.ck && !a.ck_offsets && a.N > 0;
    int32_t *claims = reinterpret_cast<int32_t *>(a.ws + p.off_claims);
    float *carry = reinterpret_cast<float *>(a.ws + p.off_carry);
    const int ck_chunks = (a.ck || a.ck_offsets) ? a.ck_interval / kChunk : 0;
    const int ck_cap = ck_chunks ? a.T / a.ck_interval : 0;
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, a.stream, a.cu, a.N, a.T,
                       p.max_chunks, meta, table, reinterpret_cast<float *>(a.ws + p.off_null), D, p.P, segs,
                       ck_chunks, ck_cap, ck_off, a.ck_offsets, pipe ? claims : nullptr, pipe ? p.blocks : 0);
    if (hipGetLastError() != hipSuccess) return -1;

    if constexpr (!F32IO) {
        if (!pipe &&
            launch_intra_bf16<D>(a, meta, table, reinterpret_cast<const float *>(a.ws + p.off_null), slabs) != 0)
            return -1;
    } else {
        if (launch_intra_f32<D>(a, meta, table, slabs) != 0) return -1;
    }

    if constexpr (!F32IO) {
        // the fused call's new conv window: after the intra kernel has read
        // the old one (the two may be the same buffer); pipelined, after the
        // last run
        if (a.fused && !pipe && launch_conv_window(false, a.fused->xq, a.fused->xk, a.fused->xv, a.cu, a.N, a.T, a.H, D,
                                          a.fused->win_in, a.fused->win_out, a.stream) != 0)
            return -1;
    }
    if (a.N == 0) return 0;
    const int nseg = a.N * p.P;
    const int unit_blocks = (nseg * a.H + 7) / 8 * 8;
    float *trans = reinterpret_cast<float *>(a.ws + p.off_trans);
    float *s_in = reinterpret_cast<float *>(a.ws + p.off_sin);
    auto inter = [&](auto mode, hipStream_t st = nullptr, int blk_lo = 0, int blk_hi = 0,
                     float *blk_carry = nullptr) -> bool {
        constexpr int M = decltype(mode)::value;
        using SHP = InterShape<D, F32IO, M>;
        constexpr int groups = SHP::GROUPS;
        if (!set_lds(&inter_kernel<D, F32IO, M>, SHP::lds_bytes)) return false;
        const FusedIO *fx = M == kModeGate ? a.fused : nullptr;
        hipLaunchKernelGGL((inter_kernel<D, F32IO, M>), dim3(unit_blocks * groups), dim3(SHP::NT), SHP::lds_bytes,
                           blk_carry ? st : a.stream, a.h0, s_in, segs, table, nseg, a.H, p.max_chunks, slabs,
                           p.slab_bytes, a.o, a.hT, trans, groups, meta, ck_off, a.ck, ck_chunks,
                           fx ? static_cast<const uint16_t *>(fx->g) : nullptr, fx ? fx->w : nullptr,
                           fx ? fx->eps : 0.f, blk_lo, blk_hi, blk_carry);
        return hipGetLastError() == hipSuccess;
    };
    if constexpr (!F32IO) {
        if (pipe) {
            // Chunk blocks [j per, (j + 1) per): the intra kernel of block
            // j + 1 (on the caller's stream, after a short delay so that the
            // chain's workgroups take their CUs first) runs beside the inter
            // kernel of block j (on a helper stream); the state crosses block
            // boundaries through `carry`.  Events order the two streams; no
            // kernel waits on another.
            PipeStreams *ps = pipe_streams();
            if (!ps) return -1;
            const int B = p.blocks;
            // run boundaries: the last run a tenth of the table (its inter
            // kernel runs alone, with nothing left to overlap), the others
            // equal.  At the K3 shape: 5.13 ms with equal thirds, 5.06 with
            // a short last run.
            int bnd[kMaxBlocks + 1];
            {
                const int last = std::max(1, p.max_chunks / 10);
                const int rest = p.max_chunks - last;
                for (int j = 0; j < B; ++j) bnd[j] = (int)((long long)rest * j / (B - 1));
                bnd[B - 1] = rest;
                bnd[B] = p.max_chunks;
            }
            const float *null_row = reinterpret_cast<const float *>(a.ws + p.off_null);
            // The fused call runs its feature path as passes of its own here:
            // before the intra kernel of each run, the feature kernel stages
            // that run's q, k, v in the workspace, and the plain intra kernel
            // reads them; the new conv window is written after the last run.
            // Inside the intra kernel the feature math lengthens every item
            // of a kernel bound by latency, which costs more than the HBM
            // round trip of q, k, v it saves; o still never reaches memory.
            PrefillArgs ia = a;
            FeatureArgs fa;
            if (a.fused) {
                if (!p.staged) return -1;
                const size_t qkv = align256((size_t)a.T * a.H * D * 2);
                unsigned char *qs = a.ws + p.off_qkv;
                fa.f32io = false;
                fa.xq = a.fused->xq; fa.xk = a.fused->xk; fa.xv = a.fused->xv;
                fa.wq = a.fused->wq; fa.wk = a.fused->wk; fa.wv = a.fused->wv;
                fa.cu = a.cu; fa.N = a.N; fa.T = a.T; fa.H = a.H; fa.d = D;
                fa.win_in = a.fused->win_in; fa.win_out = nullptr;
                fa.q = qs; fa.k = qs + qkv; fa.v = qs + 2 * qkv;
                fa.stream = a.stream;
                fa.table = table;
                fa.nchunks = meta + a.N;
                ia.q = fa.q; ia.k = fa.k; ia.v = fa.v;
                ia.fused = nullptr;
            }
            auto intra_block = [&](int j) {
                if (a.fused) {
                    fa.c_lo = bnd[j];
                    fa.c_hi = bnd[j + 1];
                    if (launch_features(fa) != 0) return -1;
                }
                return launch_intra_bf16<D>(ia, meta, table, null_row, slabs, bnd[j] * a.H, bnd[j + 1] * a.H,
                                            claims + j);
            };
            if (intra_block(0) != 0 || hipEventRecord(ps->ev[0], a.stream) != hipSuccess) return -1;
            for (int j = 0; j < B; ++j) {
                if (hipStreamWaitEvent(ps->s1, ps->ev[j], 0) != hipSuccess) return -1;
                const int lo = bnd[j], hi = j == B - 1 ? INT_MAX : bnd[j + 1];
                if (!(a.fused ? inter(std::integral_constant<int, kModeGate>{}, ps->s1, lo, hi, carry)
                              : inter(std::integral_constant<int, kModeOutput>{}, ps->s1, lo, hi, carry)))
                    return -1;
                if (j + 1 < B) {
                    hipLaunchKernelGGL(pipeline_delay_kernel, dim3(1), dim3(64), 0, a.stream, kPipeDelayTicks);
                    if (hipGetLastError() != hipSuccess || intra_block(j + 1) != 0 ||
                        hipEventRecord(ps->ev[j + 1], a.stream) != hipSuccess)
                        return -1;
                }
            }
            // the fused call's new conv window, once every run's features
            // have read the old one (the two may be the same buffer)
            if (a.fused && launch_conv_window(false, a.fused->xq, a.fused->xk, a.fused->xv, a.cu, a.N, a.T, a.H, D,
                                              a.fused->win_in, a.fused->win_out, a.stream) != 0)
                return -1;
            if (hipEventRecord(ps->ev[kMaxBlocks], ps->s1) != hipSuccess ||
                hipStreamWaitEvent(a.stream, ps->ev[kMaxBlocks], 0) != hipSuccess)
                return -1;
            return 0;
        }
    }
    if (p.P > 1) {
        // the transition of every segment but a sequence's last, then the
        // incoming state of every segment
        if (!inter(std::integral_constant<int, kModeTrans>{})) return -1;
        hipLaunchKernelGGL((combine_kernel<D>), dim3(a.N * a.H * (D / 16)), dim3(D * 4), 0, a.stream, a.h0, segs,
                           a.N, a.H, p.P, trans, s_in);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    if constexpr (!F32IO) {
        if (a.fused) return inter(std::integral_constant<int, kModeGate>{}) ? 0 : -1;
    }
    if (!inter(std::integral_constant<int, kModeOutput>{})) return -1;
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
