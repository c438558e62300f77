// kda_intra.hip -- intra-chunk kernel of the bf16 prefill path for gfx950.
//
// One 4-wave workgroup per (chunk, head) item, persistent over items, two
// workgroups per CU (77 KiB of LDS each at d = 128), so that one workgroup's
// memory traffic, barriers and serial steps overlap the other's math.  Per
// item it computes, in the chunk form of the s1mplewind "kimi-k3" notes
// (section "Chunkwise 形式", steps 1-6):
//   A_kk = StrictTril(Diag(beta)(Gamma*K)(K/Gamma)^T),  A_qk = Tril((Gamma*Q)(K/Gamma)^T)
//   T = (I + A_kk)^{-1},  M = T Diag(beta),  W = M (Gamma*K),  U = M V
// and writes the slab the inter-chunk kernel consumes (kda_chunk.h): -W,
// Gamma*Q, ((gamma_C/Gamma)*K)^T, A_qk, gamma_C and U.
//
// Decays use the block-relative form of the devpress K3 walk-through (§3.2,
// Eq 5): within a 16-token block the gate sums to at least -80, so every
// factor below is exp2 of a log-decay difference that is <= 0, or <= 80 ln 2
// ... on a diagonal block.
//
// Ownership: wave w holds row block b = (w + rot) & 3 (rot varies by item so
// that the unequal per-block work spreads over the SIMDs); lane (ln, lg) =
// (l % 16, l / 16) holds row 16b + ln and channels 16kt + 4lg + {0..3} of
// every K16 tile kt.  That is the MFMA row-operand layout, so the block's
// keys and queries feed the Gram products straight from registers:
//   tile (I, b), I >= b, of A_kk is  kr_I (A, rows r) x ke_b fac (B, rows i)
//   and of A_qk^T is                 ke_b fac (A, rows i) x qr_I (B, rows r),
// with kr = k exp2(Gl), qr = q exp2(Gl) (Gl: log-decay from the block start,
// inclusive) and ke = k exp2(bt - Gl) (bt: the block's total log-decay); fac
// is exp2(-bt_b) on the diagonal tile and the decay of the blocks strictly
// between b and I otherwise.  Only kr and qr of blocks 1..3 go through LDS.
// Diagonal tiles, where fac reaches e^80, and the U product are split-bf16
// (hi + lo, good to about 2^-16); off-diagonal Gram tiles have every factor
// <= 1 and use fp16 operands (one MFMA), and so does W = M (Gamma*K), whose
// result is stored in fp16 anyway: rounding M and Gamma*K (<= 1) to fp16
// first leaves the chain's error where the final rounding puts it.
//
// Phases (barriers between them):
//   1  gate, block-local cumulative log-decay (DPP row scan), kr / qr / ke
//   F  per-channel decay factors of the chunk
//   2  Gamma*Q, K~^T (transposed by an identity MFMA), Gram tiles -> A_kk, A_qk
//   3  Gamma*K (fp16) and V tiles into LDS; inverses of the four
//      diagonal 16x16 blocks (forward substitution)
//   4  off-diagonal blocks of T, one block column per wave (fp32 MFMA)
//   4b M = T Diag(beta): split bf16 fragments (for U) and fp16 ones (for W)
//   5  -W and U, stored in the slab
// ---------------------------------------------------------------------------
#include "kda_chunk.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Transpose of a 16x16 tile held in the row-operand layout (lane (m, g) holds
// X[m][4g + j]), rounded to fp16: as the A operand of a 16x16x16 fp16 MFMA
// against the identity it gives D = X, whose accumulator lane (n, g) holds
// X[4g + j][n] -- four consecutive rows of column n.  Exact for finite values.
__device__ __forceinline__ u32x2 transpose_tile_f16(f32x4 x, int lane) {
    const int n = lane & 15, g = lane >> 4;
    const u32x2 a = quad_to_f16(x);
    const uint32_t one = 0x3c00u;  // fp16 1.0
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = (4 * g + j == n) ? one : 0u;
    const u32x2 b = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b),
                                                          zero4(), 0, 0, 0);
    return quad_to_f16(d);
}

// Row-major 16x16 tiles of 16-bit values in LDS (512 bytes: 16 rows of 16
// channels), written straight from the row layout.  ds_read_b64_tr_b16 with
// lane l reading the tile's bytes [8 l, 8 l + 8) returns to lane (n, g) rows
// 4g .. 4g+3 of column n: the tile's transpose in the MFMA operand layout.
__device__ __forceinline__ u32x2 tile_tr(const unsigned char *tile, int lane) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) s16x4 *)(tile + lane * 8)));
}
// K32 operand over row blocks 2f and 2f + 1 of channel tile t, tiles indexed
// [t][row block] from `base`.
__device__ __forceinline__ u32x4 tile_tr_k32(const unsigned char *base, int t, int f, int lane) {
    const u32x2 a = tile_tr(base + (size_t)(t * 4 + 2 * f) * 512, lane);
    const u32x2 c = tile_tr(base + (size_t)(t * 4 + 2 * f + 1) * 512, lane);
    return u32x4{a[0], a[1], c[0], c[1]};
}

// A zero the compiler cannot see through.  Lane-dependent constants built
// from `lane + opaque_zero()` inside the item loop are rebuilt per item
// instead of being hoisted out of the loop and kept live (or spilled) across it.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

template <int D>
struct Intra4Lds {
    static constexpr int KT = D / 16, NP = D / 32;
    static constexpr size_t FR = 1024;
    // X, phases 1-2: fp16 row fragments of kr and qr of row blocks 1..3,
    //   [block - 1][kr, qr][pair p], read by the off-diagonal Gram tiles.
    // X, phases 3-5: Gamma*K (fp16) and V as row-major 16x16 tiles
    //   [channel tile t][row block], read back transposed (tile_tr); from
    //   phase 4b, the fp16 M fragments [aqk_frag(I, pj)] at M16.
    static constexpr size_t X = 0;
    static constexpr size_t XB = 12 * NP * FR;
    static constexpr size_t GKT = X, VT = X + 4 * KT * FR;
    // the six fp16 M fragments: between Gamma*K and V where they fit (d >= 64),
    // else after everything else
    static constexpr bool M16_IN_X = GKT + KT * 2048 + 6 * FR <= VT;
    // A_kk, then T: the diagonal blocks in place, T_IJ (I > J) at block (J, I).
    static constexpr int AP = 68;
    static constexpr size_t A = X + XB;
    // F, phases 1-3: block log-decay totals bt [4][D], then 18 factor rows
    //   [18][D]: exp2(-bt_J) (0..3), prefix decays pfx_I (4..7), suffix
    //   decays sfx_J (8..11), decays strictly between J < I (12 + off_index).
    // F, phases 4b-5: M split fragments [aqk_frag(I, pj)][hi, lo].
    static constexpr size_t F = A + 64 * AP * 4;
    static constexpr size_t FB = 12 * FR;
    static constexpr size_t BETA = F + FB;
    static constexpr size_t CLAIM = BETA + 64 * 4;          // [4] int: claimed items
    static constexpr size_t M16 = M16_IN_X ? GKT + KT * 2048 : CLAIM + 16;
    static constexpr size_t bytes = M16_IN_X ? CLAIM + 16 : M16 + 6 * FR;
    static_assert((4 + 18) * D * 4 <= (int)FB, "bt and the factors fit the M region");
};

// Raw inputs of the lane's row for one item.
template <int D>
struct Rows4 {
    static constexpr int KT = D / 16;
    float beta;
    f32x4 z[KT];
    u32x2 k[KT], q[KT], v[KT];
};

// Rows past the chunk's end read the null row instead (z = -inf, so the gate
// is 0 and nothing decays; k = q = v = 0; beta = 0), which makes every later
// step correct for them without masks.  Loads are unconditional.
template <int D>
__device__ __forceinline__ void row_sources(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *z,
                                            const float *null_row, int4 ent, int h, int H, int row,
                                            const float *&zr, const uint16_t *&kr, const uint16_t *&qr,
                                            const uint16_t *&vr, size_t &trow, bool &ok) {
    ok = row < ent.z;
    trow = (size_t)(ent.y + row) * H + h;
    const uint16_t *nz16 = reinterpret_cast<const uint16_t *>(null_row + D);
    zr = ok ? z + trow * D : null_row;
    kr = ok ? k + trow * D : nz16;
    qr = ok ? q + trow * D : nz16;
    vr = ok ? v + trow * D : nz16;
}
// z and beta: fetched one item ahead (the gate needs them first)
template <int D>
__device__ __forceinline__ void load_rows4_z(Rows4<D> &R, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                             const float *z, const float *beta, const float *null_row, int4 ent,
                                             int h, int H, int row, int lg) {
    constexpr int KT = D / 16;
    const float *zr; const uint16_t *kr, *qr, *vr; size_t trow; bool ok;
    row_sources<D>(q, k, v, z, null_row, ent, h, H, row, zr, kr, qr, vr, trow, ok);
    R.beta = ok ? beta[trow] : null_row[2 * D];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) R.z[kt] = ld4(zr + 16 * kt + 4 * lg);
}
// k, q: loaded at the start of the item, in flight while the gate runs
template <int D>
__device__ __forceinline__ void load_rows4_kq(Rows4<D> &R, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                               const float *z, const float *null_row, int4 ent, int h, int H,
                                               int row, int lg) {
    constexpr int KT = D / 16;
    const float *zr; const uint16_t *kr, *qr, *vr; size_t trow; bool ok;
    row_sources<D>(q, k, v, z, null_row, ent, h, H, row, zr, kr, qr, vr, trow, ok);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        const int c = 16 * kt + 4 * lg;
        R.k[kt] = *reinterpret_cast<const u32x2 *>(kr + c);
        R.q[kt] = *reinterpret_cast<const u32x2 *>(qr + c);
    }
}
// v: loaded when the Gram phase has released its registers
template <int D>
__device__ __forceinline__ void load_rows4_v(Rows4<D> &R, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                             const float *z, const float *null_row, int4 ent, int h, int H, int row,
                                             int lg) {
    constexpr int KT = D / 16;
    const float *zr; const uint16_t *kr, *qr, *vr; size_t trow; bool ok;
    row_sources<D>(q, k, v, z, null_row, ent, h, H, row, zr, kr, qr, vr, trow, ok);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) R.v[kt] = *reinterpret_cast<const u32x2 *>(vr + 16 * kt + 4 * lg);
}

// The q / k / v feature path of the fused prefill, in place of a row load:
// ShortConv(4) -> Swish (-> L2Norm over the row's D channels when NORM),
// rounded to bf16 and packed exactly like a loaded row, so that every later
// step is the unfused kernel's (the unfused pipeline hands q, k, v over in
// bf16 as well).  out[kt] = channels 16 kt + 4 lg .. + 3 of row 16 b + ln of
// the chunk.  Taps on the three earlier tokens come from the lanes of the
// same 16-lane row by DPP shifts; the block's first three rows take them from
// the three rows before the block, which lanes 0..2 load: from x inside the
// sequence, or, at a sequence's first chunk (ent.w set), from the carried
// window (zeros without one).  Rows past the chunk's end give zeros, like
// the null row of the unfused kernel.  Tap order, Swish and the L2 norm's
// hardware reciprocal square root follow the feature kernel.
// The row SFT tokens before lane ln's: lane ln - SFT of the same 16-lane row
// (row_shr), or for ln < SFT the pre-block row ln - SFT + 3, held by lane
// ln + 3 - SFT (row_shl).
template <int SFT>
__device__ __forceinline__ u32x2 earlier_tap(u32x2 own, u32x2 pre, int ln) {
    u32x2 r;
#pragma unroll
    for (int wd = 0; wd < 2; ++wd) {
        const uint32_t from_row = __builtin_amdgcn_update_dpp(0, own[wd], 0x110 + SFT, 0xf, 0xf, true);
        const uint32_t from_pre =
            SFT == 3 ? pre[wd] : __builtin_amdgcn_update_dpp(0, pre[wd], 0x100 + (3 - SFT), 0xf, 0xf, true);
        r[wd] = ln >= SFT ? from_row : from_pre;
    }
    return r;
}

template <int D, bool NORM>
__device__ __forceinline__ void feature_row(u32x2 (&out)[D / 16], const uint16_t *x, const float *w,
                                            const uint16_t *win, int which, int4 ent, int h, int H, int b, int ln,
                                            int lg) {
    constexpr int KT = D / 16;
    const int row = 16 * b + ln;
    const bool ok = row < ent.z;
    const bool live = 16 * b < ent.z;                     // the block has rows
    const uint16_t *xr = x + ((size_t)(ent.y + (ok ? row : 0)) * H + h) * D + 4 * lg;
    const uint16_t *pr = nullptr;
    if (live && ln < 3) {
        if (b > 0 || ent.w == 0)
            pr = x + ((size_t)(ent.y + 16 * b - 3 + ln) * H + h) * D + 4 * lg;
        else if (win)
            pr = win + ((size_t)(ent.x * 3 + ln) * H + h) * (3 * D) + which * D + 4 * lg;
    }
    u32x2 own[KT], pre[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        own[kt] = live ? *reinterpret_cast<const u32x2 *>(xr + 16 * kt) : u32x2{0u, 0u};
        pre[kt] = pr ? *reinterpret_cast<const u32x2 *>(pr + 16 * kt) : u32x2{0u, 0u};
    }
    // taps of channel 4 lg + j of tile kt: f32x4 index 16 kt + j from wr
    const f32x4 *wr = reinterpret_cast<const f32x4 *>(w + ((size_t)h * D + 4 * lg) * 4);
    auto pack = [&](f32x4 y) -> u32x2 {
        return ok ? u32x2{f32x2_to_bf16x2(y[0], y[1]), f32x2_to_bf16x2(y[2], y[3])} : u32x2{0u, 0u};
    };
    f32x4 f[NORM ? KT : 1];
    float ss = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        u32x2 tap[4];                                     // tap i meets token t - 3 + i
        tap[3] = own[kt];
        tap[2] = earlier_tap<1>(own[kt], pre[kt], ln);
        tap[1] = earlier_tap<2>(own[kt], pre[kt], ln);
        tap[0] = earlier_tap<3>(own[kt], pre[kt], ln);
        f32x4 tv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) tv[i] = quad_f32<false>(tap[i]);
        f32x4 fk;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x4 wj = wr[16 * kt + c];
            float u = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) u += wj[i] * tv[i][c];
            fk[c] = swish(u);
        }
        if constexpr (NORM) {
            f[kt] = fk;
            ss += fk[0] * fk[0] + fk[1] * fk[1] + fk[2] * fk[2] + fk[3] * fk[3];
        } else {
            out[kt] = pack(fk);                           // no norm: each tile is final
        }
    }
    if constexpr (NORM) {
        ss += __shfl_xor(ss, 16, 64);                     // the row's other channel groups (lg)
        ss += __shfl_xor(ss, 32, 64);
        const float inv = fast_rsq(ss);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) out[kt] = pack(f[kt] * inv);
    }
}

template <int D, bool FEAT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) intra4_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ z, const float *__restrict__ A, const float *__restrict__ beta,
    const int32_t *__restrict__ meta, const int4 *__restrict__ table, const float *__restrict__ null_row, int N,
    int H, int max_chunks, unsigned char *__restrict__ slabs, size_t slab_stride, FusedIO fx, int item_lo,
    int item_hi, int *__restrict__ claims) {
    using SL = Slab<D, false>;
    using LY = Intra4Lds<D>;
    constexpr int KT = D / 16, NP = D / 32;
    constexpr size_t FR = LY::FR;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    unsigned char *X = lds_raw + LY::X;
    float (*a)[LY::AP] = reinterpret_cast<float (*)[LY::AP]>(lds_raw + LY::A);
    float *Fp = reinterpret_cast<float *>(lds_raw + LY::F);
    float *bt_lds = Fp;                 // [4][D]
    float *fac_lds = Fp + 4 * D;        // [18][D]
    unsigned char *msp = lds_raw + LY::F;
    float *sbeta = reinterpret_cast<float *>(lds_raw + LY::BETA);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index in an SGPR
    const int stride = gridDim.x;
    // block rotation: differs between neighbouring workgroups and advances per item
    const int rot0 = blockIdx.x + 2 * (2 * (int)blockIdx.x >= (int)gridDim.x);

    // Items [lo, hi): the whole table, each workgroup taking every stride-th
    // item; or, with `claims`, one block of a pipelined prefill whose items
    // the workgroups claim from a counter, so that workgroups that start late
    // (their CUs busy with the previous block's chain) take fewer.  A
    // workgroup keeps two claims ahead of its current item; tid 0 claims and
    // publishes through LDS, read by every wave after a barrier.
    const int total = meta[N] * H;
    const int lo = claims ? item_lo : 0;
    const int hi = claims ? min(item_hi, total) : total;
    int *claim_lds = reinterpret_cast<int *>(lds_raw + LY::CLAIM);
    int it, it_nx;
    if (claims) {
        if (tid == 0) {
            claim_lds[1] = lo + atomicAdd(claims, 1);
            claim_lds[2] = lo + atomicAdd(claims, 1);
        }
        __syncthreads();
        it = __builtin_amdgcn_readfirstlane(claim_lds[1]);
        it_nx = __builtin_amdgcn_readfirstlane(claim_lds[2]);
    } else {
        it = lo + (int)blockIdx.x;
        it_nx = it + stride;
    }
    if (it >= hi) return;
    // Chunk-table entries and A_h are read through the scalar cache, whose
    // loads every barrier waits for: fetch them one item ahead of their use.
    int4 ent = table[it / H];
    int4 ent_next = it_nx < hi ? table[it_nx / H] : make_int4(0, 0, 0, 0);
    float a_cur = A[it % H];
    // Raw inputs of the current item; the next item's are fetched during the
    // solve (phase 4), when few registers are live.
    Rows4<D> R;
    load_rows4_z<D>(R, q, k, v, z, beta, null_row, ent, it % H, H, 16 * ((wave + rot0) & 3) + (threadIdx.x & 15),
                    (threadIdx.x >> 4) & 3);
    __builtin_amdgcn_s_waitcnt(0);

    for (int iter = 0; it < hi; ++iter) {
        const int chunk = it / H, h = it % H;
        const int b = (wave + rot0 + iter) & 3;        // this wave's row block
        // lane coordinates, rebuilt per item (see opaque_zero)
        const int lane = (tid & 63) + opaque_zero();
        const int ln = lane & 15, lg = lane >> 4;
        const int row = 16 * b + ln;
        unsigned char *slab = slabs + ((size_t)h * max_chunks + chunk) * slab_stride;
        const float nel = -__expf(a_cur) * kLog2e;       // the gate's exp2 argument per unit z
        const int it_next = it_nx;
        int it_after = it_next + stride;
        int4 ent_after = make_int4(0, 0, 0, 0);
        if (claims) {
            if (tid == 0) claim_lds[0] = lo + atomicAdd(claims, 1);   // read after the first barrier
        } else if (it_after < hi) {
            ent_after = table[it_after / H];
        }
        const float a_next = it_next < hi ? A[it_next % H] : 0.f;

        // ---- phase 1: gate, block-local cumulative log2-decay, row operands
        if constexpr (FEAT) {
            feature_row<D, true>(R.k, static_cast<const uint16_t *>(fx.xk), fx.wk,
                                 static_cast<const uint16_t *>(fx.win_in), 1, ent, h, H, b, ln, lg);
            feature_row<D, true>(R.q, static_cast<const uint16_t *>(fx.xq), fx.wq,
                                 static_cast<const uint16_t *>(fx.win_in), 0, ent, h, H, b, ln, lg);
        } else {
            // the item's row loads issue ahead of the other workgroup's work,
            // so their latency starts early (likewise the next item's gate
            // inputs in phase 4)
            __builtin_amdgcn_s_setprio(3);
            load_rows4_kq<D>(R, q, k, v, z, null_row, ent, h, H, row, lg);
            __builtin_amdgcn_s_setprio(0);
        }
        if (lg == 0) sbeta[row] = R.beta;
        f32x4 kr[KT], qr[KT], ke[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const f32x4 kq = quad_f32<false>(R.k[kt]);
            const f32x4 qq = quad_f32<false>(R.q[kt]);
            f32x4 gl, bt, rf, kev;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gl[j] = row16_inclusive_scan(gate_log2_nel(nel, R.z[kt][j]));
                bt[j] = row16_last(gl[j]);
                rf[j] = fast_exp2(gl[j]);
                kev[j] = kq[j] * fast_exp2(bt[j] - gl[j]);
            }
            kr[kt] = kq * rf;
            qr[kt] = qq * rf;
            ke[kt] = kev;
            if (ln == 15) *reinterpret_cast<f32x4 *>(bt_lds + b * D + 16 * kt + 4 * lg) = bt;
        }
        if (b > 0) {   // other blocks read these for their off-diagonal tiles (fp16)
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                *reinterpret_cast<u32x4 *>(X + ((size_t)((b - 1) * 2 + 0) * NP + p) * FR + lane * 16) =
                    quads_to_f16(kr[2 * p], kr[2 * p + 1]);
                *reinterpret_cast<u32x4 *>(X + ((size_t)((b - 1) * 2 + 1) * NP + p) * FR + lane * 16) =
                    quads_to_f16(qr[2 * p], qr[2 * p + 1]);
            }
        }
        __syncthreads();
        if (claims) {
            it_after = __builtin_amdgcn_readfirstlane(claim_lds[0]);
            if (it_after < hi) ent_after = table[it_after / H];
        }

        // ---- per-channel decay factors
        for (int c = tid; c < D; c += 256) {
            const float b0 = bt_lds[c], b1 = bt_lds[D + c], b2 = bt_lds[2 * D + c], b3 = bt_lds[3 * D + c];
            float *f = fac_lds + c;
            f[0 * D] = fast_exp2(-b0);
            f[1 * D] = fast_exp2(-b1);
            f[2 * D] = fast_exp2(-b2);
            f[3 * D] = fast_exp2(-b3);
            f[4 * D] = 1.f;
            f[5 * D] = fast_exp2(b0);
            f[6 * D] = fast_exp2(b0 + b1);
            f[7 * D] = fast_exp2(b0 + b1 + b2);
            f[8 * D] = fast_exp2(b1 + b2 + b3);
            f[9 * D] = fast_exp2(b2 + b3);
            f[10 * D] = fast_exp2(b3);
            f[11 * D] = 1.f;
            f[12 * D] = 1.f;             // (0,1)
            f[13 * D] = fast_exp2(b1);       // (0,2)
            f[14 * D] = fast_exp2(b1 + b2);  // (0,3)
            f[15 * D] = 1.f;             // (1,2)
            f[16 * D] = fast_exp2(b2);       // (1,3)
            f[17 * D] = 1.f;             // (2,3)
            reinterpret_cast<float *>(slab + SL::gamma)[c] = fast_exp2(b0 + b1 + b2 + b3);
        }
        __syncthreads();

        // ---- phase 2: Gamma*Q, K~^T, Gram tiles (I, b) for I >= b
        // Wave b owns 4 - b Gram tiles, so the waves reach the barrier after
        // this phase at different times while the other workgroup on the CU
        // competes for issue.  A wave priority that follows the tile count
        // (kept through the diagonal solve behind the barrier) lets the
        // longest chain issue first.
        if (b == 0) __builtin_amdgcn_s_setprio(3);
        else if (b == 1) __builtin_amdgcn_s_setprio(2);
        else if (b == 2) __builtin_amdgcn_s_setprio(1);
        {
            const float *pfx = fac_lds + (4 + b) * D;
            const float *sfx = fac_lds + (8 + b) * D;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int c0 = 32 * p + 4 * lg, c1 = c0 + 16;
                store_f16(slab + SL::qg + ((size_t)(b * NP + p) * 64 + lane) * 16, qr[2 * p] * ld4(pfx + c0),
                          qr[2 * p + 1] * ld4(pfx + c1));
            }
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const u32x2 kd = transpose_tile_f16(ke[t] * ld4(sfx + 16 * t + 4 * lg), lane);
                *reinterpret_cast<u32x2 *>(slab + SL::kdT + ((size_t)(t * SL::NCF + (b >> 1)) * 64 + lane) * 16 +
                                           (b & 1) * 8) = kd;
            }
        }
        for (int I = b; I < 4; ++I) {
            const float *fac = fac_lds + (I == b ? b : 12 + off_index(b, I)) * D;
            f32x4 akk = zero4(), aqt = zero4();
            if (I == b) {
                // diagonal tile: the wave's own rows; fac = exp2(-bt_b) reaches
                // e^80, beyond fp16, so split-bf16 operands
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const int c0 = 32 * p + 4 * lg, c1 = c0 + 16;
                    u32x4 kch, kcl, krh, krl, qrh, qrl;
                    quads_to_bf16_split(ke[2 * p] * ld4(fac + c0), ke[2 * p + 1] * ld4(fac + c1), kch, kcl);
                    quads_to_bf16_split(kr[2 * p], kr[2 * p + 1], krh, krl);
                    quads_to_bf16_split(qr[2 * p], qr[2 * p + 1], qrh, qrl);
                    akk = mma3_bf16(krh, krl, kch, kcl, akk);
                    aqt = mma3_bf16(kch, kcl, qrh, qrl, aqt);
                }
            } else {
                // off-diagonal tile: every factor is a decay <= 1 and |k|, |q| <= 1,
                // so fp16 operands (11-bit mantissas) in range
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const int c0 = 32 * p + 4 * lg, c1 = c0 + 16;
                    const u32x4 kc = quads_to_f16(ke[2 * p] * ld4(fac + c0), ke[2 * p + 1] * ld4(fac + c1));
                    const u32x4 kx = *reinterpret_cast<const u32x4 *>(X + ((size_t)((I - 1) * 2 + 0) * NP + p) * FR +
                                                                      lane * 16);
                    const u32x4 qx = *reinterpret_cast<const u32x4 *>(X + ((size_t)((I - 1) * 2 + 1) * NP + p) * FR +
                                                                      lane * 16);
                    akk = mma_f16_k32(kx, kc, akk);
                    aqt = mma_f16_k32(kc, qx, aqt);
                }
            }
            // A_kk tile: lane (n = i, g) holds the sum for rows r = 4g + j of block I
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rl = 4 * lg + j;
                float x = akk[j] * sbeta[16 * I + rl];
                if (I == b && ln >= rl) x = 0.f;
                a[16 * I + rl][16 * b + ln] = x;
            }
            // A_qk: lane (n = r, g) holds columns i = 4g + j of row r -- the
            // operand fragment of row tile I, column block b
            f32x4 aq;
#pragma unroll
            for (int j = 0; j < 4; ++j) aq[j] = (I == b && 4 * lg + j > ln) ? 0.f : aqt[j];
            unsigned char *base = slab + SL::aqk + ((size_t)aqk_frag(I, b >> 1) * 64 + lane) * 16 + (b & 1) * 8;
            *reinterpret_cast<u32x2 *>(base) = quad_to_f16(aq);
            if (I == b && (b & 1) == 0)  // the tile right of an even diagonal shares its fragment
                *reinterpret_cast<u32x2 *>(base + 8) = u32x2{0u, 0u};
        }
        __syncthreads();

        // ---- phase 3: Gamma*K (fp16) and V into X as row-major tiles
        if constexpr (!FEAT) load_rows4_v<D>(R, q, k, v, z, null_row, ent, h, H, row, lg);
        {
            const float *pfx = fac_lds + (4 + b) * D;
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const f32x4 gk = kr[t] * ld4(pfx + 16 * t + 4 * lg);   // Gamma*K <= 1
                const size_t tb = (size_t)(t * 4 + b) * 512 + ln * 32 + lg * 8;   // row ln, channels 4lg..
                *reinterpret_cast<u32x2 *>(X + LY::GKT + tb) = quad_to_f16(gk);
            }
        }
        if (lane < 16) {
            // column `lane` of (I + A_bb)^{-1}: forward substitution, updating
            // every later row as soon as an entry is final
            const int o = 16 * b;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == lane) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < 15; ++i) {
                const float ci = x[i];
#pragma unroll
                for (int r = i + 1; r < 16; ++r) x[r] -= a[o + r][o + i] * ci;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) a[o + r][o + lane] = x[r];
        }
        __builtin_amdgcn_s_setprio(0);
        // V last: its loads, issued at the top of the phase, complete behind
        // the Gamma*K split and the diagonal solve instead of stalling them
        if constexpr (FEAT)
            feature_row<D, false>(R.v, static_cast<const uint16_t *>(fx.xv), fx.wv,
                                  static_cast<const uint16_t *>(fx.win_in), 2, ent, h, H, b, ln, lg);
#pragma unroll
        for (int t = 0; t < KT; ++t)
            *reinterpret_cast<u32x2 *>(X + LY::VT + (size_t)(t * 4 + b) * 512 + ln * 32 + lg * 8) = R.v[t];
        __syncthreads();

        // the gate inputs of the next item
        __builtin_amdgcn_s_setprio(3);
        if (it_next < hi)
            load_rows4_z<D>(R, q, k, v, z, beta, null_row, ent_next, it_next % H, H,
                            16 * ((wave + rot0 + iter + 1) & 3) + ln, lg);
        __builtin_amdgcn_s_setprio(0);
        // ---- phase 4: T_IJ = -T_II sum_{J<=m<I} A_Im T_mJ, stored at block (J, I).
        // Block column J needs only A, the diagonal inverses and its own
        // earlier blocks, so wave J computes the whole column in order with
        // no barrier in between, keeping each block in registers (an
        // accumulator is the B operand of the next product).
        if (wave < 3) {
            const int J = wave;
            f32x4 tc[4];
#pragma unroll
            for (int I = 1; I < 4; ++I) {
                if (I > J) {
                    f32x4 x = mma_f32_k16(lds_quad(a, 16 * I + ln, 16 * J + 4 * lg),
                                          lds_col4(a, 16 * J + 4 * lg, 16 * J + ln), zero4());
#pragma unroll
                    for (int m = 1; m < I; ++m)
                        if (m > J) x = mma_f32_k16(lds_quad(a, 16 * I + ln, 16 * m + 4 * lg), tc[m], x);
                    tc[I] = -mma_f32_k16(lds_quad(a, 16 * I + ln, 16 * I + 4 * lg), x, zero4());
#pragma unroll
                    for (int j = 0; j < 4; ++j) a[16 * J + 4 * lg + j][16 * I + ln] = tc[I][j];
                }
            }
        }
        __syncthreads();

        // ---- phase 4b: M = T Diag(beta) for the rows of block b, split, and in fp16
#pragma unroll
        for (int pj = 0; pj < 2; ++pj) {
            if (2 * pj <= b) {
                f32x4 x[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int J = 2 * pj + s;
                    const f32x4 tq = J < b ? lds_quad(a, 16 * J + ln, 16 * b + 4 * lg)
                                           : (J == b ? lds_quad(a, 16 * b + ln, 16 * b + 4 * lg) : zero4());
                    x[s] = tq * ld4(sbeta + 16 * J + 4 * lg);
                }
                u32x4 hi, lo;
                quads_to_bf16_split(x[0], x[1], hi, lo);
                unsigned char *d = msp + (size_t)aqk_frag(b, pj) * 2 * FR + lane * 16;
                *reinterpret_cast<u32x4 *>(d) = hi;
                *reinterpret_cast<u32x4 *>(d + FR) = lo;
                *reinterpret_cast<u32x4 *>(X + LY::M16 + (size_t)aqk_frag(b, pj) * FR + lane * 16) =
                    quads_to_f16(x[0], x[1]);
            }
        }
        __syncthreads();

        // ---- phase 5: -W (from W^T tiles) and U
        // Raised priority: this phase's MFMA chains and slab stores end the
        // item, and issuing them ahead of the other workgroup's work hands
        // the item over sooner.
        __builtin_amdgcn_s_setprio(1);
        for_wave_units<4 * NP, 4>(wave, [&](int unit) {
            const int p = unit % NP, I = unit / NP;
            f32x4 acc0 = zero4(), acc1 = zero4();
            for (int pj = 0; pj <= (I >> 1); ++pj) {
                const u32x4 m16 =
                    *reinterpret_cast<const u32x4 *>(X + LY::M16 + (size_t)aqk_frag(I, pj) * FR + lane * 16);
                acc0 = mma_f16_k32(tile_tr_k32(X + LY::GKT, 2 * p, pj, lane), m16, acc0);
                acc1 = mma_f16_k32(tile_tr_k32(X + LY::GKT, 2 * p + 1, pj, lane), m16, acc1);
            }
            store_f16(slab + SL::negW + ((size_t)(I * NP + p) * 64 + lane) * 16, -acc0, -acc1);
        });
        {
            // U tiles of this wave, then one power-of-two exponent for all of them
            constexpr int NU = (4 * KT + 3) / 4;
            f32x4 uacc[NU];
            float m = 0.f;
#pragma unroll
            for (int r = 0; r < NU; ++r) {
                const int unit = wave + 4 * r;
                const int w = unit % KT, I = unit / KT;
                f32x4 acc = zero4();
                if ((4 * KT) % 4 == 0 || unit < 4 * KT) {
                    for (int pj = 0; pj <= (I >> 1); ++pj) {
                        const unsigned char *mb = msp + (size_t)aqk_frag(I, pj) * 2 * FR + lane * 16;
                        const u32x4 vb = tile_tr_k32(X + LY::VT, w, pj, lane);
                        acc = mma_bf16_k32(*reinterpret_cast<const u32x4 *>(mb), vb, acc);
                        acc = mma_bf16_k32(*reinterpret_cast<const u32x4 *>(mb + FR), vb, acc);
                    }
                }
                uacc[r] = acc;
#pragma unroll
                for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(acc[j]));
            }
            const int e = scale_exp(wave_max_nonneg(m));
            const float sc = exp2i(-e);
#pragma unroll
            for (int r = 0; r < NU; ++r) {
                const int unit = wave + 4 * r;
                const int w = unit % KT, I = unit / KT;
                *reinterpret_cast<u32x2 *>(slab + SL::u + ((size_t)(I * KT + w) * 64 + lane) * 8) =
                    quad_to_f16(uacc[r] * sc);
                if (lane == 0) reinterpret_cast<int *>(slab + SL::uexp)[I * KT + w] = e;
            }
        }
        __builtin_amdgcn_s_setprio(0);
        it = it_next;
        it_nx = it_after;
        ent = ent_next;
        ent_next = ent_after;
        a_cur = a_next;
        __syncthreads();
    }
}

template <int D>
int launch_intra_bf16(const PrefillArgs &a, const int32_t *meta, const int4 *table, const float *null_row,
                      unsigned char *slabs, int item_lo, int item_hi, int *claims) {
    using LY = Intra4Lds<D>;
    const long long items = claims ? (long long)item_hi - item_lo : (long long)a.plan.max_chunks * a.H;
    if (items <= 0) return 0;
    const int grid = (int)std::min<long long>(items, 2LL * device_cus());
    auto launch = [&](auto kernel, const FusedIO &fx) -> int {
        if (!set_lds(kernel, LY::bytes)) return -1;
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), LY::bytes, a.stream, reinterpret_cast<const uint16_t *>(a.q),
                           reinterpret_cast<const uint16_t *>(a.k), reinterpret_cast<const uint16_t *>(a.v), a.z, a.A,
                           a.beta, meta, table, null_row, a.N, a.H, a.plan.max_chunks, slabs, a.plan.slab_bytes, fx,
                           item_lo, item_hi, claims);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    };
    if (a.fused) return launch(intra4_kernel<D, true>, *a.fused);
    return launch(intra4_kernel<D, false>, FusedIO{});
}

template int launch_intra_bf16<32>(const PrefillArgs &, const int32_t *, const int4 *, const float *,
                                     unsigned char *, int, int, int *);
template int launch_intra_bf16<64>(const PrefillArgs &, const int32_t *, const int4 *, const float *,
                                     unsigned char *, int, int, int *);
template int launch_intra_bf16<128>(const PrefillArgs &, const int32_t *, const int4 *, const float *,
                                     unsigned char *, int, int, int *);

}  // namespace kda
