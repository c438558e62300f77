// kda_intra_f32.hip -- intra-chunk kernel of the fp32 prefill path for gfx950.
//
// Same algebra as the bf16 path (kda_intra.hip; the chunk form of the
// s1mplewind "kimi-k3" notes, section "Chunkwise 形式", steps 1-6), computed
// with fp32 MFMA throughout so that the fp32 path meets its 1e-5 bar:
//   A_kk = StrictTril(Diag(beta)(Gamma*K)(K/Gamma)^T),  A_qk = Tril((Gamma*Q)(K/Gamma)^T)
//   T = (I + A_kk)^{-1},  M = T Diag(beta),  W = M (Gamma*K),  U = M V
// and the block-relative decays of the devpress K3 walk-through (§3.2, Eq 5):
// every factor is exp2 of a log-decay difference within or between 16-token
// blocks, so it is <= 1, or <= e^80 on a diagonal block.
//
// Persistent workgroups of 8 waves, one per CU (the fp32 operands need 146
// KiB of LDS).  In phase 1 wave w owns row block (w & 3) and key-channel half
// (w >> 2); lane (ln, lg) = (l % 16, l / 16) holds row 16 (w & 3) + ln and
// channels 16kt + 4lg + {0..3}.  The next item's raw inputs are fetched into
// registers while the current one is computed.
// ---------------------------------------------------------------------------
#include "kda_chunk.h"
#include "kda_device.h"
#include "kda_internal.h"

#include <algorithm>

namespace kda {

template <int D>
struct IntraF32Lds {
    static constexpr int P = D + 4;   // fp32 row pitch (floats)
    float kr[64][P];      // k_r exp2(Gl_r)
    float qr[64][P];      // q_r exp2(Gl_r)
    float ke[64][P];      // k_i exp2(bt_J - Gl_i); V after the Gram phase
    float a[64][68];      // A_kk, then T = (I + A_kk)^{-1} in place
    float beta[64];
    float bt[4][D];       // block log2-decay totals
    float pfx[4][D];      // exp2(sum_{m<I} bt_m)       chunk start -> start of block I
    float sfx[4][D];      // exp2(sum_{m>J} bt_m)       end of block J -> chunk end
    float dg[4][D];       // exp2(-bt_J)                undo one block: diagonal column factor
    float off[6][D];      // exp2(sum_{J<m<I} bt_m)     blocks strictly between J and I
};

constexpr int kF32Waves = 8;

// Raw inputs of one item for one lane: row block (wave & 3), channel half
// (wave >> 2).  Rows past the chunk's end load the chunk's first row; the
// consumer masks them.
template <int D>
struct IntraF32Regs {
    static constexpr int KH = D / 32;  // K16 tiles per channel half
    float beta;
    f32x4 z[KH], k[KH], q[KH], v[KH];
};

template <int D>
__device__ __forceinline__ void intra_f32_load(IntraF32Regs<D> &R, const float *q, const float *k, const float *v,
                                               const float *z, const float *beta, int4 ent, int h, int H, int lane,
                                               int wave) {
    constexpr int KH = D / 32;
    const int ln = lane & 15, lg = lane >> 4;
    const int row = 16 * (wave & 3) + ln;
    const size_t trow = (size_t)(ent.y + (row < ent.z ? row : 0)) * H + h;
    const size_t base = trow * D + (D / 2) * (wave >> 2) + 4 * lg;
    R.beta = beta[trow];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
        const size_t idx = base + 16 * kk;
        R.z[kk] = ld4(z + idx);
        R.k[kk] = ld4(k + idx);
        R.q[kk] = ld4(q + idx);
        R.v[kk] = ld4(v + idx);
    }
}

template <int D>
__global__ void __launch_bounds__(64 * kF32Waves) intra_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ z, const float *__restrict__ A, const float *__restrict__ beta,
    const int32_t *__restrict__ meta, const int4 *__restrict__ table, int N, int H, int max_chunks,
    unsigned char *__restrict__ slabs, size_t slab_stride) {
    using SL = Slab<D, true>;
    using LDS = IntraF32Lds<D>;
    constexpr int KT = D / 16, KH = D / 32;
    constexpr int NW = kF32Waves, NTH = 64 * NW;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    LDS &s = *reinterpret_cast<LDS *>(lds_raw);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index in an SGPR
    const int ln = lane & 15, lg = lane >> 4;
    const int blk = wave & 3, half = wave >> 2;   // phase-1 ownership: row block, channel half
    const int total = meta[N] * H;
    const int stride = gridDim.x;

    int it = blockIdx.x;
    if (it >= total) return;
    IntraF32Regs<D> R;
    int4 ent = table[it / H];
    intra_f32_load<D>(R, q, k, v, z, beta, ent, it % H, H, lane, wave);
    // Chunk-table entries and A_h are read through the scalar cache: fetch
    // them one item ahead of their use.
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
        f32x4 vreg[KH];
#pragma unroll
        for (int kk = 0; kk < KH; ++kk) {
            const int kt = half * KH + kk;
            const int c0 = 16 * kt + 4 * lg;
            const f32x4 kq = ok ? R.k[kk] : zero4();
            const f32x4 qq = ok ? R.q[kk] : zero4();
            vreg[kk] = ok ? R.v[kk] : zero4();
            f32x4 gl, bt, rf, kev;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gl[j] = row16_inclusive_scan(ok ? gate_log2(ea, R.z[kk][j]) : 0.f);
                bt[j] = row16_last(gl[j]);
                rf[j] = fast_exp2(gl[j]);
                kev[j] = kq[j] * fast_exp2(bt[j] - gl[j]);
            }
            *reinterpret_cast<f32x4 *>(&s.ke[row][c0]) = kev;
            if (ln == 15) *reinterpret_cast<f32x4 *>(&s.bt[blk][c0]) = bt;
            *reinterpret_cast<f32x4 *>(&s.kr[row][c0]) = kq * rf;
            *reinterpret_cast<f32x4 *>(&s.qr[row][c0]) = qq * rf;
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
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int c0 = 16 * kt + 4 * lg;
                const f32x4 kc = lds_quad(s.ke, 16 * J + ln, c0) * ld4(fac + c0);
                akk = mma_f32_k16(lds_quad(s.kr, 16 * I + ln, c0), kc, akk);
                aqt = mma_f32_k16(kc, lds_quad(s.qr, 16 * I + ln, c0), aqt);
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
            *reinterpret_cast<f32x4 *>(slab + SL::aqk + ((size_t)(I * 4 + J) * 64 + lane) * 16) = aq;
        });

        // Gamma*Q fragments (row tile I, key tile f) and the transposed,
        // end-of-chunk-decayed keys ((gamma_C/Gamma)*K)^T (key tile t, row tile J).
        for_wave_units<4 * SL::NKF, NW>(wave, [&](int fr) {
            const int I = fr / SL::NKF, f = fr % SL::NKF;
            const int c0 = 16 * f + 4 * lg;
            *reinterpret_cast<f32x4 *>(slab + SL::qg + ((size_t)fr * 64 + lane) * 16) =
                lds_quad(s.qr, 16 * I + ln, c0) * ld4(&s.pfx[I][c0]);
        });
        for_wave_units<KT * SL::NCF, NW>(wave, [&](int fr) {
            const int t = fr / SL::NCF, J = fr % SL::NCF;
            const int c = 16 * t + ln;
            *reinterpret_cast<f32x4 *>(slab + SL::kdT + ((size_t)fr * 64 + lane) * 16) =
                lds_col4(s.ke, 16 * J + 4 * lg, c) * s.sfx[J][c];
        });
        __syncthreads();

        // ---- phase 3: V into the freed ke array; the next item's inputs;
        // the diagonal 16x16 inverses, in place.
#pragma unroll
        for (int kk = 0; kk < KH; ++kk)
            *reinterpret_cast<f32x4 *>(&s.ke[row][16 * (half * KH + kk) + 4 * lg]) = vreg[kk];
        if (it_next < total) intra_f32_load<D>(R, q, k, v, z, beta, ent_next, it_next % H, H, lane, wave);
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

        // ---- phase 5: -W fragments (from W^T tiles) and U tiles, M = T Diag(beta).
        // W^T tile (t, I) = sum_J (Gamma*K)^T_{tJ} M^T_{JI}: the accumulator
        // lane (n = r, g) holds W[16I + r][16t + 4g + j], the A-operand
        // fragment of -W in the state-propagation product.
        for_wave_units<4 * SL::NKF, NW>(wave, [&](int unit) {
            const int I = unit / SL::NKF, t = unit % SL::NKF;
            f32x4 acc = zero4();
            for (int J = 0; J <= I; ++J) {
                const int cJ = 16 * J + 4 * lg;
                const f32x4 mq = lds_quad(s.a, 16 * I + ln, cJ) * ld4(&s.beta[cJ]);
                const f32x4 gk = lds_col4(s.kr, 16 * J + 4 * lg, 16 * t + ln) * s.pfx[J][16 * t + ln];
                acc = mma_f32_k16(gk, mq, acc);
            }
            *reinterpret_cast<f32x4 *>(slab + SL::negW + ((size_t)(I * SL::NKF + t) * 64 + lane) * 16) = -acc;
        });
        // U tile (I, w) = sum_J M_{IJ} V_{Jw}, in the accumulator layout the
        // state-propagation kernel starts V' from.
        for_wave_units<4 * KT, NW>(wave, [&](int unit) {
            const int I = unit / KT, w = unit % KT;
            f32x4 acc = zero4();
            for (int J = 0; J <= I; ++J) {
                const int cJ = 16 * J + 4 * lg;
                const f32x4 mq = lds_quad(s.a, 16 * I + ln, cJ) * ld4(&s.beta[cJ]);
                acc = mma_f32_k16(mq, lds_col4(s.ke, 16 * J + 4 * lg, 16 * w + ln), acc);
            }
            *reinterpret_cast<f32x4 *>(slab + SL::u + ((size_t)(I * KT + w) * 64 + lane) * 16) = acc;
        });
        ent = ent_next;
        ent_next = ent_after;
        a_cur = a_next;
        __syncthreads();
    }
}

template <int D>
int launch_intra_f32(const PrefillArgs &a, const int32_t *meta, const int4 *table, unsigned char *slabs) {
    const long long items = (long long)a.plan.max_chunks * a.H;
    if (items <= 0) return 0;
    const size_t lds = sizeof(IntraF32Lds<D>);
    if (!set_lds(&intra_f32_kernel<D>, lds)) return -1;
    const int grid = (int)std::min<long long>(items, (long long)device_cus());
    hipLaunchKernelGGL(intra_f32_kernel<D>, dim3(grid), dim3(64 * kF32Waves), lds, a.stream,
                       reinterpret_cast<const float *>(a.q), reinterpret_cast<const float *>(a.k),
                       reinterpret_cast<const float *>(a.v), a.z, a.A, a.beta, meta, table, a.N, a.H,
                       a.plan.max_chunks, slabs, a.plan.slab_bytes);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template int launch_intra_f32<32>(const PrefillArgs &, const int32_t *, const int4 *, unsigned char *);
template int launch_intra_f32<64>(const PrefillArgs &, const int32_t *, const int4 *, unsigned char *);
template int launch_intra_f32<128>(const PrefillArgs &, const int32_t *, const int4 *, unsigned char *);

}  // namespace kda
