// kda_features.hip -- the KDA feature path and output gate for gfx950.
//
// Feature path ("Kimi K3：架构、训练与推理系统研究" §3.2; devpress K3
// walk-through §3.1):  q = L2Norm(Swish(ShortConv(x_q))), k likewise,
// v = Swish(ShortConv(x_v)).  ShortConv is a causal depthwise convolution
// over the tokens of a sequence with 4 taps per channel (tap 3 on the current
// token); before a sequence's first token it reads the carried window, the
// last three pre-convolution tokens of the previous call ("Kimi K3：架构…"
// §3.4: the ShortConv state is a short window of projected tokens).
// Output gate ("Kimi K3：架构…" §3.3; devpress §3.3 Eq 6):
// y = Sigmoid(g) * RMSNorm(o), RMSNorm over a head's dv channels with a
// per-channel weight; g = W_g x is an input.
//
// All three kernels stream rows of [T][H][d]: one lane per 4 channels, the
// d/4 lanes of a (token, head) row inside one wavefront, so the L2 and RMS
// reductions are lane exchanges.
#include "kda_device.h"
#include "kda_internal.h"

#include <algorithm>

namespace kda {

constexpr int kTaps = 4;

// Four consecutive elements of an io-dtype array (8 or 16 bytes).
template <bool F32IO>
__device__ __forceinline__ void store_io4(void *p, size_t i, f32x4 x) {
    if constexpr (F32IO)
        *reinterpret_cast<f32x4 *>(static_cast<float *>(p) + i) = x;
    else
        *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p) + i) =
            u32x2{f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3])};
}

// Clamped bounds of sequence n, as the prefill reads them.
__device__ __forceinline__ void seq_bounds(const int32_t *cu, int n, int T, int &s, int &e) {
    s = min(max(cu[n], 0), T);
    e = min(max(cu[n + 1], 0), T);
}

// ShortConv -> Swish (-> L2Norm for q and k).  blockIdx.z: 0 = q, 1 = k, 2 = v;
// blockIdx.y: a span of 1024 channels of the [H][d] row (256 / (d / 4)
// heads); blockIdx.x: a range of TR tokens (tile0 plus a reordering of
// blockIdx.x, below).  The block
// first copies rows t0 - 3 .. t0 + TR - 1 of its span into LDS (direct
// global -> LDS copies, 16 bytes per lane), then every thread walks its 4
// channels through the range, reading the four taps of each token from LDS.
// Only taps before a sequence's first token read the carried window instead.
// With a chunk table (the pipelined fused prefill), only the tokens of chunks
// [c_lo, c_hi) are written: from the first token of chunk c_lo to that of
// chunk c_hi (the end when c_hi is past the last chunk, nchunks[0] of them).
template <int D, bool F32IO, int TR>
__global__ void __launch_bounds__(256) shortconv_kernel(
    const void *__restrict__ xq, const void *__restrict__ xk, const void *__restrict__ xv,
    const float *__restrict__ wq, const float *__restrict__ wk, const float *__restrict__ wv,
    const int32_t *__restrict__ cu, int N, int T, int H, const void *__restrict__ win,
    void *__restrict__ q, void *__restrict__ k, void *__restrict__ v, int tile0, const int4 *__restrict__ table,
    const int32_t *__restrict__ nchunks, int c_lo, int c_hi) {
    constexpr int G = D / 4;                     // lanes per row
    constexpr int SPAN = 1024;                   // channels per block: 256 lanes x 4
    constexpr int EB = F32IO ? 4 : 2;            // bytes per element
    constexpr int P = kTaps - 1;                 // earlier taps
    constexpr int ROWS = TR + P;
    constexpr int PPR = SPAN * EB / 16;          // 16-byte pieces per staged row
    __shared__ __attribute__((aligned(16))) unsigned char tile[ROWS * SPAN * EB];

    const int which = blockIdx.z;
    const void *x = which == 0 ? xq : which == 1 ? xk : xv;
    const float *w = which == 0 ? wq : which == 1 ? wk : wv;
    void *out = which == 0 ? q : which == 1 ? k : v;
    const int CW = 3 * D;                        // window channels per head: q | k | v
    const size_t rowc = (size_t)H * D;           // channels per token row
    const int ch0 = blockIdx.y * SPAN;           // first channel of the span
    // Workgroups are dealt to the eight XCDs in turn (their L2 caches are
    // separate), so launch index x takes token tile (x % 8) * per + x / 8:
    // each XCD walks a contiguous range of tiles in order, and the three
    // rows before a tile are the previous tile's last rows, just read into
    // the same L2.  The last gridDim.x % 8 workgroups keep their own tiles.
    int tx = (int)blockIdx.x;
    {
        const int per = (int)gridDim.x / 8;
        if (tx < 8 * per) tx = (tx % 8) * per + tx / 8;
    }
    const int t0 = (tile0 + tx) * TR, t1 = min(t0 + TR, T);
    // the tokens this launch writes (every thread reads the same entries)
    int w_lo = 0, w_hi = T;
    if (table) {
        const int nc = nchunks[0];
        w_lo = c_lo < nc ? table[c_lo].y : T;
        w_hi = c_hi < nc ? table[c_hi].y : T;
    }
    if (t0 >= t1 || t1 <= w_lo || t0 >= w_hi) return;   // uniform: before any barrier

    // stage rows t0 - 3 .. t1 - 1 of channels [ch0, ch0 + SPAN): direct
    // global -> LDS copies of 16 bytes per lane, zeros outside the tensor
    // (the copy writes lane l's 16 bytes at the wave's LDS base + 16 l: the
    // base is passed wave-uniform, so lanes that skip the copy shift nothing)
    const unsigned char *xb = static_cast<const unsigned char *>(x);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    // the copies issue ahead of the other workgroups' arithmetic on the CU
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int i0 = 0; i0 < ROWS * PPR; i0 += 256) {
        const int i = i0 + threadIdx.x;
        unsigned char *wave_base = tile + (size_t)(i0 + 64 * wave) * 16;
        if (i < ROWS * PPR) {
            const int r = i / PPR, pc = i % PPR;
            const int pos = t0 - P + r;
            const size_t ch = (size_t)ch0 + (size_t)pc * 16 / EB;
            if (pos >= 0 && pos < t1 && ch < rowc)
                __builtin_amdgcn_global_load_lds(xb + ((size_t)pos * rowc + ch) * EB,
                                                 (__attribute__((address_space(3))) void *)wave_base, 16, 0, 0);
            else
                *reinterpret_cast<u32x4 *>(tile + (size_t)i * 16) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int hl = threadIdx.x / G, c0 = 4 * (threadIdx.x % G);
    const int h = ch0 / D + hl;
    if (h >= H) return;                          // whole row groups only; no barrier follows
    const f32x4 *wt = reinterpret_cast<const f32x4 *>(w + ((size_t)h * D + c0) * kTaps);
    const f32x4 wj[4] = {wt[0], wt[1], wt[2], wt[3]};   // channel c0 + j: taps wj[j][0..3]
    auto staged = [&](int r) -> f32x4 {          // this thread's 4 channels of staged row r
        const unsigned char *p = tile + ((size_t)r * SPAN + hl * D + c0) * EB;
        if constexpr (F32IO) {
            return *reinterpret_cast<const f32x4 *>(p);
        } else {
            const u32x2 b = *reinterpret_cast<const u32x2 *>(p);
            return f32x4{bf16_lo_half(b[0]), bf16_hi_half(b[0]), bf16_lo_half(b[1]), bf16_hi_half(b[1])};
        }
    };
    // the sequence holding t0: the last n with cu[n] <= t0
    int n = 0, hi = N - 1;
    while (n < hi) {
        const int mid = (n + hi + 1) >> 1;
        if (min(max(cu[mid], 0), T) <= t0) n = mid; else hi = mid - 1;
    }
    int s, e;
    seq_bounds(cu, n, T, s, e);
    auto finish = [&](int t, const f32x4 (&tap)[kTaps]) {
        f32x4 f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float u = 0.f;
#pragma unroll
            for (int i = 0; i < kTaps; ++i) u += wj[c][i] * tap[i][c];
            f[c] = swish(u);
        }
        if (which < 2) {
            float ss = f[0] * f[0] + f[1] * f[1] + f[2] * f[2] + f[3] * f[3];
            ss = lane_group_sum<G>(ss);
            f = f * fast_rsq(ss);
        }
        store_io4<F32IO>(out, ((size_t)t * H + h) * D + c0, f);
    };
    const bool whole = t0 >= w_lo && t1 <= w_hi;
    if (whole && t1 - t0 == TR && s <= t0 - P && t1 <= e) {
        // the whole range and the three rows before it in one sequence
#pragma unroll
        for (int j = 0; j < TR; ++j) {
            f32x4 tap[kTaps];
#pragma unroll
            for (int i = 0; i < kTaps; ++i) tap[i] = staged(j + i);
            finish(t0 + j, tap);
        }
        return;
    }
    for (int t = max(t0, w_lo); t < min(t1, w_hi); ++t) {
        while (t >= e && n < N - 1) {
            ++n;
            seq_bounds(cu, n, T, s, e);
        }
        f32x4 tap[kTaps];
#pragma unroll
        for (int i = 0; i < kTaps; ++i) {
            const int pos = t - P + i;
            const int wi = pos - s + P;
            if (pos >= s)
                tap[i] = staged(t - t0 + i);
            else
                tap[i] = (win && wi >= 0)
                             ? load_io4<F32IO>(win, ((size_t)(n * P + wi) * H + h) * CW + which * D + c0)
                             : zero4();
        }
        finish(t, tap);
    }
}

// The carried window after the call: the last three tokens of [window, sequence]
// for every (sequence, head, channel).  Each thread reads its three values
// before writing them, so win_out may be win_in.
template <bool F32IO>
__global__ void __launch_bounds__(256) conv_window_kernel(const void *__restrict__ xq, const void *__restrict__ xk,
                                                          const void *__restrict__ xv, const int32_t *__restrict__ cu,
                                                          int N, int T, int H, int D, const void *win_in,
                                                          void *win_out) {
    const int CW = 3 * D, groups = CW / 4;
    const long long items = (long long)N * H * groups;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < items; i += (long long)gridDim.x * 256) {
        const int g = (int)(i % groups);
        const int h = (int)((i / groups) % H);
        const int n = (int)(i / ((long long)groups * H));
        const int ch = 4 * g, which = ch / D, c0 = ch % D;
        const void *x = which == 0 ? xq : which == 1 ? xk : xv;
        int s, e;
        seq_bounds(cu, n, T, s, e);
        if (e < s) e = s;
        f32x4 val[kTaps - 1];
#pragma unroll
        for (int j = 0; j < kTaps - 1; ++j) {
            const int pos = e - (kTaps - 1) + j;
            if (pos >= s)
                val[j] = load_io4<F32IO>(x, ((size_t)pos * H + h) * D + c0);
            else if (win_in)
                val[j] = load_io4<F32IO>(win_in, ((size_t)(n * (kTaps - 1) + pos - s + kTaps - 1) * H + h) * CW + ch);
            else
                val[j] = zero4();
        }
#pragma unroll
        for (int j = 0; j < kTaps - 1; ++j) {
            store_io4<F32IO>(win_out, ((size_t)(n * (kTaps - 1) + j) * H + h) * CW + ch, val[j]);
        }
    }
}

// y = Sigmoid(g) * o / sqrt(mean(o^2) + eps) * w, per (token, head) row of D.
// y may be o or g: a thread reads its elements before writing them.  Each
// thread takes RPT rows per pass, all loads first.
template <int D, bool F32IO, int RPT>
__global__ void __launch_bounds__(256) output_gate_kernel(const void *o, const void *g, const float *__restrict__ w,
                                                          float eps, long long rows, void *y) {
    constexpr int G = D / 4;
    constexpr int RPB = 256 / G;
    const int c0 = 4 * (threadIdx.x % G);
    const f32x4 wv = *reinterpret_cast<const f32x4 *>(w + c0);
    for (long long base = (long long)blockIdx.x * RPB * RPT; base < rows; base += (long long)gridDim.x * RPB * RPT) {
        f32x4 ov[RPT], gv[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const long long r = base + m * RPB + threadIdx.x / G;
            if (r < rows) {
                ov[m] = load_io4<F32IO>(o, (size_t)r * D + c0);
                gv[m] = load_io4<F32IO>(g, (size_t)r * D + c0);
            }
        }
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const long long r = base + m * RPB + threadIdx.x / G;
            if (r >= rows) break;                // uniform over a row's lanes
            float ss = ov[m][0] * ov[m][0] + ov[m][1] * ov[m][1] + ov[m][2] * ov[m][2] + ov[m][3] * ov[m][3];
            ss = lane_group_sum<G>(ss);
            const float inv = fast_rsq(ss * (1.f / D) + eps);
            f32x4 out;
#pragma unroll
            for (int j = 0; j < 4; ++j) out[j] = ov[m][j] * inv * wv[j] * fast_rcp(1.f + __expf(-gv[m][j]));
            store_io4<F32IO>(y, (size_t)r * D + c0, out);
        }
    }
}

// Blocks for a grid-stride launch over `rows` rows: enough to fill the device
// several times, never more than the rows need.
static unsigned stride_blocks(long long rows, int rows_per_block) {
    const long long need = (rows + rows_per_block - 1) / rows_per_block;
    const long long cap = 256LL * 32;
    return (unsigned)std::max(1LL, std::min(need, cap));
}

template <int D, bool F32IO>
static int launch_features_t(const FeatureArgs &a) {
    // tokens per tile: TR + 3 staged rows of 1024 channels, 32 KiB in bf16
    // (five workgroups per CU) and 44 KiB in fp32
    constexpr int TR = F32IO ? 8 : 13;
    if (a.T > 0) {
        // token tiles: all, or (chunk run) those that can hold its tokens.
        // Chunk c starts at token 64 (c - N) at the earliest (every chunk but
        // a sequence's last is full) and at 64 c at the latest.
        long long lo = 0, hi = a.T;
        if (a.table) {
            lo = std::max(0LL, 64LL * ((long long)a.c_lo - a.N));
            hi = std::min((long long)a.T, 64LL * a.c_hi);
        }
        const long long tile0 = lo / TR, tiles = hi > lo ? (hi + TR - 1) / TR - tile0 : 0;
        if (tiles > 0) {
            const dim3 grid((unsigned)tiles, (unsigned)(((long long)a.H * D + 1023) / 1024), 3);
            hipLaunchKernelGGL((shortconv_kernel<D, F32IO, TR>), grid, dim3(256), 0, a.stream, a.xq, a.xk, a.xv,
                               a.wq, a.wk, a.wv, a.cu, a.N, a.T, a.H, a.win_in, a.q, a.k, a.v, (int)tile0, a.table,
                               a.nchunks, a.c_lo, a.c_hi);
            if (hipGetLastError() != hipSuccess) return -1;
        }
    }
    if (a.table) return 0;                // the caller writes the window after the last run
    if (a.win_out && a.N > 0) {
        const long long items = (long long)a.N * a.H * (3 * D / 4);
        hipLaunchKernelGGL((conv_window_kernel<F32IO>), dim3(stride_blocks(items, 256)), dim3(256), 0, a.stream, a.xq,
                           a.xk, a.xv, a.cu, a.N, a.T, a.H, D, a.win_in, a.win_out);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

int launch_conv_window(bool f32io, const void *xq, const void *xk, const void *xv, const int32_t *cu, int N, int T,
                       int H, int d, const void *win_in, void *win_out, hipStream_t stream) {
    if (!win_out || N <= 0) return 0;
    const long long items = (long long)N * H * (3 * d / 4);
    if (f32io)
        hipLaunchKernelGGL((conv_window_kernel<true>), dim3(stride_blocks(items, 256)), dim3(256), 0, stream, xq, xk,
                           xv, cu, N, T, H, d, win_in, win_out);
    else
        hipLaunchKernelGGL((conv_window_kernel<false>), dim3(stride_blocks(items, 256)), dim3(256), 0, stream, xq, xk,
                           xv, cu, N, T, H, d, win_in, win_out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_features(const FeatureArgs &a) {
    switch (a.d) {
        case 32: return a.f32io ? launch_features_t<32, true>(a) : launch_features_t<32, false>(a);
        case 64: return a.f32io ? launch_features_t<64, true>(a) : launch_features_t<64, false>(a);
        case 128: return a.f32io ? launch_features_t<128, true>(a) : launch_features_t<128, false>(a);
    }
    return -1;
}

template <int D, bool F32IO>
static int launch_gate_t(const GateArgs &a) {
    constexpr int RPB = 256 / (D / 4), RPT = 4;
    const long long rows = (long long)a.T * a.H;
    if (rows == 0) return 0;
    hipLaunchKernelGGL((output_gate_kernel<D, F32IO, RPT>), dim3(stride_blocks(rows, RPB * RPT)), dim3(256), 0,
                       a.stream, a.o, a.g, a.w, a.eps, rows, a.y);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_output_gate(const GateArgs &a) {
    switch (a.dv) {
        case 32: return a.f32io ? launch_gate_t<32, true>(a) : launch_gate_t<32, false>(a);
        case 64: return a.f32io ? launch_gate_t<64, true>(a) : launch_gate_t<64, false>(a);
        case 128: return a.f32io ? launch_gate_t<128, true>(a) : launch_gate_t<128, false>(a);
    }
    return -1;
}

}  // namespace kda
