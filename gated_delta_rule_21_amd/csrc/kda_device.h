// kda_device.h -- device-side helpers shared by the gfx950 KDA kernels:
// bf16 conversion and splitting, the bounded gate, and 16x16 MFMA tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Chunk length of the chunkwise prefill and the MFMA tile edge.
constexpr int kChunk = 64;
constexpr int kTile = 16;

// log2(e) and g_min * log2(e): the kernels keep log-decays in base 2 so that
// every exponential is a single v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kGminLog2e = -5.0f * 1.4426950408889634f;

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  fp32 -> bf16 uses the hardware packed convert
// (v_cvt_pk_bf16_f32, round to nearest even).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf16_lo_half(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_half(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }


// Load element i of an io-dtype array as fp32.
template <bool F32IO>
__device__ __forceinline__ float load_io(const void *p, size_t i) {
    if constexpr (F32IO) {
        return reinterpret_cast<const float *>(p)[i];
    } else {
        return bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
    }
}
// Elements i .. i + 3 (i a multiple of 4) of an io-dtype array as fp32.
template <bool F32IO>
__device__ __forceinline__ f32x4 load_io4(const void *p, size_t i) {
    if constexpr (F32IO) {
        return *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(p) + i);
    } else {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(p) + i);
        return f32x4{bf16_lo_half(w[0]), bf16_hi_half(w[0]), bf16_lo_half(w[1]), bf16_hi_half(w[1])};
    }
}
template <bool F32IO>
__device__ __forceinline__ void store_io(void *p, size_t i, float x) {
    if constexpr (F32IO) {
        reinterpret_cast<float *>(p)[i] = x;
    } else {
        reinterpret_cast<__bf16 *>(p)[i] = (__bf16)x;
    }
}

// ---------------------------------------------------------------------------
// Bounded gate in base 2: g * log2(e) with g = -5 sigmoid(exp(A_h) z)
// (devpress K3 walk-through §3.2, Eq 5; "Kimi K3：架构…" §3.2).
// `ea` is exp(A_h).  sigmoid saturates to exactly 0 or 1 at the ends, so the
// result spans [-5 log2 e, 0].
// ---------------------------------------------------------------------------
// The same with nel = -exp(A_h) log2(e) precomputed once per head.
__device__ __forceinline__ float gate_log2_nel(float nel, float z) {
    return kGminLog2e * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * nel));
}
__device__ __forceinline__ float gate_log2(float ea, float z) {
    float x = ea * z;
    float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
    return kGminLog2e * s;
}

// Swish and the norms of the feature path and the output gate use the
// hardware reciprocal and reciprocal square root (about 1 ulp) instead of
// IEEE division: their outputs are rounded to the io dtype, and a correctly
// rounded division costs about ten instructions.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsq(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float swish(float u) { return u * fast_rcp(1.f + __expf(-u)); }

// 2^x on the transcendental unit (v_exp_f32).  Results below 2^-126 may
// flush to zero; every use here is a decay factor whose true value is then
// negligible.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// 16x16 MFMA tiles.  Fragment convention used by every kernel here:
//   A operand (16 x K16):  lane (m, g) = (l % 16, l / 16) holds A[m][4g + j], j = 0..3
//   B operand (K16 x 16):  lane (n, g) holds B[4g + j][n]
//   accumulator (16x16):   lane (n, g) holds D[4g + j][n]
// so an accumulator is directly a B operand of the next product.  Two K16
// tiles are fused into one 16x16x32 bf16 MFMA by concatenating the lanes'
// quads (A and B use the same slot for the same k, which is all the
// instruction needs).  fp32 operands use four 16x16x4 MFMAs per K16 tile.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma_bf16_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32_k16(f32x4 a, f32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

// Two fp32 quads (K16 tiles t0, t1) -> one bf16 K32 fragment, rounded (hi)
// or split into hi and lo parts.
__device__ __forceinline__ u32x4 quads_to_bf16(f32x4 x0, f32x4 x1) {
    return u32x4{f32x2_to_bf16x2(x0[0], x0[1]), f32x2_to_bf16x2(x0[2], x0[3]),
                 f32x2_to_bf16x2(x1[0], x1[1]), f32x2_to_bf16x2(x1[2], x1[3])};
}
// The fp32 values of a packed bf16 fragment (slot order).
__device__ __forceinline__ void bf16_to_quads(u32x4 w, f32x4 &x0, f32x4 &x1) {
    x0 = f32x4{bf16_lo_half(w[0]), bf16_hi_half(w[0]), bf16_lo_half(w[1]), bf16_hi_half(w[1])};
    x1 = f32x4{bf16_lo_half(w[2]), bf16_hi_half(w[2]), bf16_lo_half(w[3]), bf16_hi_half(w[3])};
}
__device__ __forceinline__ void quads_to_bf16_split(f32x4 x0, f32x4 x1, u32x4 &hi, u32x4 &lo) {
    hi = quads_to_bf16(x0, x1);
    f32x4 h0, h1;
    bf16_to_quads(hi, h0, h1);
    lo = quads_to_bf16(x0 - h0, x1 - h1);
}

// ---------------------------------------------------------------------------
// fp16 operands of the serial state chain (v_cvt_pk_f16_f32, round to
// nearest even; v_mfma_f32_16x16x32_f16).
// ---------------------------------------------------------------------------
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f32x2_to_f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
__device__ __forceinline__ u32x4 quads_to_f16(f32x4 x0, f32x4 x1) {
    return u32x4{f32x2_to_f16x2(x0[0], x0[1]), f32x2_to_f16x2(x0[2], x0[3]),
                 f32x2_to_f16x2(x1[0], x1[1]), f32x2_to_f16x2(x1[2], x1[3])};
}
__device__ __forceinline__ u32x2 quad_to_f16(f32x4 x) {
    return u32x2{f32x2_to_f16x2(x[0], x[1]), f32x2_to_f16x2(x[2], x[3])};
}
// fp32 values of four packed fp16 (exact).
__device__ __forceinline__ f32x4 f16x4_to_quad(u32x2 w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x4, w), f32x4);
}
__device__ __forceinline__ f32x4 mma_f16_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Power-of-two scaling for fp16 operands: scale_for(m) = 2^-e with e chosen
// so that m * 2^-e lies in [2^11, 2^12) (m > 0), i.e. well inside the fp16
// range whatever the magnitude of the data.  Multiplying by a power of two
// is exact, so scaling and unscaling change no bits of the mantissas.
__device__ __forceinline__ int scale_exp(float m) {
    const int be = (int)((__float_as_uint(m) >> 23) & 0xffu);   // biased exponent of m
    int e = be - 127 - 11;
    e = be == 0 ? 0 : e;
    return min(max(e, -100), 100);
}
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// DPP lane movement inside 16-lane rows: row_shr:n (0x110 + n) shifts in
// from lower lanes with zero fill; row_newbcast:n (0x150 + n) broadcasts lane
// n of every row to that row.
#define KDA_DPP(x, ctrl) \
    __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), (ctrl), 0xf, 0xf, true))

// Maximum over the 64 lanes of a wavefront of values x >= 0: a DPP max-scan
// inside each 16-lane row, then the four row maxima through readlane.  The
// result is wave-uniform.  Non-negative floats order like their bit patterns,
// so the scan runs on the integers: one DPP-fused integer max per step, with
// no NaN quieting around it, and the last three maxima in scalar registers.
__device__ __forceinline__ float wave_max_nonneg(float x) {
    uint32_t u = __float_as_uint(x);
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x111, 0xf, 0xf, true));
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x112, 0xf, 0xf, true));
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x114, 0xf, 0xf, true));
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x118, 0xf, 0xf, true));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)u, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)u, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)u, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)u, 63);
    return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// Sum over each aligned group of W consecutive lanes (W a power of two up
// to 64), every lane of the group receiving it: a butterfly over the lane
// index bits, low bit first.  Inside a 16-lane row the partners are reached
// by DPP moves, with no trip through the LDS unit: the quad permutations
// [1,0,3,2] and [2,3,0,1], then the half-row mirror and the row mirror,
// whose partners hold the same values as lane ^ 4 and lane ^ 8 once each
// quad, then each half-row, is uniform.  The result equals that of the
// shuffle butterfly bit for bit (each step adds the same two values).
template <int W>
__device__ __forceinline__ float lane_group_sum(float x) {
    static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "lane group");
    x += KDA_DPP(x, 0xb1);
    if constexpr (W >= 4) x += KDA_DPP(x, 0x4e);
    if constexpr (W >= 8) x += KDA_DPP(x, 0x141);
    if constexpr (W >= 16) x += KDA_DPP(x, 0x140);
    if constexpr (W >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (W >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

// Lane 15 of each 16-lane row, broadcast to the row.
__device__ __forceinline__ float row16_last(float x) { return KDA_DPP(x, 0x15f); }

// acc + (ah + al)(bh + bl) without the lo*lo term: a product of two
// split operands, good to about 2^-16 relative per term.
__device__ __forceinline__ f32x4 mma3_bf16(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c) {
    c = mma_bf16_k32(ah, bh, c);
    c = mma_bf16_k32(ah, bl, c);
    return mma_bf16_k32(al, bh, c);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda
