// kda_chunk.h -- definitions shared by the chunkwise prefill kernels: the
// per-(chunk, head) slab that the intra-chunk kernels write and the
// inter-chunk kernel reads, and small device and host helpers.
#pragma once

#include "kda_device.h"

#include <hip/hip_runtime.h>

namespace kda {

// ---------------------------------------------------------------------------
// Slab layout (bytes from the slab start).  A "fragment" is 64 lanes x 16 B
// in the lane order of the MFMA operand it feeds (kda_device.h).  fp32 path:
// fp32 fragments, one K16 tile each.  bf16 path: the operands of the serial
// state chain are stored in fp16, one fragment spanning two K16 tiles (one
// 16x16x32 MFMA); they are bounded by construction (|Gamma*Q|, |K~| <= 1,
// W and A_qk are products of contractions), and the state-carrying side of
// every chain product is scaled by a power of two per chunk before it is
// rounded to fp16.  U is stored per 16x16 tile in fp16 times 2^-e, with the
// tile's exponent e (from its largest magnitude) kept after gamma_C.  Of
// A_qk's 8 fp16 fragments only the 6 that are not all zero are stored.
// ---------------------------------------------------------------------------
template <int D, bool F32>
struct Slab {
    static constexpr int KT = D / 16;                 // 16-wide key / value tiles
    static constexpr int NKF = F32 ? D / 16 : D / 32; // fragments over d per 16-row tile
    static constexpr int NCF = F32 ? 4 : 2;           // fragments over the 64 chunk rows
    static constexpr int SPL = 1;                     // one fragment per operand tile (fp32 or fp16)
    static constexpr int NAQ = F32 ? 4 * NCF : 6;     // A_qk fragments stored
    static constexpr size_t FRAG = 1024;
    static constexpr size_t UT = F32 ? FRAG : FRAG / 2;         // bytes per U tile
    static constexpr size_t negW = 0;                           // -W      [I][NKF][SPL]
    static constexpr size_t qg = negW + 4 * NKF * SPL * FRAG;   // Gamma*Q [I][NKF][SPL]
    static constexpr size_t kdT = qg + 4 * NKF * SPL * FRAG;    // ((gamma_C/Gamma)*K)^T [t][NCF][SPL]
    static constexpr size_t aqk = kdT + KT * NCF * SPL * FRAG;  // A_qk    [NAQ]
    static constexpr size_t gamma = aqk + NAQ * FRAG;           // gamma_C [D] fp32, then
    static constexpr size_t uexp = gamma + D * 4;               //   U tile exponents [I][KT] int32 (bf16)
    static constexpr size_t u = gamma + FRAG;                   // U (accumulator layout) [I][KT]
    static constexpr size_t bytes = u + 4 * KT * UT;
    // The inter-chunk kernel stages two regions through LDS, A = [-W | Gamma*Q]
    // and B = [K~^T | A_qk | gamma], each a whole number of fragments; an LDS
    // buffer holds them at their slab offsets.  U goes to registers.
    static constexpr int FA = (int)((kdT - negW) / FRAG);
    static constexpr int FB = (int)((u - kdT) / FRAG);
    static_assert(D * 4 + 4 * KT * 4 <= (int)FRAG, "gamma and the U exponents fit one fragment");
};

// A_qk fragment index (bf16 path) of row tile I, column pair qf: tiles 0 and
// 1 need one fragment, tiles 2 and 3 two.
__device__ __forceinline__ int aqk_frag(int I, int qf) { return I < 2 ? I : 2 * I - 2 + qf; }

// Store two fp32 quads (K16 tiles t, t + 1) as one fp16 fragment.
__device__ __forceinline__ void store_f16(unsigned char *dst, f32x4 x0, f32x4 x1) {
    *reinterpret_cast<u32x4 *>(dst) = quads_to_f16(x0, x1);
}

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
__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// Inclusive prefix sum over the 16 lanes of each DPP row (row_shr by 1, 2,
// 4, 8; lanes shifted in from outside the row read 0).
__device__ __forceinline__ float row16_inclusive_scan(float x) {
#define KDA_SHR(n)                                                                          \
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + (n), 0xf, \
                                                    0xf, true))
    KDA_SHR(1);
    KDA_SHR(2);
    KDA_SHR(4);
    KDA_SHR(8);
#undef KDA_SHR
    return x;
}

// Units [0, n) spread over NW waves with a trip count fixed at compile time
// (only the last pass is conditional, and only when NW does not divide n),
// so the number of stores a wave has in flight is known to the compiler.
template <int n, int NW, typename F>
__device__ __forceinline__ void for_wave_units(int wave, F &&f) {
#pragma unroll
    for (int r = 0; r < (n + NW - 1) / NW; ++r) {
        const int unit = wave + r * NW;
        if (n % NW == 0 || unit < n) f(unit);
    }
}

template <bool F32IO, typename Q>
__device__ __forceinline__ f32x4 quad_f32(Q x) {
    if constexpr (F32IO) {
        return x;
    } else {
        return f32x4{bf16_lo_half(x[0]), bf16_hi_half(x[0]), bf16_lo_half(x[1]), bf16_hi_half(x[1])};
    }
}

// ---------------------------------------------------------------------------
// Host helpers.
// ---------------------------------------------------------------------------
static inline int device_cus() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
    }
    return cus;
}

template <typename K>
static inline bool set_lds(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess;
}

}  // namespace kda
