// gemv_core.h -- the k-step of the matrix-core decode product, shared by the
// single-layer GEMVs (gemv.hip) and the grouped one (group.hip).
//
// A k-step is 4 consecutive k-blocks (i2: 256 weights, b3: 320, b1: 512).  In
// a k-step, lane l (i = l % 16, g = l / 16) holds the 16-byte chunk of row
// 16*tile + i at k-block 4*step + g; NMF activation operands of 16 tokens x
// 64 k (v_mfma_i32_16x16x64_i8) multiply the unpacked weights.  The result
// lane l holds tokens 4g .. 4g+3 of weight row i.
#pragma once

#include "common.h"

namespace bl {

// Signed weights of one i2 word (16 weights, natural k order).  v_perm_b32
// with selector bytes c in {0, 1, 2} picks byte c of 0x000100ff: -1, 0, +1.
__device__ __forceinline__ v4i i2_word_signed(uint32_t w)
{
    v4i r;
    r[0] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, w & 0x03030303u));
    r[1] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, (w >> 2) & 0x03030303u));
    r[2] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, (w >> 4) & 0x03030303u));
    r[3] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, (w >> 6) & 0x03030303u));
    return r;
}

template <int LAYOUT>
struct StepShape;
template <>
struct StepShape<LAYOUT_I2> {
    static constexpr int NMF = 4, KBLK = 64;
};
template <>
struct StepShape<LAYOUT_B3> {
    static constexpr int NMF = 5, KBLK = 80;
};
template <>
struct StepShape<LAYOUT_B1> {
    static constexpr int NMF = 8, KBLK = 128;
};

// Signed weights of half h of a b1 word (16 binary weights 16h .. 16h+15 of
// the word's 32, natural k order): (w >> (4h + s)) & 0x01010101 holds the bits
// of weights 16h + 4s .. +3 as bytes, and v_perm_b32 maps 0 -> -1, 1 -> +1.
__device__ __forceinline__ v4i b1_half_signed(uint32_t w, int h)
{
    v4i r;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        r[s] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000001ffu, (w >> (4 * h + s)) & 0x01010101u));
    return r;
}

// Layouts whose k-step multiplies unsigned codes, with no per-word conversion
// to signed bytes: the digits c = T + 1 in {0, 1, 2} for b3, the bit
// b = (T + 1) / 2 for b1.  Then sum_k q T = acc - S (b3) or 2 acc - S (b1)
// with S = sum_k q[m][k], the same for every weight row, computed once per
// wave (act_sum_step).  (i2 keeps the signed form: with its cheap unpack the
// extra MFMAs of S cancel the saved instructions, measured on the 70B layers.)
template <int LAYOUT>
constexpr bool kOffsetCodes = LAYOUT != LAYOUT_I2;

template <int LAYOUT>
__device__ __forceinline__ int offset_fix(int acc, int s)
{
    return LAYOUT == LAYOUT_B1 ? 2 * acc - s : acc - s;
}
template <int LAYOUT>
__device__ __forceinline__ v4i offset_fix(v4i acc, v4i s)
{
    return LAYOUT == LAYOUT_B1 ? 2 * acc - s : acc - s;
}

// sacc[m] += sum of the activations of one k-step, in the MFMA output layout
// (the product with an all-ones B operand; every weight row gets the same sum).
template <int NMF>
__device__ __forceinline__ void act_sum_step(const v4i (&a)[NMF], v4i &sacc)
{
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
    for (int d = 0; d < NMF; ++d) sacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d], ones, sacc, 0, 0, 0);
}

// One k-step of TW tiles: unpack the weight chunks and accumulate.
template <int LAYOUT, int TW, int NMF>
__device__ __forceinline__ void gemv_step(const uint4 (&b)[TW], const v4i (&a)[NMF], v4i (&acc)[TW])
{
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const uint32_t wd[4] = {b[t].x, b[t].y, b[t].z, b[t].w};
        if constexpr (LAYOUT == LAYOUT_I2 && kOffsetCodes<LAYOUT>) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const v4i bt = {static_cast<int>(wd[d] & 0x03030303u), static_cast<int>((wd[d] >> 2) & 0x03030303u),
                                static_cast<int>((wd[d] >> 4) & 0x03030303u),
                                static_cast<int>((wd[d] >> 6) & 0x03030303u)};
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d], bt, acc[t], 0, 0, 0);
            }
        } else if constexpr (LAYOUT == LAYOUT_I2) {
#pragma unroll
            for (int d = 0; d < 4; ++d)
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d], i2_word_signed(wd[d]), acc[t], 0, 0, 0);
        } else if constexpr (LAYOUT == LAYOUT_B1 && kOffsetCodes<LAYOUT>) {
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const uint32_t w = wd[d / 2] >> (4 * (d % 2));
                const v4i bt = {static_cast<int>(w & 0x01010101u), static_cast<int>((w >> 1) & 0x01010101u),
                                static_cast<int>((w >> 2) & 0x01010101u), static_cast<int>((w >> 3) & 0x01010101u)};
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d], bt, acc[t], 0, 0, 0);
            }
        } else if constexpr (LAYOUT == LAYOUT_B1) {
#pragma unroll
            for (int d = 0; d < 8; ++d)
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d], b1_half_signed(wd[d / 2], d % 2), acc[t], 0, 0,
                                                               0);
        } else {
            // unsigned digits c = T + 1: the caller subtracts sum_k q (act_sum_step)
            B3Digits dg[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) dg[q] = b3_word_digits(wd[q]);
#pragma unroll
            for (int d = 0; d < 5; ++d) {
                v4i bt = {static_cast<int>(dg[0].d[d]), static_cast<int>(dg[1].d[d]), static_cast<int>(dg[2].d[d]),
                          static_cast<int>(dg[3].d[d])};
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d], bt, acc[t], 0, 0, 0);
            }
        }
    }
}

} // namespace bl
