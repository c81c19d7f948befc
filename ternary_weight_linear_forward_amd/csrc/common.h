// common.h -- device helpers shared by the libbitlinear kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

// dtype / layout codes of the C ABI (bitlinear.h).
enum { DT_F32 = 0, DT_BF16 = 1, DT_I8 = 2, DT_I32 = 3 };
enum { LAYOUT_I2 = 0, LAYOUT_B3 = 1, LAYOUT_B1 = 2 };

// A chunk is 16 bytes: one row's weights for one k-block; a tile is 16 rows.
constexpr int TILE_ROWS = 16;
constexpr int CHUNK_BYTES = 16;
constexpr int I2_KBLOCK = 64;
constexpr int B3_KBLOCK = 80;
// Word of four "T = 0" codes (c = 1 in every 2-bit field): padding for i2.
constexpr uint32_t I2_ZERO_WORD = 0x55555555u;

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// binary32 -> bfloat16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    uint32_t lsb = (u >> 16) & 1u;
    return static_cast<uint16_t>((u + 0x7fffu + lsb) >> 16);
}

// Four 2-bit offset codes c in {0,1,2}, one per byte, to signed bytes T = c - 1:
// c + 0x7f stays below 0x100 in every byte (no carries), and xor 0x80 maps
// 0x7f, 0x80, 0x81 to 0xff, 0x00, 0x01.
__device__ __forceinline__ uint32_t codes_to_signed(uint32_t c)
{
    return (c + 0x7f7f7f7fu) ^ 0x80808080u;
}

// The four words of signed weights held in one i2 word (16 weights, natural
// k order): word s covers weights 4s .. 4s+3 of the word's 16.
__device__ __forceinline__ v4i i2_word_to_signed16(uint32_t w)
{
    v4i r;
    r[0] = static_cast<int>(codes_to_signed(w & 0x03030303u));
    r[1] = static_cast<int>(codes_to_signed((w >> 2) & 0x03030303u));
    r[2] = static_cast<int>(codes_to_signed((w >> 4) & 0x03030303u));
    r[3] = static_cast<int>(codes_to_signed((w >> 6) & 0x03030303u));
    return r;
}

template <int XDT>
__device__ __forceinline__ float load_x(const void *X, int64_t idx)
{
    if constexpr (XDT == DT_F32)
        return static_cast<const float *>(X)[idx];
    else
        return bf16_bits_to_float(static_cast<const uint16_t *>(X)[idx]);
}

// Per-token quantisation of a row with absmax beta: q = clamp(rint(x * (127 /
// beta)), -127, 127), ties to even, evaluated as RN32(x~ * RN32(127 / b)) with
// b = beta / 2^e in [1, 2) and x~ = x / 2^e.  Dividing the row by a power of
// two does not change x / beta, so q is the same for a row and for the row
// scaled by 2^k.  Wherever 127 / beta is a finite binary32 (beta >= 2^-96 is
// enough) that equals RN32(x * RN32(127 / beta)): then pre = 1.  Below, 127 /
// beta would overflow (for beta < 127 / FLT_MAX), so x and beta are first
// multiplied by pre = 2^64, exactly (x <= beta < 2^-96), which brings beta
// into [2^-85, 2^-32) where the division is finite; the product x * pre * s
// is then the same real number as x~ * RN32(127 / b), rounded once.
struct TokenQuant {
    float pre; // 1 or 2^64, exact
    float s;   // RN32(127 / (beta * pre)), or 0 for beta = 0
};

__device__ __forceinline__ TokenQuant token_quant(float beta)
{
    const float pre = beta < 0x1p-96f ? 0x1p64f : 1.0f;
    TokenQuant t;
    t.pre = pre;
    t.s = beta > 0.0f ? 127.0f / (beta * pre) : 0.0f;
    return t;
}

// RN32(x * pre * s): x * pre is exact, so this is one rounding of the real
// product.  |result| <= 127 (1 + 2^-24)^2 < 127.5 for |x| <= beta.
__device__ __forceinline__ float token_scaled(float x, TokenQuant t) { return (x * t.pre) * t.s; }

// Four activations of a row whose absmax is beta (every |x| <= beta) to int8,
// packed in order: the values quant_one gives.  Every |RN32(x pre s)| < 127.5,
// so the clamp never acts; adding 1.5 * 2^23 (its own correctly rounded add:
// the build does not contract) rounds to an integer with ties to even, and the
// low byte of the sum is the int8 in two's complement.  Three v_perm_b32
// gather the four bytes: about 3.75 instructions per value against 8.
__device__ __forceinline__ uint32_t quant4_bounded(float x0, float x1, float x2, float x3, TokenQuant t)
{
    const uint32_t b0 = __float_as_uint(token_scaled(x0, t) + 12582912.0f);
    const uint32_t b1 = __float_as_uint(token_scaled(x1, t) + 12582912.0f);
    const uint32_t b2 = __float_as_uint(token_scaled(x2, t) + 12582912.0f);
    const uint32_t b3 = __float_as_uint(token_scaled(x3, t) + 12582912.0f);
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u); // q0, q1 in bytes 0, 1
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u); // q2, q3
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// One activation to int8: clamp(rint(x * pre * s), -127, 127), ties to even,
// as the low byte of the result.
__device__ __forceinline__ uint32_t quant_one(float x, TokenQuant t)
{
    float r = __builtin_rintf(token_scaled(x, t));
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return static_cast<uint32_t>(static_cast<int>(r)) & 0xffu;
}

// Per-token rescale factor (gamma * beta) / 127 in binary32.
__device__ __forceinline__ float token_scale(float gamma, float beta)
{
    float gb = gamma * beta;
    return gb / 127.0f;
}

// Store one output element: raw accumulator, or float(acc) * r in fp32 / bf16.
__device__ __forceinline__ void store_out(void *Y, int y_dtype, int64_t ldy, int64_t m, int64_t n, int acc,
                                          float r)
{
    const int64_t idx = m * ldy + n;
    if (y_dtype == DT_I32) {
        static_cast<int *>(Y)[idx] = acc;
    } else {
        float y = static_cast<float>(acc) * r;
        if (y_dtype == DT_F32)
            static_cast<float *>(Y)[idx] = y;
        else
            static_cast<uint16_t *>(Y)[idx] = float_to_bf16_rne(y);
    }
}

// |y| of one output element exactly as store_out stores it (fp32 or bf16).
__device__ __forceinline__ float stored_abs(int y_dtype, int acc, float r)
{
    const float y = static_cast<float>(acc) * r;
    if (y_dtype == DT_F32) return fabsf(y);
    return __uint_as_float((static_cast<uint32_t>(float_to_bf16_rne(y)) & 0x7fffu) << 16);
}

// Lane-wise product of two pairs of 16-bit integers (low 16 bits kept).
__device__ __forceinline__ uint32_t pk_mul_u16(uint32_t a, uint32_t b)
{
    typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
    v2u16 x = __builtin_bit_cast(v2u16, a), y = __builtin_bit_cast(v2u16, b);
    return __builtin_bit_cast(uint32_t, static_cast<v2u16>(x * y));
}

// Base-3 digits of the four b3 bytes of w.  A b3 byte holds the five-digit
// base-3 number v (digit 0 most significant) as u = ceil(256 v / 243), the
// fixed-point fraction v / 243 rounded up.  Then H_t = floor(u 3^t / 256) is
// the number formed by the leading t digits (an exhaustive check over the 243
// values confirms it), so digit t is H_{t+1} - 3 H_t.  The products u 3^t fit
// 16-bit lanes (u 3^5 < 2^16), two bytes per instruction, and their high
// bytes are gathered into one word per t with v_perm_b32.  Because the result
// of X_{t+1} - 3 X_t is a whole word of byte digits 0..2, the subtraction is
// exact on the packed word.  d[t] byte j = digit t of byte j of w.
struct B3Digits {
    uint32_t d[5];
};

__device__ __forceinline__ B3Digits b3_word_digits(uint32_t w)
{
    const uint32_t even = w & 0x00ff00ffu;                         // bytes 0 and 2
    const uint32_t odd = __builtin_amdgcn_perm(0u, w, 0x0c030c01u); // bytes 1 and 3
    uint32_t X[6];
    uint32_t p3 = 1;
#pragma unroll
    for (int t = 1; t <= 5; ++t) {
        p3 *= 3;
        const uint32_t ze = pk_mul_u16(even, p3 * 0x00010001u), zo = pk_mul_u16(odd, p3 * 0x00010001u);
        X[t] = __builtin_amdgcn_perm(zo, ze, 0x07030501u); // high byte of each lane, bytes in order
    }
    B3Digits r;
    r.d[0] = X[1];
#pragma unroll
    for (int t = 1; t < 5; ++t) {
        // 3 X_t as one full-rate shift-add: written as a multiply or as
        // x + (x << 1), the compiler forms a quarter-rate v_mad_u64_u32
        uint32_t x3;
        asm("v_lshl_add_u32 %0, %1, 1, %1" : "=v"(x3) : "v"(X[t]));
        r.d[t] = X[t + 1] - x3;
    }
    return r;
}

// The b3 byte of five "T = 0" weights: v = 121 (all digits 1), stored as
// ceil(256 * 121 / 243) = 128; four of them make the padding word.
constexpr uint32_t B3_ZERO_WORD = 0x80808080u;

// b3 byte of the digits c_0 .. c_4 (c_0 most significant): v = sum c_t 3^(4-t),
// stored as ceil(256 v / 243).
__device__ __forceinline__ uint32_t b3_encode(uint32_t v) { return (256u * v + 242u) / 243u; }

// Maximum of a non-negative value over the wave, in every lane: running
// maxima within rows of 16 lanes (DPP row shifts; lanes shifted in from
// outside the row read 0), then row 15's value broadcast into the next rows
// (row_bcast:15, row_bcast:31), and lane 63's result read back.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float x)
{
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true);
    return fmaxf(x, __int_as_float(y));
}

__device__ __forceinline__ float wave_max_nonneg(float v)
{
    v = dpp_max_step<0x111, 0xf>(v); // row_shr:1
    v = dpp_max_step<0x112, 0xf>(v); // row_shr:2
    v = dpp_max_step<0x114, 0xf>(v); // row_shr:4
    v = dpp_max_step<0x118, 0xf>(v); // row_shr:8
    v = dpp_max_step<0x142, 0xa>(v); // row_bcast:15
    v = dpp_max_step<0x143, 0xc>(v); // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

} // namespace bl
