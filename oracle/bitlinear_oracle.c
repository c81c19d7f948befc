/*
 * bitlinear_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * A plain, slow, obviously-correct CPU implementation of the BitLinear forward
 * pass of BitNet b1.58.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header,
 * table or constant with the HIP library and includes no HIP header.
 *
 * What the sources say, and what is a reading of them:
 *   - "The Era of 1-bit LLMs" abstract (searcharxiv page, Abstract): every
 *     weight of BitNet b1.58 is ternary, one of {-1, 0, +1}.
 *   - LIT-380 record (dmarx anthology), Key takeaways, bullet 1: nn.Linear is
 *     replaced by BitLinear; weights are mapped to {-1, 0, +1} by an absmean
 *     quantisation function; activations are 8-bit.
 *   - LIT-380, Key takeaways, bullet 4: the matrix product turns into integer
 *     addition with no multiplications.
 *   - HackerPapers digest, thread "GPUs Go Brrr": 1.58 bits is 2 bits in
 *     practice; thread "How to pack ternary numbers in 8-bit bytes": ternary
 *     values can be packed several to a byte (base 3).
 * The pages print no formula.  The formulas below are the plainest reading
 * consistent with those statements (one per-tensor scale gamma = mean|W|,
 * per-token absmax to 127, exact integer product, rescale gamma*beta/127);
 * every open point (rounding, ties, operation order, layout) is fixed here and
 * listed with its justification in the design notes.
 *
 * Arithmetic: IEEE-754 binary32 with round-to-nearest-even, compiled with
 * -ffp-contract=off and without fast-math.  The integer product accumulates in
 * int64 and checks that the result fits int32.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

enum {
    ORACLE_OK = 0,
    ORACLE_ERR_NONFINITE = 1, /* a NaN or infinity in a float input            */
    ORACLE_ERR_RANGE = 2,     /* an int32 accumulator would overflow           */
    ORACLE_ERR_CODE = 3,      /* a packed byte holds a code that is never written */
    ORACLE_ERR_ARG = 4        /* a size is out of range                        */
};

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ------------------------------------------------------------------------ */
/* gamma = mean |W|, exact, rounded once to binary32 (ties to even).        */
/* ------------------------------------------------------------------------ */
/*
 * Every finite |w| equals m * 2^(p - 149) with m < 2^24 an integer and
 * p = max(biased_exponent, 1) - 1 in [0, 253].  So the exact sum S of all |w|
 * is an integer number of units 2^-149.  S is kept in a 512-bit little-endian
 * integer (8 limbs); 2^24 * 2^253 * 2^40 elements stay far below 2^512.
 */
#define NLIMB 8

static void big_add_shifted(uint64_t *acc, uint64_t m, unsigned shift)
{
    unsigned limb = shift / 64, bit = shift % 64;
    uint64_t lo = m << bit;
    uint64_t hi = bit ? (m >> (64 - bit)) : 0;
    unsigned __int128 s = (unsigned __int128)acc[limb] + lo;
    acc[limb] = (uint64_t)s;
    uint64_t carry = (uint64_t)(s >> 64) + hi;
    for (unsigned i = limb + 1; i < NLIMB && carry; ++i) {
        s = (unsigned __int128)acc[i] + carry;
        acc[i] = (uint64_t)s;
        carry = (uint64_t)(s >> 64);
    }
}

/*
 * The exact sum as an 8-limb integer in units of 2^-149.
 * Returns ORACLE_ERR_NONFINITE if any element is NaN or infinite.
 */
static int exact_abs_sum(const float *w, int64_t count, uint64_t sum[NLIMB])
{
    memset(sum, 0, NLIMB * sizeof(uint64_t));
    for (int64_t i = 0; i < count; ++i) {
        uint32_t b = bits_of(w[i]) & 0x7fffffffu;
        uint32_t e = b >> 23, f = b & 0x7fffffu;
        if (e == 255) return ORACLE_ERR_NONFINITE;
        uint64_t m = e ? (f | 0x800000u) : f;
        unsigned p = e ? e - 1 : 0;
        if (m) big_add_shifted(sum, m, p);
    }
    return ORACLE_OK;
}

/*
 * Nearest binary32 (ties to even) to the rational value S * 2^-149 / D.
 * Q = floor(S * 2^64 / D) is formed by long division, so Q counts units of
 * 2^-213 and 'sticky' records a non-zero remainder.  The result's ulp, in the
 * same units, is 2^max(msb(Q) - 23, 64): 2^64 units = 2^-149, the subnormal ulp.
 */
static float round_ratio_to_f32(const uint64_t S[NLIMB], uint64_t D)
{
    uint64_t num[NLIMB + 1], Q[NLIMB + 1];
    num[0] = 0;
    for (int i = 0; i < NLIMB; ++i) num[i + 1] = S[i]; /* S << 64 */
    unsigned __int128 rem = 0;
    for (int i = NLIMB; i >= 0; --i) {
        unsigned __int128 cur = (rem << 64) | num[i];
        Q[i] = (uint64_t)(cur / D);
        rem = cur % D;
    }
    int sticky = rem != 0;
    int msb = -1;
    for (int i = NLIMB; i >= 0 && msb < 0; --i)
        if (Q[i]) msb = i * 64 + 63 - __builtin_clzll(Q[i]);
    if (msb < 0) return 0.0f; /* S == 0 */
    int shift = msb - 23 > 64 ? msb - 23 : 64;
    /* mantissa = Q >> shift (at most 24 bits), plus the bits below it */
    uint64_t mant = 0;
    for (int b = msb; b >= shift; --b)
        mant = (mant << 1) | ((Q[b / 64] >> (b % 64)) & 1u);
    int half = (Q[(shift - 1) / 64] >> ((shift - 1) % 64)) & 1u;
    int below = sticky;
    for (int b = shift - 2; b >= 0 && !below; --b)
        if ((Q[b / 64] >> (b % 64)) & 1u) below = 1;
    if (half && (below || (mant & 1u))) mant += 1; /* may reach 2^24: still exact */
    return ldexpf((float)mant, shift - 213);
}

/* gamma of a tensor of 'count' fp32 weights (count >= 1). */
int oracle_absmean(const float *w, int64_t count, float *gamma)
{
    uint64_t S[NLIMB];
    if (count <= 0 || count > ((int64_t)1 << 40)) return ORACLE_ERR_ARG;
    int st = exact_abs_sum(w, count, S);
    if (st) return st;
    *gamma = round_ratio_to_f32(S, (uint64_t)count);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Ternarisation: T = clamp(rint(w / gamma), -1, +1); gamma == 0 gives T = 0 */
/* ------------------------------------------------------------------------ */
int oracle_ternarize(const float *w, int64_t count, float gamma, int8_t *t)
{
    if (!isfinite(gamma)) return ORACLE_ERR_NONFINITE;
    for (int64_t i = 0; i < count; ++i) {
        if (!isfinite(w[i])) return ORACLE_ERR_NONFINITE;
        if (gamma == 0.0f) { t[i] = 0; continue; }
        float r = rintf(w[i] / gamma); /* IEEE division, then ties-to-even */
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        t[i] = (int8_t)r;
    }
    return ORACLE_OK;
}

/* Binary weights, the predecessor variant: the original BitNet used weights  */
/* -1 or +1 (HackerPapers digest of the paper's threads; LIT-380, Key        */
/* takeaways, bullet 2, contrasts three states with two).  No formula is on   */
/* the pages; reading: T = sign(w) with w >= 0 (including -0) giving +1, and  */
/* the same scale gamma = mean|W| as the ternary path.                        */
/* ------------------------------------------------------------------------ */
int oracle_binarize(const float *w, int64_t count, int8_t *t)
{
    for (int64_t i = 0; i < count; ++i) {
        if (!isfinite(w[i])) return ORACLE_ERR_NONFINITE;
        t[i] = w[i] >= 0.0f ? 1 : -1;
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Packed layouts (a convention of this library; the pages fix none).        */
/* ------------------------------------------------------------------------ */
/*
 * Both layouts store the code c = T + 1 in {0, 1, 2} and pad with T = 0.
 * Rows are grouped in tiles of 16; inside a tile the chunks are ordered by
 * k-block, then by row.  A chunk is 16 bytes and holds one row's weights for
 * one k-block.
 *
 * "i2" (2 bits per weight): a k-block is 64 weights.  The chunk of row n and
 * k-block kb starts at byte ((n/16)*KB + kb)*256 + (n%16)*16, KB = ceil(K/64).
 * Its little-endian 32-bit word d (d = 0..3) holds weights kb*64 + 16d + 4s + j
 * (s, j = 0..3) at bits 8j + 2s .. 8j + 2s + 1.
 *
 * "b3" (base 3, 5 weights per byte): a k-block is 80 weights.  The chunk of
 * row n and k-block kb starts at byte ((n/16)*KB3 + kb)*256 + (n%16)*16,
 * KB3 = ceil(K/80).  Its byte i (i = 0..15) holds the five weights
 * kb*80 + 16t + i (t = 0..4) as the base-3 number v = sum_t c_t * 3^(4 - t)
 * (weight t = 0 the most significant digit), stored as the byte
 * ceil(256 * v / 243): v / 243 as an 8-bit fixed-point fraction, rounded up.
 * The map is one-to-one (v = floor(243 * byte / 256) recovers v), so 243 of
 * the 256 byte values occur.  Digit t of bytes 0..15 covers 16 consecutive
 * weights.
 *
 * "b1" (1 bit per weight, binary weights only): a k-block is 128 weights.  The
 * chunk of row n and k-block kb starts at byte ((n/16)*KB1 + kb)*256 +
 * (n%16)*16, KB1 = ceil(K/128).  Its word d (d = 0..3) holds weights
 * kb*128 + 32d + 4s + j (s = 0..7, j = 0..3) at bit 8j + s: 1 for +1, 0 for
 * -1.  Bits past K (and rows past N) are 0; binary weights have no zero, so
 * those positions carry a weight and the product must meet zero activations
 * there.
 */
static int8_t t_at(const int8_t *t, int64_t N, int64_t K, int64_t n, int64_t k)
{
    return (n < N && k < K) ? t[n * K + k] : 0;
}

int64_t oracle_packed_bytes(int64_t N, int64_t K, int layout)
{
    int64_t NT = (N + 15) / 16;
    int64_t KB = layout == 0 ? (K + 63) / 64 : (layout == 1 ? (K + 79) / 80 : (K + 127) / 128);
    return NT * KB * 256;
}

int oracle_pack_i2(const int8_t *t, int64_t N, int64_t K, uint8_t *p)
{
    int64_t NT = (N + 15) / 16, KB = (K + 63) / 64;
    for (int64_t n = 0; n < NT * 16; ++n)
        for (int64_t kb = 0; kb < KB; ++kb) {
            uint8_t *chunk = p + ((n / 16) * KB + kb) * 256 + (n % 16) * 16;
            for (int d = 0; d < 4; ++d)
                for (int j = 0; j < 4; ++j) {
                    unsigned byte = 0;
                    for (int s = 0; s < 4; ++s) {
                        int64_t k = kb * 64 + 16 * d + 4 * s + j;
                        int8_t v = t_at(t, N, K, n, k);
                        if (v < -1 || v > 1) return ORACLE_ERR_ARG;
                        byte |= (unsigned)(v + 1) << (2 * s);
                    }
                    chunk[4 * d + j] = (uint8_t)byte;
                }
        }
    return ORACLE_OK;
}

int oracle_unpack_i2(const uint8_t *p, int64_t N, int64_t K, int8_t *t)
{
    int64_t KB = (K + 63) / 64;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t kb = k / 64, r = k % 64;
            int d = (int)(r / 16), s = (int)((r % 16) / 4), j = (int)(r % 4);
            uint8_t byte = p[((n / 16) * KB + kb) * 256 + (n % 16) * 16 + 4 * d + j];
            unsigned c = (byte >> (2 * s)) & 3u;
            if (c == 3) return ORACLE_ERR_CODE;
            t[n * K + k] = (int8_t)((int)c - 1);
        }
    return ORACLE_OK;
}

int oracle_pack_b3(const int8_t *t, int64_t N, int64_t K, uint8_t *p)
{
    int64_t NT = (N + 15) / 16, KB = (K + 79) / 80;
    for (int64_t n = 0; n < NT * 16; ++n)
        for (int64_t kb = 0; kb < KB; ++kb) {
            uint8_t *chunk = p + ((n / 16) * KB + kb) * 256 + (n % 16) * 16;
            for (int i = 0; i < 16; ++i) {
                unsigned byte = 0;
                for (int d = 0; d < 5; ++d) {
                    int8_t v = t_at(t, N, K, n, kb * 80 + 16 * d + i);
                    if (v < -1 || v > 1) return ORACLE_ERR_ARG;
                    byte = byte * 3 + (unsigned)(v + 1);
                }
                chunk[i] = (uint8_t)((256 * byte + 242) / 243); /* ceil(256 v / 243) */
            }
        }
    return ORACLE_OK;
}

int oracle_unpack_b3(const uint8_t *p, int64_t N, int64_t K, int8_t *t)
{
    int64_t KB = (K + 79) / 80;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t kb = k / 80, r = k % 80;
            unsigned byte = p[((n / 16) * KB + kb) * 256 + (n % 16) * 16 + r % 16];
            unsigned v = (243 * byte) / 256;
            if ((256 * v + 242) / 243 != byte) return ORACLE_ERR_CODE; /* not a b3 byte */
            unsigned digit = v;
            for (int d = 4; d > (int)(r / 16); --d) digit /= 3;
            t[n * K + k] = (int8_t)((int)(digit % 3) - 1);
        }
    return ORACLE_OK;
}

int oracle_pack_b1(const int8_t *t, int64_t N, int64_t K, uint8_t *p)
{
    int64_t NT = (N + 15) / 16, KB = (K + 127) / 128;
    for (int64_t n = 0; n < NT * 16; ++n)
        for (int64_t kb = 0; kb < KB; ++kb) {
            uint8_t *chunk = p + ((n / 16) * KB + kb) * 256 + (n % 16) * 16;
            for (int d = 0; d < 4; ++d)
                for (int j = 0; j < 4; ++j) {
                    unsigned byte = 0;
                    for (int s = 0; s < 8; ++s) {
                        int64_t k = kb * 128 + 32 * d + 4 * s + j;
                        if (n >= N || k >= K) continue; /* padding: bit 0 */
                        int8_t v = t[n * K + k];
                        if (v != 1 && v != -1) return ORACLE_ERR_ARG;
                        byte |= (unsigned)(v == 1) << s;
                    }
                    chunk[4 * d + j] = (uint8_t)byte;
                }
        }
    return ORACLE_OK;
}

int oracle_unpack_b1(const uint8_t *p, int64_t N, int64_t K, int8_t *t)
{
    int64_t KB = (K + 127) / 128;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t kb = k / 128, r = k % 128;
            int d = (int)(r / 32), s = (int)((r % 32) / 4), j = (int)(r % 4);
            uint8_t byte = p[((n / 16) * KB + kb) * 256 + (n % 16) * 16 + 4 * d + j];
            t[n * K + k] = (byte >> s) & 1u ? 1 : -1;
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Per-token absmax activation quantisation to int8 (Qb = 127).              */
/* ------------------------------------------------------------------------ */
/* bfloat16 is the top half of a binary32, so widening is exact. */
void oracle_bf16_to_f32(const uint16_t *x, int64_t count, float *out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = float_of((uint32_t)x[i] << 16);
}

/*
 * beta_m = max_k |x_mk|, and q_mk = clamp(rint(x_mk * (127 / beta_m)), -127,
 * 127) with ties to even, evaluated in binary32 as follows.  Let 2^e be the
 * power of two with 1 <= beta_m / 2^e < 2, and write b = beta_m / 2^e and
 * x~ = x_mk / 2^e (exact real numbers).  Then
 *     s = RN32(127 / b)          (one correctly rounded division per token)
 *     q = clamp(rint(RN32(x~ * s)), -127, 127).
 * Dividing a whole row by 2^e leaves every ratio x / beta unchanged, so q is
 * the same for a row and for the row scaled by any power of two (as long as
 * the scaled row is still exact in binary32).  Wherever 127 / beta_m is a
 * finite binary32 (beta_m >= 127 / FLT_MAX, about 3.7e-37) this is the same
 * as RN32(x * RN32(127 / beta_m)), because then RN32(127 / beta_m) = s / 2^e
 * exactly; for smaller beta_m that form would overflow to infinity, this one
 * does not.  beta_m = 0 (an all-zero row) gives q = 0.
 * x is [M x K] with row stride ldx; the rounding is done in binary64, where
 * x~ and the product x~ * s (24 x 24 significant bits) are exact, and the
 * product is rounded once to binary32.
 */
int oracle_quant_act(const float *x, int64_t M, int64_t K, int64_t ldx, int8_t *q, float *beta)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * ldx;
        float b = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(row[k])) return ORACLE_ERR_NONFINITE;
            float a = fabsf(row[k]);
            if (a > b) b = a;
        }
        beta[m] = b;
        if (b == 0.0f) {
            for (int64_t k = 0; k < K; ++k) q[m * K + k] = 0;
            continue;
        }
        int E;
        (void)frexpf(b, &E);               /* b = f * 2^E, 0.5 <= f < 1 */
        const int e = E - 1;               /* 1 <= b / 2^e < 2          */
        const float bn = ldexpf(b, -e);    /* exact: b's significand    */
        const float s = 127.0f / bn;       /* in (63.5, 127]            */
        for (int64_t k = 0; k < K; ++k) {
            const double xn = ldexp((double)row[k], -e); /* exact in binary64 */
            const float v = (float)(xn * (double)s);     /* exact product, one rounding */
            float r = rintf(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[m * K + k] = (int8_t)r;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Exact integer product: acc[m][n] = sum_k q[m][k] * T[n][k].               */
/* ------------------------------------------------------------------------ */
int oracle_matmul(const int8_t *q, const int8_t *t, int64_t M, int64_t N, int64_t K, int32_t *acc)
{
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)q[m * K + k] * (int64_t)t[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) bad = 1;
            acc[m * N + n] = (int32_t)s;
        }
    return bad ? ORACLE_ERR_RANGE : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Rescale: r_m = (gamma * beta_m) / 127, y = float(acc) * r_m.              */
/* ------------------------------------------------------------------------ */
void oracle_rescale(const int32_t *acc, const float *beta, float gamma, int64_t M, int64_t N, float *y)
{
    for (int64_t m = 0; m < M; ++m) {
        float gb = gamma * beta[m];
        float r = gb / 127.0f;
        for (int64_t n = 0; n < N; ++n) y[m * N + n] = (float)acc[m * N + n] * r;
    }
}

/* binary32 -> bfloat16, round to nearest, ties to even (finite inputs). */
void oracle_f32_to_bf16(const float *y, int64_t count, uint16_t *out)
{
    for (int64_t i = 0; i < count; ++i) {
        uint32_t u = bits_of(y[i]);
        u += 0x7fffu + ((u >> 16) & 1u);
        out[i] = (uint16_t)(u >> 16);
    }
}
