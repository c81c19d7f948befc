// weights.hip -- absmean ternarisation and packing of BitLinear weights.
//
// LIT-380 record (dmarx anthology), Key takeaways, bullet 1: an absmean
// function maps the weights to {-1, 0, +1}.  Reading: one scale per tensor,
// gamma = mean|W|, and T = clamp(rint(W / gamma), -1, 1) with ties to even.
//
// gamma must be bit-identical however the sum is ordered, so it is computed
// exactly: every finite |w| is m * 2^(p - 149) with m < 2^24 and
// p = max(biased exponent, 1) - 1, so per-exponent integer sums of m are exact
// and order-free (integer atomics).  A one-thread kernel turns the 256 sums
// into the rational S * 2^-149 / (N K) and rounds it once to binary32.
//
// Done once per weight tensor at load time; not part of the per-token path.
#include "common.h"
#include "launch.h"

namespace bl {

__global__ void k_zero_u64(unsigned long long *p, int n)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

// Per-exponent sums of the 24-bit significands of |W|.
// buckets[e] accumulates m for every weight whose biased exponent is e
// (e == 255 counts non-finite values, which are outside the contract).
__global__ __launch_bounds__(256) void k_abs_buckets(const float *__restrict__ W, int64_t N, int64_t K,
                                                     int64_t ldw, unsigned long long *__restrict__ buckets)
{
    __shared__ unsigned long long lds[256];
    lds[threadIdx.x] = 0ull;
    __syncthreads();
    const bool vec = (K % 4 == 0) && (ldw % 4 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0);
    for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
        const float *row = W + n * ldw;
        if (vec) {
            for (int64_t k = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4; k < K;
                 k += static_cast<int64_t>(gridDim.x) * 1024) {
                float4 v = *reinterpret_cast<const float4 *>(row + k);
                float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t b = __float_as_uint(e4[j]) & 0x7fffffffu;
                    uint32_t e = b >> 23;
                    uint32_t m = e ? ((b & 0x7fffffu) | 0x800000u) : b;
                    if (e == 255u) m = 1u;
                    if (m) atomicAdd(&lds[e], static_cast<unsigned long long>(m));
                }
            }
        } else {
            for (int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; k < K;
                 k += static_cast<int64_t>(gridDim.x) * 256) {
                uint32_t b = __float_as_uint(row[k]) & 0x7fffffffu;
                uint32_t e = b >> 23;
                uint32_t m = e ? ((b & 0x7fffffu) | 0x800000u) : b;
                if (e == 255u) m = 1u;
                if (m) atomicAdd(&lds[e], static_cast<unsigned long long>(m));
            }
        }
    }
    __syncthreads();
    unsigned long long v = lds[threadIdx.x];
    if (v) atomicAdd(&buckets[threadIdx.x], v);
}

// gamma = RN32( S * 2^-149 / count ), S = sum_e buckets[e] * 2^(max(e,1)-1).
// S is held in base-2^24 digits; the quotient gets three extra digits
// (72 fractional bits) plus a sticky remainder, enough to round exactly.
__global__ void k_gamma_finalize(const unsigned long long *__restrict__ buckets, int64_t count,
                                 float *__restrict__ gamma)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    if (buckets[255] != 0ull) { // a non-finite weight
        *gamma = __uint_as_float(0x7fc00000u);
        return;
    }
    constexpr int ND = 16;      // 16 * 24 = 384 bits, above the 318 that S can use
    constexpr int FRAC = 3;     // extra quotient digits
    unsigned long long dig[ND + FRAC];
    for (int i = 0; i < ND + FRAC; ++i) dig[i] = 0ull;
    // S * 2^72: digit index offset FRAC.
    for (int e = 0; e < 255; ++e) {
        unsigned long long B = buckets[e];
        if (!B) continue;
        int p = (e ? e : 1) - 1;
        // split B into 24-bit pieces, each shifted by p
        for (int piece = 0; piece < 3; ++piece) {
            unsigned long long part = (B >> (24 * piece)) & 0xffffffull;
            if (!part) continue;
            int bit = p + 24 * piece;
            int di = FRAC + bit / 24, off = bit % 24;
            unsigned long long v = part << off; // < 2^47
            dig[di] += v & 0xffffffull;
            dig[di + 1] += v >> 24;
        }
    }
    for (int i = 0; i < ND + FRAC - 1; ++i) { // carry-normalise to 24-bit digits
        dig[i + 1] += dig[i] >> 24;
        dig[i] &= 0xffffffull;
    }
    const unsigned long long D = static_cast<unsigned long long>(count);
    unsigned long long q[ND + FRAC];
    unsigned long long rem = 0ull;
    for (int i = ND + FRAC - 1; i >= 0; --i) {
        unsigned long long cur = (rem << 24) | dig[i]; // rem < D < 2^40
        q[i] = cur / D;
        rem = cur % D;
    }
    // Q counts units of 2^-(149 + 72) = 2^-221.
    int msb = -1;
    for (int i = ND + FRAC - 1; i >= 0 && msb < 0; --i)
        if (q[i]) msb = i * 24 + (63 - __builtin_clzll(q[i]));
    if (msb < 0) { *gamma = 0.0f; return; }
    int shift = msb - 23;
    if (shift < 72) shift = 72; // the binary32 ulp is at least 2^-149
    auto qbit = [&](int b) -> unsigned { return b < 0 ? 0u : static_cast<unsigned>((q[b / 24] >> (b % 24)) & 1ull); };
    unsigned long long mant = 0ull;
    for (int b = msb; b >= shift; --b) mant = (mant << 1) | qbit(b);
    unsigned half = qbit(shift - 1);
    bool lower = rem != 0ull;
    for (int b = shift - 2; b >= 0 && !lower; --b) lower = qbit(b) != 0u;
    if (half && (lower || (mant & 1ull))) ++mant;
    if (mant == (1ull << 24)) { mant >>= 1; ++shift; }
    uint32_t bits;
    if (mant < (1ull << 23)) {
        bits = static_cast<uint32_t>(mant); // subnormal: shift == 72
    } else {
        uint32_t be = static_cast<uint32_t>(shift - 71); // biased exponent
        bits = (be << 23) | (static_cast<uint32_t>(mant) & 0x7fffffu);
    }
    *gamma = __uint_as_float(bits);
}

// T = clamp(rint(fl32(w / gamma)), -1, 1).  For x >= 0, rint(fl32(x)) >= 1
// exactly when fl32(x) > 0.5, i.e. when x > 0.5 + 2^-25 (below 0.5 the binary32
// spacing is 2^-25, above it 2^-24, and the midpoint 0.5 + 2^-25 rounds to the
// even 0.5).  So T != 0 iff 2|w| > gamma * (1 + 2^-24), a comparison that is
// exact in binary64 (a 24-bit by 25-bit product).
__global__ __launch_bounds__(256) void k_ternarize(const float *__restrict__ W, int64_t N, int64_t K,
                                                   int64_t ldw, const float *__restrict__ gamma_p,
                                                   int8_t *__restrict__ T)
{
    const float gamma = *gamma_p;
    const bool ok = gamma > 0.0f && gamma <= 3.4028234663852886e38f;
    const double thr = static_cast<double>(gamma) * (1.0 + 0x1p-24);
    for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
        for (int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; k < K;
             k += static_cast<int64_t>(gridDim.x) * 256) {
            float w = W[n * ldw + k];
            int8_t t = 0;
            if (ok && 2.0 * static_cast<double>(fabsf(w)) > thr) t = w > 0.0f ? 1 : -1;
            T[n * K + k] = t;
        }
    }
}

// Binary weights (the predecessor variant, weights -1 or +1): T = +1 where
// w >= 0 (including -0), -1 where w < 0.
__global__ __launch_bounds__(256) void k_binarize(const float *__restrict__ W, int64_t N, int64_t K, int64_t ldw,
                                                  int8_t *__restrict__ T)
{
    for (int64_t n = blockIdx.y; n < N; n += gridDim.y)
        for (int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; k < K;
             k += static_cast<int64_t>(gridDim.x) * 256)
            T[n * K + k] = W[n * ldw + k] >= 0.0f ? 1 : -1;
}

// i2 packing: one thread per (row n, k-block kb) writes one 16-byte chunk.
// Consecutive threads write consecutive chunks of a tile.
__global__ __launch_bounds__(256) void k_pack_i2(const int8_t *__restrict__ T, int64_t N, int64_t K,
                                                 int64_t ldt, int64_t KB, int64_t nchunks,
                                                 uint8_t *__restrict__ P)
{
    int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= nchunks) return;
    int64_t tile = idx / (KB * 16);
    int64_t rem = idx % (KB * 16);
    int64_t kb = rem / 16, r = rem % 16;
    int64_t n = tile * 16 + r;
    uint32_t word[4];
    for (int d = 0; d < 4; ++d) {
        uint32_t w = 0;
        for (int s = 0; s < 4; ++s)
            for (int j = 0; j < 4; ++j) {
                int64_t k = kb * 64 + 16 * d + 4 * s + j;
                int v = (n < N && k < K) ? T[n * ldt + k] : 0;
                w |= static_cast<uint32_t>(v + 1) << (8 * j + 2 * s);
            }
        word[d] = w;
    }
    uint4 out = make_uint4(word[0], word[1], word[2], word[3]);
    *reinterpret_cast<uint4 *>(P + idx * 16) = out;
}

// b3 packing: one thread per (row n, 80-weight block kb); byte i holds
// weights 16t + i (t = 0..4) of the block as the base-3 number v (t = 0 most
// significant), stored as ceil(256 v / 243) (see b3_word_digits).
__global__ __launch_bounds__(256) void k_pack_b3(const int8_t *__restrict__ T, int64_t N, int64_t K,
                                                 int64_t ldt, int64_t KB, int64_t nchunks,
                                                 uint8_t *__restrict__ P)
{
    int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= nchunks) return;
    int64_t tile = idx / (KB * 16);
    int64_t rem = idx % (KB * 16);
    int64_t kb = rem / 16, r = rem % 16;
    int64_t n = tile * 16 + r;
    uint32_t word[4] = {0, 0, 0, 0};
    for (int i = 0; i < 16; ++i) {
        uint32_t b = 0;
        for (int t = 0; t < 5; ++t) {
            int64_t k = kb * 80 + 16 * t + i;
            int v = (n < N && k < K) ? T[n * ldt + k] : 0;
            b = b * 3u + static_cast<uint32_t>(v + 1);
        }
        word[i / 4] |= b3_encode(b) << (8 * (i % 4));
    }
    *reinterpret_cast<uint4 *>(P + idx * 16) = make_uint4(word[0], word[1], word[2], word[3]);
}

// b3 -> i2 transcode (a load-time step).  One thread per b3 chunk
// (row r of tile, block kb3: weights 80 kb3 .. +79).  Digit t of its 16 bytes
// is the 16 weights k0 = 80 kb3 + 16 t .. k0+15, which is exactly i2 word
// d = (k0 % 64) / 16 of i2 block kb2 = k0 / 64 (80 and 64 are multiples of
// 16): the thread decodes the chunk once and writes five i2 words.  i2 words
// past the b3 blocks (only when 64 * KB2 > 80 * KB3) are padding, T = 0; the
// thread of the row's last b3 chunk writes them.
__global__ __launch_bounds__(256) void k_b3_to_i2(const uint8_t *__restrict__ P3, int64_t KB3, int64_t KB2,
                                                  int64_t nchunks, uint8_t *__restrict__ P2)
{
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; // (tile * KB3 + kb3) * 16 + r
    if (idx >= nchunks) return;
    const int64_t r = idx & 15, tk = idx >> 4;
    const int64_t tile = tk / KB3, kb3 = tk - tile * KB3;
    const uint4 c = *reinterpret_cast<const uint4 *>(P3 + idx * 16);
    const uint32_t bw[4] = {c.x, c.y, c.z, c.w};
    // word t: byte i = 4q + j of the chunk (weight k0 + i) at bits 8j + 2q
    uint32_t out[5] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const B3Digits dg = b3_word_digits(bw[q]); // byte j of dg.d[t]: digit t of byte 4q + j
#pragma unroll
        for (int t = 0; t < 5; ++t) out[t] |= dg.d[t] << (2 * q);
    }
    uint32_t *row = reinterpret_cast<uint32_t *>(P2) + tile * KB2 * 64 + r * 4; // word (kb2, d) at kb2 * 64 + d
#pragma unroll
    for (int t = 0; t < 5; ++t) {
        const int64_t k0 = kb3 * 80 + 16 * t;
        if (k0 < KB2 * 64) row[(k0 >> 6) * 64 + ((k0 >> 4) & 3)] = out[t];
    }
    if (kb3 == KB3 - 1)
        for (int64_t k0 = KB3 * 80; k0 < KB2 * 64; k0 += 16) row[(k0 >> 6) * 64 + ((k0 >> 4) & 3)] = I2_ZERO_WORD;
}

hipError_t launch_b3_to_i2(const uint8_t *P3, int64_t N, int64_t K, uint8_t *P2, hipStream_t stream)
{
    const int64_t NT = (N + 15) / 16, KB3 = (K + 79) / 80, KB2 = (K + 63) / 64;
    const int64_t nchunks = NT * KB3 * 16;
    hipLaunchKernelGGL(k_b3_to_i2, dim3(static_cast<unsigned>((nchunks + 255) / 256)), dim3(256), 0, stream, P3,
                       KB3, KB2, nchunks, P2);
    return hipGetLastError();
}

// b1 packing: one thread per (row n, 128-weight block kb); word d holds
// weights kb*128 + 32d + 4s + j at bit 8j + s (1 for T > 0, else 0); bits
// past K or N are 0.
__global__ __launch_bounds__(256) void k_pack_b1(const int8_t *__restrict__ T, int64_t N, int64_t K,
                                                 int64_t ldt, int64_t KB, int64_t nchunks,
                                                 uint8_t *__restrict__ P)
{
    int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= nchunks) return;
    int64_t tile = idx / (KB * 16);
    int64_t rem = idx % (KB * 16);
    int64_t kb = rem / 16, r = rem % 16;
    int64_t n = tile * 16 + r;
    uint32_t word[4];
    for (int d = 0; d < 4; ++d) {
        uint32_t w = 0;
        for (int s = 0; s < 8; ++s)
            for (int j = 0; j < 4; ++j) {
                int64_t k = kb * 128 + 32 * d + 4 * s + j;
                if (n < N && k < K && T[n * ldt + k] > 0) w |= 1u << (8 * j + s);
            }
        word[d] = w;
    }
    *reinterpret_cast<uint4 *>(P + idx * 16) = make_uint4(word[0], word[1], word[2], word[3]);
}

// b1 -> i2 transcode (a load-time step): one thread per i2 word, 16 weights
// k0 .. k0+15 (k0 = 64 kb2 + 16 d).  They are half h = (k0 % 32) / 16 of b1
// word q = (k0 % 128) / 32 of block k0 / 128: weight 4s + j of the i2 word is
// bit 8j + 4h + s of that b1 word, and its code is 2 (T = +1) or 0 (T = -1).
// Positions at or past K and rows at or past N become code 1 (T = 0): binary
// padding carries a weight, i2 padding must not, so the result is byte for
// byte the i2 packing of the same weights.
__global__ __launch_bounds__(256) void k_b1_to_i2(const uint8_t *__restrict__ P1, int64_t KB1, int64_t KB2,
                                                  int64_t N, int64_t K, int64_t nwords, uint8_t *__restrict__ P2)
{
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; // ((tile*KB2 + kb2)*16 + r)*4 + d
    if (idx >= nwords) return;
    const int d = static_cast<int>(idx & 3);
    const int64_t chunk = idx >> 2, r = chunk & 15, tk = chunk >> 4;
    const int64_t tile = tk / KB2, kb2 = tk - tile * KB2;
    const int64_t k0 = kb2 * 64 + 16 * d;
    const int64_t kb1 = k0 >> 7;
    const int q = static_cast<int>((k0 >> 5) & 3), h = static_cast<int>((k0 >> 4) & 1);
    const uint32_t w = reinterpret_cast<const uint32_t *>(P1)[((tile * KB1 + kb1) * 16 + r) * 4 + q];
    uint32_t out = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) out |= ((w >> (4 * h + s)) & 0x01010101u) << (2 * s + 1); // code 2 or 0
    if (k0 + 16 > K) { // the block straddles K: positions past it become T = 0 (code 1)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (k0 + e >= K) {
                const int sh = 8 * (e % 4) + 2 * (e / 4);
                out = (out & ~(3u << sh)) | (1u << sh);
            }
    }
    if (tile * 16 + r >= N) out = 0x55555555u; // a padding row
    reinterpret_cast<uint32_t *>(P2)[idx] = out;
}

hipError_t launch_b1_to_i2(const uint8_t *P1, int64_t N, int64_t K, uint8_t *P2, hipStream_t stream)
{
    const int64_t NT = (N + 15) / 16, KB1 = (K + 127) / 128, KB2 = (K + 63) / 64;
    const int64_t nwords = NT * KB2 * 16 * 4;
    hipLaunchKernelGGL(k_b1_to_i2, dim3(static_cast<unsigned>((nwords + 255) / 256)), dim3(256), 0, stream, P1, KB1,
                       KB2, N, K, nwords, P2);
    return hipGetLastError();
}

static unsigned grid_rows(int64_t N) { return static_cast<unsigned>(N < 65535 ? N : 65535); }

// gamma = mean|W| (exact, one rounding): bucket sums, then one wave finishes.
static void launch_absmean(const float *W, int64_t N, int64_t K, int64_t ldw, float *gamma, void *ws,
                           hipStream_t stream)
{
    unsigned long long *buckets = static_cast<unsigned long long *>(ws);
    hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(256), 0, stream, buckets, 256);
    // enough workgroups to cover the chip; each covers a k-range of many rows
    int64_t kchunks = (K + 1023) / 1024;
    unsigned gx = static_cast<unsigned>(kchunks < 64 ? kchunks : 64);
    int64_t want_rows = (2048 + gx - 1) / gx;
    unsigned gy = static_cast<unsigned>(N < want_rows ? N : want_rows);
    hipLaunchKernelGGL(k_abs_buckets, dim3(gx, gy), dim3(256), 0, stream, W, N, K, ldw, buckets);
    hipLaunchKernelGGL(k_gamma_finalize, dim3(1), dim3(64), 0, stream, buckets, N * K, gamma);
}

static dim3 elementwise_grid(int64_t N, int64_t K)
{
    int64_t kb = (K + 255) / 256;
    return dim3(static_cast<unsigned>(kb < 1024 ? kb : 1024), grid_rows(N));
}

hipError_t launch_quantize_weights(const float *W, int64_t N, int64_t K, int64_t ldw, int8_t *T, float *gamma,
                                   void *ws, hipStream_t stream)
{
    launch_absmean(W, N, K, ldw, gamma, ws, stream);
    hipLaunchKernelGGL(k_ternarize, elementwise_grid(N, K), dim3(256), 0, stream, W, N, K, ldw, gamma, T);
    return hipGetLastError();
}

hipError_t launch_binarize_weights(const float *W, int64_t N, int64_t K, int64_t ldw, int8_t *T, float *gamma,
                                   void *ws, hipStream_t stream)
{
    launch_absmean(W, N, K, ldw, gamma, ws, stream);
    hipLaunchKernelGGL(k_binarize, elementwise_grid(N, K), dim3(256), 0, stream, W, N, K, ldw, T);
    return hipGetLastError();
}

hipError_t launch_pack(const int8_t *T, int64_t N, int64_t K, int64_t ldt, int layout, uint8_t *P,
                       hipStream_t stream)
{
    int64_t NT = (N + 15) / 16;
    int64_t KB = layout == LAYOUT_I2 ? (K + 63) / 64 : (layout == LAYOUT_B3 ? (K + 79) / 80 : (K + 127) / 128);
    int64_t nchunks = NT * KB * 16;
    unsigned blocks = static_cast<unsigned>((nchunks + 255) / 256);
    if (layout == LAYOUT_I2)
        hipLaunchKernelGGL(k_pack_i2, dim3(blocks), dim3(256), 0, stream, T, N, K, ldt, KB, nchunks, P);
    else if (layout == LAYOUT_B3)
        hipLaunchKernelGGL(k_pack_b3, dim3(blocks), dim3(256), 0, stream, T, N, K, ldt, KB, nchunks, P);
    else
        hipLaunchKernelGGL(k_pack_b1, dim3(blocks), dim3(256), 0, stream, T, N, K, ldt, KB, nchunks, P);
    return hipGetLastError();
}

} // namespace bl
