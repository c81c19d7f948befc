// gemv.hip -- the decode product acc[m][n] = sum_k q[m][k] * T[n][k] for a few
// tokens, followed by the rescale y = float(acc) * (gamma * beta_m) / 127.
//
// LIT-380 record (dmarx anthology), Key takeaways, bullet 4: with ternary
// weights the product needs only additions and subtractions.  The same
// record's closing section notes that on stock GPUs the memory saving is what
// survives: this path streams 2 bits per weight from HBM and is bound by it.
//
// Two kernels:
//  * k_gemv_addsub: vector-ALU add/subtract.  A lane owns one weight row; the
//    activation words are wave-uniform (scalar registers).  The offset code
//    c = T + 1 in {0, 1, 2} goes through v_dot4_i32_i8: sum_k c*q adds q where
//    T = 0, adds 2q where T = +1, adds nothing where T = -1; subtracting
//    sum_k q afterwards leaves sum_{T=+1} q - sum_{T=-1} q exactly.
//  * k_gemv_mfma: tiles of 16 tokens x 16 rows x 64 weights on the int8 matrix
//    cores, weights unpacked in registers to signed bytes.  Used where the
//    vector ALU cannot keep up with HBM (more than a few tokens).
#include "common.h"
#include "launch.h"

namespace bl {

// 16 int8 activations q[m][k0 .. k0+15] as one MFMA operand; zero outside
// [0, M) x [0, K).  Rows of Xq are 16-byte aligned and k0 % 16 == 0.
__device__ __forceinline__ v4i load_a16(const int8_t *__restrict__ Xq, int64_t ldq, int64_t m, int64_t M,
                                        int64_t K, int64_t k0)
{
    v4i r = {0, 0, 0, 0};
    if (m >= M || k0 >= K) return r;
    const int8_t *p = Xq + m * ldq + k0;
    if (k0 + 16 <= K) return *reinterpret_cast<const v4i *>(p);
    uint32_t w[4] = {0, 0, 0, 0};
    for (int j = 0; j < 16; ++j)
        if (k0 + j < K) w[j / 4] |= (static_cast<uint32_t>(p[j]) & 0xffu) << (8 * (j % 4));
    r[0] = static_cast<int>(w[0]);
    r[1] = static_cast<int>(w[1]);
    r[2] = static_cast<int>(w[2]);
    r[3] = static_cast<int>(w[3]);
    return r;
}

// ---------------------------------------------------------------------------
// MFMA GEMV: one workgroup = one 16-row tile x one group of 16 tokens; its four
// waves take the k-steps (4 k-blocks = 256 weights) round-robin and reduce
// through LDS.  In a k-step, lane l (i = l % 16, g = l / 16) loads the 16-byte
// chunk of row 16*tile + i at k-block 4*step + g; MFMA number d (i2: word d,
// 16 weights; b3: base-3 digit d of the 16 bytes) pairs it with the matching
// 16 activations of token i.
// ---------------------------------------------------------------------------
template <int LAYOUT>
__global__ __launch_bounds__(256) void k_gemv_mfma(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                   const float *__restrict__ gamma_p,
                                                   const int8_t *__restrict__ Xq, int64_t ldq,
                                                   const float *__restrict__ beta, int64_t M, int64_t N,
                                                   int64_t K, void *__restrict__ Y, int y_dtype, int64_t ldy)
{
    __shared__ v4i red[4][64];
    const int wave = wave_id(), lane = lane_id();
    const int i = lane & 15, g = lane >> 4;
    const int64_t tile = blockIdx.x;
    const int64_t m = static_cast<int64_t>(blockIdx.y) * 16 + i; // token of the A operand
    const uint8_t *ptile = P + tile * KB * 256;
    const int64_t nsteps = (KB + 3) / 4;
    v4i acc = {0, 0, 0, 0};
    for (int64_t s = wave; s < nsteps; s += 4) {
        const int64_t kb = 4 * s + g;
        if constexpr (LAYOUT == LAYOUT_I2) {
            uint4 w = make_uint4(I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD);
            if (kb < KB) w = *reinterpret_cast<const uint4 *>(ptile + kb * 256 + i * 16);
            const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                v4i a = load_a16(Xq, ldq, m, M, K, kb * 64 + 16 * d);
                v4i b = i2_word_to_signed16(wd[d]);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
            }
        } else {
            uint4 w = make_uint4(0x79797979u, 0x79797979u, 0x79797979u, 0x79797979u); // 121 = all T = 0
            if (kb < KB) w = *reinterpret_cast<const uint4 *>(ptile + kb * 256 + i * 16);
            const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
            // digit t of byte j holds weight kb*80 + 5j + t
#pragma unroll
            for (int t = 0; t < 5; ++t) {
                uint32_t bw[4] = {0, 0, 0, 0}, aw[4] = {0, 0, 0, 0};
                const uint32_t div = t == 0 ? 81u : t == 1 ? 27u : t == 2 ? 9u : t == 3 ? 3u : 1u;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    uint32_t byte = (wd[j / 4] >> (8 * (j % 4))) & 0xffu;
                    uint32_t digit = (byte / div) % 3u;
                    bw[j / 4] |= ((digit + 0xffu) & 0xffu) << (8 * (j % 4)); // digit - 1 as a byte
                    int64_t k = kb * 80 + 5 * j + t;
                    if (m < M && k < K)
                        aw[j / 4] |= (static_cast<uint32_t>(Xq[m * ldq + k]) & 0xffu) << (8 * (j % 4));
                }
                v4i a = {static_cast<int>(aw[0]), static_cast<int>(aw[1]), static_cast<int>(aw[2]),
                         static_cast<int>(aw[3])};
                v4i b = {static_cast<int>(bw[0]), static_cast<int>(bw[1]), static_cast<int>(bw[2]),
                         static_cast<int>(bw[3])};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
            }
        }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    v4i tot = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
    // D layout: lane l holds rows (tokens) 4g + r, column (weight row) i.
    const float gamma = *gamma_p;
    const int64_t n = tile * 16 + i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t mm = static_cast<int64_t>(blockIdx.y) * 16 + 4 * g + r;
        if (mm < M && n < N) store_out(Y, y_dtype, ldy, mm, n, tot[r], token_scale(gamma, beta[mm]));
    }
}

// ---------------------------------------------------------------------------
// Add/subtract GEMV: one workgroup = 64 weight rows (4 tiles), lane l owns row
// 16*(4*blockIdx.x + l/16) + l%16; wave w takes k-blocks w, w+4, ...  For a
// k-block the 16 code words of the lane's row are formed once and dotted with
// the 16 activation words of each token (the same for the whole wave).
// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(256) void k_gemv_addsub(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                     const float *__restrict__ gamma_p,
                                                     const int8_t *__restrict__ Xq, int64_t ldq,
                                                     const float *__restrict__ beta, int64_t M, int64_t N,
                                                     int64_t K, void *__restrict__ Y, int y_dtype, int64_t ldy)
{
    __shared__ int red[4][MT][64];
    __shared__ int qsum_part[4][MT];
    const int wave = wave_id(), lane = lane_id();
    const int64_t tile = 4 * static_cast<int64_t>(blockIdx.x) + (lane >> 4);
    const int r = lane & 15;

    // sum_k q[m][k] for the correction of the offset codes
    {
        int part[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) part[t] = 0;
        const int64_t nwords = (K + 3) / 4;
        for (int64_t wi = threadIdx.x; wi < nwords; wi += 256) {
            const int64_t k = 4 * wi;
#pragma unroll
            for (int t = 0; t < MT; ++t)
                if (t < M) {
                    const int8_t *qp = Xq + t * ldq + k;
                    uint32_t wq = 0;
                    if (k + 4 <= K) {
                        wq = *reinterpret_cast<const uint32_t *>(qp);
                    } else {
                        for (int j = 0; k + j < K; ++j) wq |= (static_cast<uint32_t>(qp[j]) & 0xffu) << (8 * j);
                    }
                    part[t] = __builtin_amdgcn_sdot4(static_cast<int>(wq), 0x01010101, part[t], false);
                }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            int v = part[t];
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) qsum_part[wave][t] = v;
        }
    }

    int acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0;
    const int64_t KBF = K / 64; // k-blocks whose 64 activations are all in range
    for (int64_t kb = wave; kb < KB; kb += 4) {
        uint4 w = make_uint4(I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD);
        if (tile < NT) w = *reinterpret_cast<const uint4 *>(P + (tile * KB + kb) * 256 + r * 16);
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
        uint32_t c[16];
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int s = 0; s < 4; ++s) c[4 * d + s] = (wd[d] >> (2 * s)) & 0x03030303u;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t >= M) break;
            const int8_t *qp = Xq + t * ldq + kb * 64;
            uint32_t qd[16];
            if (kb < KBF) {
                const uint4 *q4 = reinterpret_cast<const uint4 *>(qp);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    uint4 x = q4[v];
                    qd[4 * v] = x.x; qd[4 * v + 1] = x.y; qd[4 * v + 2] = x.z; qd[4 * v + 3] = x.w;
                }
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    uint32_t word = 0;
                    for (int j = 0; j < 4; ++j) {
                        int64_t k = kb * 64 + 4 * v + j;
                        if (k < K) word |= (static_cast<uint32_t>(qp[4 * v + j]) & 0xffu) << (8 * j);
                    }
                    qd[v] = word;
                }
            }
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[t] = __builtin_amdgcn_sdot4(static_cast<int>(c[j]), static_cast<int>(qd[j]), acc[t], false);
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
    const float gamma = *gamma_p;
    const int64_t n = tile * 16 + r;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t >= M) break;
        int total = red[0][t][lane] + red[1][t][lane] + red[2][t][lane] + red[3][t][lane];
        int qs = qsum_part[0][t] + qsum_part[1][t] + qsum_part[2][t] + qsum_part[3][t];
        if (n < N) store_out(Y, y_dtype, ldy, t, n, total - qs, token_scale(gamma, beta[t]));
    }
}

hipError_t launch_gemv_mfma(const GemvArgs &a, hipStream_t stream)
{
    const int64_t NT = (a.N + 15) / 16;
    const int64_t KB = a.layout == LAYOUT_I2 ? (a.K + 63) / 64 : (a.K + 79) / 80;
    dim3 grid(static_cast<unsigned>(NT), static_cast<unsigned>((a.M + 15) / 16));
    if (a.layout == LAYOUT_I2)
        hipLaunchKernelGGL(k_gemv_mfma<LAYOUT_I2>, grid, dim3(256), 0, stream, a.P, KB, NT, a.gamma, a.Xq, a.ldq,
                           a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy);
    else
        hipLaunchKernelGGL(k_gemv_mfma<LAYOUT_B3>, grid, dim3(256), 0, stream, a.P, KB, NT, a.gamma, a.Xq, a.ldq,
                           a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy);
    return hipGetLastError();
}

template <int MT>
static void launch_addsub_mt(const GemvArgs &a, int64_t KB, int64_t NT, hipStream_t stream)
{
    dim3 grid(static_cast<unsigned>((NT + 3) / 4));
    hipLaunchKernelGGL(k_gemv_addsub<MT>, grid, dim3(256), 0, stream, a.P, KB, NT, a.gamma, a.Xq, a.ldq, a.beta,
                       a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy);
}

hipError_t launch_gemv_addsub(const GemvArgs &a, hipStream_t stream)
{
    const int64_t NT = (a.N + 15) / 16;
    const int64_t KB = (a.K + 63) / 64;
    if (a.M <= 1) launch_addsub_mt<1>(a, KB, NT, stream);
    else if (a.M <= 2) launch_addsub_mt<2>(a, KB, NT, stream);
    else if (a.M <= 4) launch_addsub_mt<4>(a, KB, NT, stream);
    else if (a.M <= 8) launch_addsub_mt<8>(a, KB, NT, stream);
    else launch_addsub_mt<16>(a, KB, NT, stream);
    return hipGetLastError();
}

} // namespace bl
