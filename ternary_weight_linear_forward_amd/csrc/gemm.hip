// gemm.hip -- the prefill product for many tokens on the int8 matrix cores.
//
// At large M the BitLinear product is a dense contraction (LIT-380 record,
// Key takeaways, bullet 4 describes it as integer additions; with thousands of
// tokens per weight the arithmetic, not HBM, is the bound), so the ternary
// weights are unpacked once per workgroup into signed int8 tiles in LDS and
// multiplied with the int8 activation tiles by v_mfma_i32_16x16x64_i8.
// The epilogue applies y = float(acc) * (gamma * beta_m) / 127.
#include "common.h"
#include "launch.h"

namespace bl {

namespace {
constexpr int BM = 128;     // tokens per workgroup
constexpr int BN = 128;     // weight rows per workgroup (8 tiles of 16)
constexpr int LDS_ROW = 80; // 64 bytes of k + 16 bytes of padding (conflict-free 16-byte reads)
} // namespace

__device__ __forceinline__ v4i gemm_load_a16(const int8_t *__restrict__ Xq, int64_t ldq, int64_t m, int64_t M,
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

// Workgroup tile 128 tokens x 128 rows; four waves in a 2 x 2 grid, each
// 64 x 64 = 4 x 4 MFMA tiles.  One k-block (64 weights) per iteration.
__global__ __launch_bounds__(256) void k_gemm_mfma_i2(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                      const float *__restrict__ gamma_p,
                                                      const int8_t *__restrict__ Xq, int64_t ldq,
                                                      const float *__restrict__ beta, int64_t M, int64_t N,
                                                      int64_t K, void *__restrict__ Y, int y_dtype, int64_t ldy)
{
    __shared__ __attribute__((aligned(16))) int8_t As[BM * LDS_ROW];
    __shared__ __attribute__((aligned(16))) int8_t Bs[BN * LDS_ROW];
    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = lane_id();
    const int wm = wave >> 1, wn = wave & 1;
    const int i = lane & 15, g = lane >> 4;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;

    v4i acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = v4i{0, 0, 0, 0};

    for (int64_t kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
            const int idx = tid + 256 * rep;
            const int row = idx >> 2, seg = idx & 3;
            v4i v = gemm_load_a16(Xq, ldq, m0 + row, M, K, kb * 64 + seg * 16);
            *reinterpret_cast<v4i *>(&As[row * LDS_ROW + seg * 16]) = v;
        }
        if (tid < BN) {
            const int64_t n = n0 + tid;
            uint4 w = make_uint4(I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD);
            if (n / 16 < NT) w = *reinterpret_cast<const uint4 *>(P + ((n / 16) * KB + kb) * 256 + (n % 16) * 16);
            *reinterpret_cast<v4i *>(&Bs[tid * LDS_ROW + 0]) = i2_word_to_signed16(w.x);
            *reinterpret_cast<v4i *>(&Bs[tid * LDS_ROW + 16]) = i2_word_to_signed16(w.y);
            *reinterpret_cast<v4i *>(&Bs[tid * LDS_ROW + 32]) = i2_word_to_signed16(w.z);
            *reinterpret_cast<v4i *>(&Bs[tid * LDS_ROW + 48]) = i2_word_to_signed16(w.w);
        }
        __syncthreads();
        v4i af[4], bf[4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
            af[a] = *reinterpret_cast<const v4i *>(&As[(wm * 64 + a * 16 + i) * LDS_ROW + 16 * g]);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            bf[b] = *reinterpret_cast<const v4i *>(&Bs[(wn * 64 + b * 16 + i) * LDS_ROW + 16 * g]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
        __syncthreads();
    }

    const float gamma = *gamma_p;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + wm * 64 + a * 16 + 4 * g + r;
            if (m >= M) continue;
            const float sc = token_scale(gamma, beta[m]);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int64_t n = n0 + wn * 64 + b * 16 + i;
                if (n < N) store_out(Y, y_dtype, ldy, m, n, acc[a][b][r], sc);
            }
        }
}

hipError_t launch_gemm_mfma(const GemvArgs &a, hipStream_t stream)
{
    const int64_t NT = (a.N + 15) / 16;
    const int64_t KB = (a.K + 63) / 64;
    dim3 grid(static_cast<unsigned>((a.N + BN - 1) / BN), static_cast<unsigned>((a.M + BM - 1) / BM));
    hipLaunchKernelGGL(k_gemm_mfma_i2, grid, dim3(256), 0, stream, a.P, KB, NT, a.gamma, a.Xq, a.ldq, a.beta, a.M,
                       a.N, a.K, a.Y, a.y_dtype, a.ldy);
    return hipGetLastError();
}

} // namespace bl
