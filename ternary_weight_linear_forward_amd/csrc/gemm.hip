// gemm.hip -- the prefill product for many tokens on the int8 matrix cores.
//
// At large M the BitLinear product (LIT-380 record, Key takeaways, bullet 4:
// integer additions of activations selected by ternary weights) is a dense
// contraction whose arithmetic, not HBM, is the bound: every packed weight is
// used by thousands of tokens.  So the ternary weights are unpacked once per
// workgroup into signed int8 tiles in LDS and multiplied with int8 activation
// tiles by v_mfma_i32_32x32x32_i8.  The epilogue applies
// y = float(acc) * (gamma * beta_m) / 127.
//
// Workgroup tile BM tokens x 128 weight rows, 4 waves in a 2 x 2 grid, each
// (BM/2) x 64 = (BM/64) x 2 MFMA tiles of 32 x 32.  Per stage 128 weights of
// k (two k-blocks): the activation tile (BM x 128 bytes) and the unpacked
// weight tile (128 x 128 bytes) sit in LDS, double-buffered, one barrier per
// stage; global loads run one stage ahead in registers.  LDS rows are padded
// to 144 bytes so that the 16-byte operand reads of a wave hit distinct banks.
#include "common.h"
#include "launch.h"

namespace bl {

namespace {
constexpr int BN = 128;       // weight rows per workgroup (8 tiles of 16)
constexpr int KSTEP = 128;    // k per LDS stage: two 64-weight k-blocks
constexpr int LDS_ROW = 144;  // 128 bytes of k + 16 bytes of padding
typedef int v16i __attribute__((ext_vector_type(16)));
} // namespace

__device__ __forceinline__ v4i gemm_i2_word_signed(uint32_t w)
{
    v4i r;
    r[0] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, w & 0x03030303u));
    r[1] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, (w >> 2) & 0x03030303u));
    r[2] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, (w >> 4) & 0x03030303u));
    r[3] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, (w >> 6) & 0x03030303u));
    return r;
}

template <int BM, int S>
__global__ __launch_bounds__(256) void k_gemm_mfma_i2(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                      const float *__restrict__ gamma_p,
                                                      const int8_t *__restrict__ Xq, int64_t ldq,
                                                      const float *__restrict__ beta, int64_t M, int64_t N,
                                                      int64_t K, void *__restrict__ Y, int y_dtype, int64_t ldy)
{
    constexpr int MI = BM / 64;             // 32-row MFMA tiles per wave along M
    constexpr int NI = 2;                   // 32-column MFMA tiles per wave along N
    constexpr int A_LOADS = BM * KSTEP / 16 / 256; // 16-byte activation loads per thread per stage
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * LDS_ROW];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * LDS_ROW];
    __shared__ float scale[BM]; // per-token rescale factors, computed once up front
    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = lane_id();
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, kh = lane >> 5; // operand row/column and 16-byte k half

    // XCD-aware tile order.  Workgroup ids are dealt round-robin to the 8 XCDs
    // (each with its own L2), so id L runs on XCD L % 8.  Tiles are numbered
    // M-block-major (t = mb * nN + nb) and XCD x takes the contiguous range of
    // tile numbers [x * W/8, (x+1) * W/8): the workgroups sharing an XCD work on
    // the same activation rows and find them in that XCD's L2.
    const int64_t nN = gridDim.x, W = static_cast<int64_t>(gridDim.x) * gridDim.y;
    const int64_t L = blockIdx.x + static_cast<int64_t>(gridDim.x) * blockIdx.y;
    int64_t t;
    {
        const int64_t per = W / 8, rem = W % 8, x = L % 8, j = L / 8;
        // XCDs 0 .. rem-1 own per+1 tiles, the others per
        t = x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
    }
    const int64_t m0 = (t / nN) * BM;
    const int64_t n0 = (t % nN) * BN;
    const int64_t nstages = (KB + 1) / 2;

    // Per-thread load sources, computed once.  Activation piece r of a stage:
    // row (tid + 256 r) / 8, 16-byte column (tid % 8).  Rows past M read row
    // M - 1 and pieces that start at or past K read offset 0: the products they
    // feed are discarded or meet packed weights that are 0 (columns past K
    // carry T = 0), so only the addresses need to be valid; a piece straddling
    // K reads up to round_up(K, 16) <= ldq.
    const int8_t *a_row[A_LOADS];
#pragma unroll
    for (int r = 0; r < A_LOADS; ++r) {
        const int64_t m = m0 + ((tid + 256 * r) >> 3);
        a_row[r] = Xq + (m < M ? m : M - 1) * ldq;
    }
    const int a_col = (tid & 7) * 16;
    // weight chunk of this thread: row tid % 128 of the tile group, k-block 2 * stage + tid / 128;
    // tiles past NT read tile NT - 1 (their outputs are never stored)
    const int64_t b_n = n0 + (tid & 127);
    const int64_t b_tile = b_n / 16 < NT ? b_n / 16 : NT - 1;
    const uint8_t *b_ptr = P + (b_tile * KB) * 256 + (b_n % 16) * 16;
    const int b_half = tid >> 7;

    v4i a_st[S][A_LOADS];
    uint4 b_st[S];
    // Every call issues the same unconditional loads, so the waits before each
    // use only need the oldest stage.  A k-block past KB reads the last one and
    // is replaced by zero weights.
    auto gload = [&](int64_t stg, v4i (&as)[A_LOADS], uint4 &bs) {
        stg = stg < nstages ? stg : nstages - 1;
        const int64_t kc = stg * KSTEP + a_col;
        const int64_t ko = kc < K ? kc : 0;
#pragma unroll
        for (int r = 0; r < A_LOADS; ++r) as[r] = *reinterpret_cast<const v4i *>(a_row[r] + ko);
        const int64_t kb = 2 * stg + b_half;
        const uint4 w = *reinterpret_cast<const uint4 *>(b_ptr + (kb < KB ? kb : KB - 1) * 256);
        bs = kb < KB ? w : make_uint4(I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD);
    };
    auto lstore = [&](int buf, const v4i (&as)[A_LOADS], const uint4 &bs) {
#pragma unroll
        for (int r = 0; r < A_LOADS; ++r)
            *reinterpret_cast<v4i *>(&As[buf][((tid + 256 * r) >> 3) * LDS_ROW + a_col]) = as[r];
        int8_t *row = &Bs[buf][(tid & 127) * LDS_ROW + b_half * 64];
        *reinterpret_cast<v4i *>(row + 0) = gemm_i2_word_signed(bs.x);
        *reinterpret_cast<v4i *>(row + 16) = gemm_i2_word_signed(bs.y);
        *reinterpret_cast<v4i *>(row + 32) = gemm_i2_word_signed(bs.z);
        *reinterpret_cast<v4i *>(row + 48) = gemm_i2_word_signed(bs.w);
    };

    v16i acc[MI][NI];
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NI; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    auto compute = [&](int buf) {
        const int8_t *abase = &As[buf][(wm * (BM / 2) + l32) * LDS_ROW + kh * 16];
        const int8_t *bbase = &Bs[buf][(wn * 64 + l32) * LDS_ROW + kh * 16];
#pragma unroll
        for (int kk = 0; kk < KSTEP / 32; ++kk) {
            v4i af[MI], bf[NI];
#pragma unroll
            for (int a = 0; a < MI; ++a) af[a] = *reinterpret_cast<const v4i *>(abase + a * 32 * LDS_ROW + kk * 32);
#pragma unroll
            for (int b = 0; b < NI; ++b) bf[b] = *reinterpret_cast<const v4i *>(bbase + b * 32 * LDS_ROW + kk * 32);
#pragma unroll
            for (int a = 0; a < MI; ++a)
#pragma unroll
                for (int b = 0; b < NI; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
        }
    };

    // the first S - 1 stages are requested up front, stage 0 goes to LDS
#pragma unroll
    for (int j = 0; j < S; ++j)
        if (j < S - 1 || S == 1) gload(j, a_st[j], b_st[j]);
    if (tid < BM) {
        const int64_t m = m0 + tid;
        scale[tid] = m < M ? token_scale(*gamma_p, beta[m]) : 0.0f;
    }
    lstore(0, a_st[0], b_st[0]);
    __syncthreads();
    // Stage st sits in LDS buffer st & 1.  At the start of its iteration the
    // loads of stage st + S - 1 go out (register stage (st + S - 1) % S, free
    // since its last content went to LDS); after the MFMAs of stage st, stage
    // st + 1 (register stage (st + 1) % S, requested S - 1 iterations ago) is
    // written to the other LDS buffer.  With S = 1 the loads of stage st + 1
    // overlap the MFMAs of stage st only.
    for (int64_t st0 = 0; st0 < nstages; st0 += S) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const int64_t st = st0 + j;
            if (st >= nstages) break;
            const int lbuf = static_cast<int>(st & 1);
            if (S == 1) gload(st + 1, a_st[0], b_st[0]);
            else gload(st + S - 1, a_st[(j + S - 1) % S], b_st[(j + S - 1) % S]);
            compute(lbuf);
            lstore(lbuf ^ 1, a_st[(j + 1) % S], b_st[(j + 1) % S]);
            __syncthreads();
        }
    }

    // 32 x 32 output layout: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int lrow = wm * (BM / 2) + a * 32 + 8 * (r / 4) + 4 * kh + (r % 4);
            const int64_t m = m0 + lrow;
            if (m >= M) continue;
            const float sc = scale[lrow];
#pragma unroll
            for (int b = 0; b < NI; ++b) {
                const int64_t n = n0 + wn * 64 + b * 32 + l32;
                if (n < N) store_out(Y, y_dtype, ldy, m, n, acc[a][b][r], sc);
            }
        }
}

hipError_t launch_gemm_mfma(const GemvArgs &a, hipStream_t stream)
{
    const int64_t NT = (a.N + 15) / 16;
    const int64_t KB = (a.K + 63) / 64;
    if (a.M > 128) {
        dim3 grid(static_cast<unsigned>((a.N + BN - 1) / BN), static_cast<unsigned>((a.M + 255) / 256));
        hipLaunchKernelGGL((k_gemm_mfma_i2<256, 1>), grid, dim3(256), 0, stream, a.P, KB, NT, a.gamma, a.Xq, a.ldq,
                           a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy);
    } else {
        dim3 grid(static_cast<unsigned>((a.N + BN - 1) / BN), static_cast<unsigned>((a.M + 127) / 128));
        hipLaunchKernelGGL((k_gemm_mfma_i2<128, 1>), grid, dim3(256), 0, stream, a.P, KB, NT, a.gamma, a.Xq, a.ldq,
                           a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy);
    }
    return hipGetLastError();
}

} // namespace bl
