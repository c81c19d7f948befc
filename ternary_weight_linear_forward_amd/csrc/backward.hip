// backward.hip -- gradients of a BitLinear layer under the straight-through
// estimator.
//
// The pages quote the BitNet paper: training uses the straight-through
// estimator, which lets the gradient bypass the non-differentiable functions
// (HackerPapers digest, comment quoting the BitNet paper on the
// straight-through estimator).  Reading: the rounding and clipping of both
// quantisers have derivative 1 and their scales (gamma, beta_m) are
// constants, so the layer acts like y = Xhat @ What^T with What = gamma * T
// and Xhat[m][k] = q[m][k] * (beta_m / 127), and
//     dX = dY @ What = gamma * (dY @ T)        [M x K]
//     dW = dY^T @ Xhat                          [N x K]  (latent weights)
// Both are fp32 contractions, run as v_mfma_f32_16x16x4f32 with fp32
// accumulation.  T comes straight from the i2-packed weights of the forward.
#include "common.h"
#include "launch.h"

namespace bl {

typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// dX = gamma * dY @ T.  Workgroup: one token group (16 tokens, blockIdx.y)
// and one 64-column k-block (blockIdx.x); its W waves split the N row tiles
// (wave w takes tiles w, w+W, ...).  For a 16-row tile the wave multiplies
// 4 row groups x 4 column groups: A = dY[16 tokens x 4 rows] (lane l: token
// l%16, row l/16), B = T[4 rows x 16 columns] (lane l: row l/16, column
// l%16, decoded from the packed word), D = dX[16 tokens x 16 columns] per
// column group.  The W partial tiles meet in LDS; wave d stores column
// group d, scaled by gamma.
// ---------------------------------------------------------------------------
constexpr int DX_MAX_WAVES = 8;

__global__ __launch_bounds__(64 * DX_MAX_WAVES) void k_bwd_dx(const uint8_t *__restrict__ P, int64_t KB,
                                                             int64_t NT, const float *__restrict__ gamma_p,
                                                             const float *__restrict__ dY, int64_t lddy, int64_t M,
                                                             int64_t N, int64_t K, float *__restrict__ dX,
                                                             int64_t lddx)
{
    __shared__ v4f red[DX_MAX_WAVES][4][64];
    const int nw = blockDim.x >> 6;
    const int wave = wave_id(), lane = lane_id();
    const int li = lane & 15, lg = lane >> 4;
    const int64_t kb = blockIdx.x;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 16;
    const int64_t ma = m0 + li; // token of this lane's A element
    const bool mvalid = ma < M;
    const float *dyrow = dY + (mvalid ? ma : 0) * lddy;
    // column 16d + li of a chunk word d: li = 4s + j sits at bits 8j + 2s
    const int sh = 8 * (li & 3) + 2 * (li >> 2);

    v4f acc[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) acc[d] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t tile = wave; tile < NT; tile += nw) {
        const uint8_t *cb = P + (tile * KB + kb) * 256;
        uint4 ch[4];
        float a[4];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            ch[rg] = *reinterpret_cast<const uint4 *>(cb + (4 * rg + lg) * 16);
            const int64_t n = tile * 16 + 4 * rg + lg;
            a[rg] = (mvalid && n < N) ? dyrow[n] : 0.0f;
        }
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const uint32_t w[4] = {ch[rg].x, ch[rg].y, ch[rg].z, ch[rg].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const float b = static_cast<float>(static_cast<int>((w[d] >> sh) & 3u) - 1);
                acc[d] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rg], b, acc[d], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) red[wave][d][lane] = acc[d];
    __syncthreads();
    const float gamma = *gamma_p;
    // D layout: lane l holds tokens 4 * (l/16) + r, column l%16 of the group
    for (int d = wave; d < 4; d += nw) {
        v4f tot = red[0][d][lane];
        for (int w = 1; w < nw; ++w) tot += red[w][d][lane];
        const int64_t k = kb * 64 + 16 * d + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + 4 * lg + r;
            if (m < M && k < K) dX[m * lddx + k] = gamma * tot[r];
        }
    }
}

// ---------------------------------------------------------------------------
// dW = dY^T @ Xhat.  Workgroup: 64 rows n x 64 columns k of dW, 4 waves of
// 32 x 32 (2 x 2 MFMA tiles); the contraction runs over the tokens, 4 per
// MFMA, 4 MFMA k-steps (16 tokens) per loop trip with all their loads issued
// first.  A = dY^T[16 rows x 4 tokens] (lane l: row l%16, token l/16),
// B = Xhat[4 tokens x 16 columns] (lane l: token l/16, column l%16), with
// Xhat = float(q) * r_m and r_m = beta_m / 127 rounded to binary32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_dw(const int8_t *__restrict__ Xq, int64_t ldq,
                                               const float *__restrict__ beta, const float *__restrict__ dY,
                                               int64_t lddy, int64_t M, int64_t N, int64_t K, float *__restrict__ dW,
                                               int64_t lddw)
{
    constexpr int U = 4; // MFMA k-steps (of 4 tokens) per trip
    const int wave = wave_id(), lane = lane_id();
    const int li = lane & 15, lg = lane >> 4;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * 64 + (wave >> 1) * 32;
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * 64 + (wave & 1) * 32;
    int64_t nn[2], kk[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        nn[i] = n0 + 16 * i + li;
        kk[i] = k0 + 16 * i + li;
    }
    v4f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t mb = 0; mb < M; mb += 4 * U) {
        float a[U][2], b[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t m = mb + 4 * u + lg;
            const bool mv = m < M;
            const int64_t mc = mv ? m : 0;
            const float r = mv ? beta[mc] / 127.0f : 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i) a[u][i] = (mv && nn[i] < N) ? dY[mc * lddy + nn[i]] : 0.0f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[u][j] = (mv && kk[j] < K) ? static_cast<float>(Xq[mc * ldq + kk[j]]) * r : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][i], b[u][j], acc[i][j], 0, 0, 0);
    }
    // D layout: lane l holds rows 4 * (l/16) + r, column l%16 of the tile
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n0 + 16 * i + 4 * lg + r;
            if (n >= N) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (kk[j] < K) dW[n * lddw + kk[j]] = acc[i][j][r];
        }
}

hipError_t launch_bwd_dx(const uint8_t *P2, const float *gamma, int64_t M, int64_t N, int64_t K, const float *dY,
                         int64_t lddy, float *dX, int64_t lddx, hipStream_t stream)
{
    const int64_t NT = (N + 15) / 16, KB = (K + 63) / 64;
    const int64_t nw = NT < DX_MAX_WAVES ? NT : DX_MAX_WAVES;
    dim3 grid(static_cast<unsigned>(KB), static_cast<unsigned>((M + 15) / 16));
    hipLaunchKernelGGL(k_bwd_dx, grid, dim3(static_cast<unsigned>(64 * nw)), 0, stream, P2, KB, NT, gamma, dY, lddy,
                       M, N, K, dX, lddx);
    return hipGetLastError();
}

hipError_t launch_bwd_dw(const int8_t *Xq, int64_t ldq, const float *beta, int64_t M, int64_t N, int64_t K,
                         const float *dY, int64_t lddy, float *dW, int64_t lddw, hipStream_t stream)
{
    dim3 grid(static_cast<unsigned>((K + 63) / 64), static_cast<unsigned>((N + 63) / 64));
    hipLaunchKernelGGL(k_bwd_dw, grid, dim3(256), 0, stream, Xq, ldq, beta, dY, lddy, M, N, K, dW, lddw);
    return hipGetLastError();
}

} // namespace bl
