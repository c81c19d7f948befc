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
// Both gradients are C[p][q] = sum_t A[t][p] B[t][q] over a contraction index
// t, computed by one body: a workgroup owns a 128 x 128 tile of C, 4 waves of
// 64 x 64 (4 x 4 MFMA tiles of 16 x 16, v_mfma_f32_16x16x4f32), and the
// contraction runs in stages of 32.  A stage's A [32 x 128] and B [32 x 128]
// sit in LDS as fp32, double-buffered: each thread fetches its share of
// stage s+1 from global memory into registers before the waves multiply
// stage s, and writes it to the other buffer after.
//   dW[n][k] = sum_m dY[m][n] Xhat[m][k]:   t = token, A = dY, B = Xhat
//   dX[m][k] = gamma sum_n dY[m][n] T[n][k]: t = weight row, A = dY^T, B = T
// MFMA operands: A tile i of a wave takes rows p = wp + 4 li + i (lane l:
// li = l % 16, contraction row l / 16 of the k-step), B tile j columns
// q = wq + 4 li + j, so a lane's four A (and four B) values of a k-step are
// one 16-byte LDS read.  LDS rows are 144 floats apart: the 4 contraction
// rows of a read fall in different banks.
// ---------------------------------------------------------------------------
constexpr int MM_T = 128;  // output tile edge
constexpr int MM_S = 32;   // contraction rows per stage
constexpr int MM_LD = 144; // LDS row stride in floats

template <class Stage>
__device__ __forceinline__ void bwd_mm_body(const Stage &st, float (*sa)[MM_S][MM_LD], float (*sb)[MM_S][MM_LD],
                                            int64_t nst, v4f (&acc)[4][4])
{
    const int wave = wave_id(), lane = lane_id();
    const int li = lane & 15, lg = lane >> 4;
    const int wp = (wave >> 1) * 64, wq = (wave & 1) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    typename Stage::Regs r;
    st.fetch(0, r);
    st.stash(r, sa[0], sb[0]);
    __syncthreads();
    for (int64_t s = 0; s < nst; ++s) {
        const int buf = static_cast<int>(s & 1);
        if (s + 1 < nst) st.fetch(s + 1, r); // in flight during the multiply
#pragma unroll
        for (int ks = 0; ks < MM_S / 4; ++ks) {
            const int t = 4 * ks + lg;
            const float4 a4 = *reinterpret_cast<const float4 *>(&sa[buf][t][wp + 4 * li]);
            const float4 b4 = *reinterpret_cast<const float4 *>(&sb[buf][t][wq + 4 * li]);
            const float a[4] = {a4.x, a4.y, a4.z, a4.w}, b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < nst) st.stash(r, sa[buf ^ 1], sb[buf ^ 1]); // last read two stages ago
        __syncthreads();
    }
}

// Store a 128 x 128 tile: C[p][q] of wave tile (i, j), register r of lane l
// is p = wp + 4 (4 (l / 16) + r) + i, q = wq + 4 (l % 16) + j.
template <class Put>
__device__ __forceinline__ void bwd_mm_store(const v4f (&acc)[4][4], int64_t p0, int64_t q0, int64_t P, int64_t Q, Put put)
{
    const int wave = wave_id(), lane = lane_id();
    const int li = lane & 15, lg = lane >> 4;
    const int64_t wp = p0 + (wave >> 1) * 64, wq = q0 + (wave & 1) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t p = wp + 4 * (4 * lg + r) + i;
            if (p >= P) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t q = wq + 4 * li + j;
                if (q < Q) put(p, q, acc[i][j][r]);
            }
        }
}

// dX stage: A[t][p] = dY[m0 + p][n] (n = nb + t) staged transposed: thread
// (p = tid / 2, half h = tid % 2) loads 16 consecutive n of token row p;
// B[t][q] = T[nb + t][k0 + q] from the packed i2 words: thread (t = tid / 8,
// c = tid % 8) unpacks the one word holding weights k0 + 16 c .. + 15 of row
// nb + t.
struct DxStage {
    const uint8_t *P;
    int64_t KB, M, N, K, lddy, m0, k0, nst;
    const float *dY;
    struct Regs {
        float a[16];
        uint32_t w;
    };
    __device__ __forceinline__ void fetch(int64_t s, Regs &r) const
    {
        const int tid = threadIdx.x;
        const int64_t nb = s * MM_S;
        {
            const int64_t m = m0 + (tid >> 1), n = nb + 16 * (tid & 1);
            const bool mv = m < M;
            const float *row = dY + (mv ? m : 0) * lddy;
#pragma unroll
            for (int e = 0; e < 16; ++e) r.a[e] = (mv && n + e < N) ? row[n + e] : 0.0f;
        }
        {
            const int64_t n = nb + (tid >> 3), k = k0 + 16 * (tid & 7);
            const bool v = n < N && k < K;
            const int64_t nc = v ? n : 0, kc = v ? k : 0;
            r.w = v ? *reinterpret_cast<const uint32_t *>(P + ((nc / 16) * KB + kc / 64) * 256 + (nc % 16) * 16 +
                                                         ((kc % 64) / 16) * 4)
                    : I2_ZERO_WORD;
        }
    }
    __device__ __forceinline__ void stash(const Regs &r, float (*sa)[MM_LD], float (*sb)[MM_LD]) const
    {
        const int tid = threadIdx.x;
        const int p = tid >> 1, t0 = 16 * (tid & 1);
#pragma unroll
        for (int e = 0; e < 16; ++e) sa[t0 + e][p] = r.a[e];
        // weight 4s + j of the word sits at bits 8j + 2s (code c = T + 1);
        // positions past K hold the zero code (padding) or the zero word
        const int t = tid >> 3, c = 16 * (tid & 7);
        float v[16];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * s + j] = static_cast<float>(static_cast<int>((r.w >> (8 * j + 2 * s)) & 3u) - 1);
#pragma unroll
        for (int e = 0; e < 16; e += 4) *reinterpret_cast<float4 *>(&sb[t][c + e]) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
    }
};

// dW stage: A[t][p] = dY[mb + t][n0 + p], B[t][q] = Xhat[mb + t][k0 + q] =
// float(q) * r_m, r_m = beta_m / 127 rounded to binary32: thread (t =
// tid / 8, c = tid % 8) loads 16 consecutive values of each.
struct DwStage {
    const int8_t *Xq;
    const float *beta, *dY;
    int64_t ldq, lddy, M, N, K, n0, k0;
    struct Regs {
        float a[16], r;
        int8_t x[16];
    };
    __device__ __forceinline__ void fetch(int64_t s, Regs &g) const
    {
        const int tid = threadIdx.x;
        const int64_t m = s * MM_S + (tid >> 3);
        const int c = 16 * (tid & 7);
        const bool mv = m < M;
        const int64_t mc = mv ? m : 0;
        g.r = mv ? beta[mc] / 127.0f : 0.0f;
        const float *yrow = dY + mc * lddy;
        const int8_t *xrow = Xq + mc * ldq;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            g.a[e] = (mv && n0 + c + e < N) ? yrow[n0 + c + e] : 0.0f;
            g.x[e] = (mv && k0 + c + e < K) ? xrow[k0 + c + e] : static_cast<int8_t>(0);
        }
    }
    __device__ __forceinline__ void stash(const Regs &g, float (*sa)[MM_LD], float (*sb)[MM_LD]) const
    {
        const int tid = threadIdx.x;
        const int t = tid >> 3, c = 16 * (tid & 7);
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
            *reinterpret_cast<float4 *>(&sa[t][c + e]) = make_float4(g.a[e], g.a[e + 1], g.a[e + 2], g.a[e + 3]);
            *reinterpret_cast<float4 *>(&sb[t][c + e]) =
                make_float4(static_cast<float>(g.x[e]) * g.r, static_cast<float>(g.x[e + 1]) * g.r,
                            static_cast<float>(g.x[e + 2]) * g.r, static_cast<float>(g.x[e + 3]) * g.r);
        }
    }
};

__global__ __launch_bounds__(256) void k_bwd_dx(const uint8_t *__restrict__ P, int64_t KB,
                                               const float *__restrict__ gamma_p, const float *__restrict__ dY,
                                               int64_t lddy, int64_t M, int64_t N, int64_t K, float *__restrict__ dX,
                                               int64_t lddx)
{
    __shared__ float sa[2][MM_S][MM_LD];
    __shared__ float sb[2][MM_S][MM_LD];
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * MM_T, k0 = static_cast<int64_t>(blockIdx.x) * MM_T;
    const DxStage st{P, KB, M, N, K, lddy, m0, k0, (N + MM_S - 1) / MM_S, dY};
    v4f acc[4][4];
    bwd_mm_body(st, sa, sb, st.nst, acc);
    const float gamma = *gamma_p;
    bwd_mm_store(acc, m0, k0, M, K, [&](int64_t m, int64_t k, float v) { dX[m * lddx + k] = gamma * v; });
}

__global__ __launch_bounds__(256) void k_bwd_dw(const int8_t *__restrict__ Xq, int64_t ldq,
                                               const float *__restrict__ beta, const float *__restrict__ dY,
                                               int64_t lddy, int64_t M, int64_t N, int64_t K, float *__restrict__ dW,
                                               int64_t lddw)
{
    __shared__ float sa[2][MM_S][MM_LD];
    __shared__ float sb[2][MM_S][MM_LD];
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * MM_T, k0 = static_cast<int64_t>(blockIdx.x) * MM_T;
    const DwStage st{Xq, beta, dY, ldq, lddy, M, N, K, n0, k0};
    v4f acc[4][4];
    bwd_mm_body(st, sa, sb, (M + MM_S - 1) / MM_S, acc);
    bwd_mm_store(acc, n0, k0, N, K, [&](int64_t n, int64_t k, float v) { dW[n * lddw + k] = v; });
}

hipError_t launch_bwd_dx(const uint8_t *P2, const float *gamma, int64_t M, int64_t N, int64_t K, const float *dY,
                         int64_t lddy, float *dX, int64_t lddx, hipStream_t stream)
{
    const int64_t KB = (K + 63) / 64;
    dim3 grid(static_cast<unsigned>((K + MM_T - 1) / MM_T), static_cast<unsigned>((M + MM_T - 1) / MM_T));
    hipLaunchKernelGGL(k_bwd_dx, grid, dim3(256), 0, stream, P2, KB, gamma, dY, lddy, M, N, K, dX, lddx);
    return hipGetLastError();
}

hipError_t launch_bwd_dw(const int8_t *Xq, int64_t ldq, const float *beta, int64_t M, int64_t N, int64_t K,
                         const float *dY, int64_t lddy, float *dW, int64_t lddw, hipStream_t stream)
{
    dim3 grid(static_cast<unsigned>((K + MM_T - 1) / MM_T), static_cast<unsigned>((N + MM_T - 1) / MM_T));
    hipLaunchKernelGGL(k_bwd_dw, grid, dim3(256), 0, stream, Xq, ldq, beta, dY, lddy, M, N, K, dW, lddw);
    return hipGetLastError();
}

} // namespace bl
