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
// is p = wp + 4 (4 (l / 16) + r) + i, q = wq + 4 (l % 16) + j, so the four
// tiles j of a lane are 4 consecutive columns: one 16-byte store where the
// row is 16-byte aligned (vec) and all four are in range.
template <class Put, class Put4>
__device__ __forceinline__ void bwd_mm_store(const v4f (&acc)[4][4], int64_t p0, int64_t q0, int64_t P, int64_t Q,
                                             bool vec, Put put, Put4 put4)
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
            if (vec && wq + 4 * li + 3 < Q) {
                put4(p, wq + 4 * li, make_float4(acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]));
                continue;
            }
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
    const bool vec = (reinterpret_cast<uintptr_t>(dX) & 15) == 0 && (lddx & 3) == 0;
    bwd_mm_store(
        acc, m0, k0, M, K, vec, [&](int64_t m, int64_t k, float v) { dX[m * lddx + k] = gamma * v; },
        [&](int64_t m, int64_t k, float4 v) {
            *reinterpret_cast<float4 *>(dX + m * lddx + k) = make_float4(gamma * v.x, gamma * v.y, gamma * v.z, gamma * v.w);
        });
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
    const bool vec = (reinterpret_cast<uintptr_t>(dW) & 15) == 0 && (lddw & 3) == 0;
    bwd_mm_store(
        acc, n0, k0, N, K, vec, [&](int64_t n, int64_t k, float v) { dW[n * lddw + k] = v; },
        [&](int64_t n, int64_t k, float4 v) { *reinterpret_cast<float4 *>(dW + n * lddw + k) = v; });
}

// ---------------------------------------------------------------------------
// Few tokens (the 128 x 128 tiles above would leave most CUs idle).
// dX = gamma * dY @ T.  Workgroup: one token group (16 tokens, blockIdx.y),
// one 64-column k-block (blockIdx.x) and one split of the weight-row tiles
// (blockIdx.z: tiles z * TPS .. min(NT, (z+1) * TPS) - 1); its W waves share
// the split's tiles (wave w takes every W-th).  For a 16-row tile the wave
// multiplies 4 row groups x 4 column groups: A = dY[16 tokens x 4 rows]
// (lane l: token l%16, row l/16), B = T[4 rows x 16 columns] (lane l: row
// l/16, column l%16, decoded from the packed word), D = dX[16 tokens x 16
// columns] per column group.  The W partial tiles meet in LDS; wave d stores
// column group d to out + z * zstride, times gamma when the tiles are not
// split (scale), else unscaled for k_bwd_dx_sum.
// ---------------------------------------------------------------------------
constexpr int DX_MAX_WAVES = 8;

__global__ __launch_bounds__(64 * DX_MAX_WAVES) void k_bwd_dx_few(const uint8_t *__restrict__ P, int64_t KB,
                                                                 int64_t NT, int64_t TPS,
                                                                 const float *__restrict__ gamma_p, int scale,
                                                                 const float *__restrict__ dY, int64_t lddy,
                                                                 int64_t M, int64_t N, int64_t K,
                                                                 float *__restrict__ out, int64_t ldo,
                                                                 int64_t zstride)
{
    __shared__ v4f red[DX_MAX_WAVES][4][64];
    const int nw = blockDim.x >> 6;
    const int wave = wave_id(), lane = lane_id();
    const int li = lane & 15, lg = lane >> 4;
    const int64_t kb = blockIdx.x;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 16;
    const int64_t t0 = static_cast<int64_t>(blockIdx.z) * TPS;
    const int64_t t1 = t0 + TPS < NT ? t0 + TPS : NT;
    const int64_t ma = m0 + li; // token of this lane's A element
    const bool mvalid = ma < M;
    const float *dyrow = dY + (mvalid ? ma : 0) * lddy;
    // column 16d + li of a chunk word d: li = 4s + j sits at bits 8j + 2s
    const int sh = 8 * (li & 3) + 2 * (li >> 2);

    v4f acc[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) acc[d] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t tile = t0 + wave; tile < t1; tile += nw) {
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
    const float g = scale ? *gamma_p : 1.0f;
    float *o = out + static_cast<int64_t>(blockIdx.z) * zstride;
    // D layout: lane l holds tokens 4 * (l/16) + r, column l%16 of the group
    for (int d = wave; d < 4; d += nw) {
        v4f tot = red[0][d][lane];
        for (int w = 1; w < nw; ++w) tot += red[w][d][lane];
        const int64_t k = kb * 64 + 16 * d + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + 4 * lg + r;
            if (m < M && k < K) o[m * ldo + k] = g * tot[r];
        }
    }
}

// One token (MT = 1; the template also holds 2 and 4, measured slower than
// k_bwd_dx_few at 4 tokens: 18 against 11.6 us for the 3B q layer): the
// 16-token MFMA tiles above would be 15/16 padding, so the product runs on the
// vector ALU (3B q 11.7 -> 9.6 us, 70B gate 106 -> 71 us).  Workgroup: one 64-column k-block
// (blockIdx.x) and one split of the weight-row tiles (blockIdx.z, as in
// k_bwd_dx_few), 4 waves taking every 4th tile of the split.  Lane l owns
// word d = l % 4 of chunk row r = l / 4, i.e. weight row tile * 16 + r and
// the 16 columns 16 d .. 16 d + 15 of the k-block (column 16 d + 4 s + j at
// bits 8 j + 2 s, code T + 1), and adds T * dY[m][row] into 16 sums per
// token.  The 16 row lanes of each word are then summed by shuffles, the 4
// waves through LDS, and the block's 64 columns stored like k_bwd_dx_few's.
template <int MT>
__global__ __launch_bounds__(256) void k_bwd_dx_vec(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                   int64_t TPS, const float *__restrict__ gamma_p, int scale,
                                                   const float *__restrict__ dY, int64_t lddy, int64_t M,
                                                   int64_t N, int64_t K, float *__restrict__ out, int64_t ldo,
                                                   int64_t zstride)
{
    __shared__ float red[4][MT][64];
    const int wave = wave_id(), lane = lane_id();
    const int r = lane >> 2, d = lane & 3;
    const int64_t kb = blockIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.z) * TPS;
    const int64_t t1 = t0 + TPS < NT ? t0 + TPS : NT;
    float acc[MT][16];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[m][c] = 0.0f;
    for (int64_t tile = t0 + wave; tile < t1; tile += 4) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(P + (tile * KB + kb) * 256 + r * 16 + d * 4);
        const int64_t n = tile * 16 + r;
        float y[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) y[m] = (m < M && n < N) ? dY[m * lddy + n] : 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float t = static_cast<float>(static_cast<int>((w >> (8 * j + 2 * s)) & 3u) - 1);
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m][4 * s + j] += t * y[m];
            }
    }
    // sum over the 16 row lanes of each word (lane bits 2..5)
#pragma unroll
    for (int off = 4; off < 64; off <<= 1)
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[m][c] += __shfl_xor(acc[m][c], off);
    if (r == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int c = 0; c < 16; ++c) red[wave][m][16 * d + c] = acc[m][c];
    }
    __syncthreads();
    const float g = scale ? *gamma_p : 1.0f;
    float *o = out + static_cast<int64_t>(blockIdx.z) * zstride;
    for (int e = threadIdx.x; e < MT * 64; e += 256) {
        const int m = e / 64, c = e % 64;
        const int64_t k = kb * 64 + c;
        if (m < M && k < K) o[m * ldo + k] = g * (red[0][m][c] + red[1][m][c] + red[2][m][c] + red[3][m][c]);
    }
}

// dX[m][k] = gamma * sum over the S <= DX_MAX_SPLITS splits of part[z][m][k],
// z in order (part: S blocks of M x K, row stride K).  Thread: column k =
// blockIdx.x * 256 + tid of token m = blockIdx.y; its S loads are all issued
// before the sum.
constexpr int DX_MAX_SPLITS = 16;

__global__ __launch_bounds__(256) void k_bwd_dx_sum(const float *__restrict__ part, int S, int64_t M, int64_t K,
                                                   const float *__restrict__ gamma_p, float *__restrict__ dX,
                                                   int64_t lddx)
{
    const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x, m = blockIdx.y;
    if (k >= K) return;
    const float *p = part + m * K + k;
    const int64_t MK = M * K;
    float v[DX_MAX_SPLITS];
#pragma unroll
    for (int z = 0; z < DX_MAX_SPLITS; ++z) v[z] = z < S ? p[z * MK] : 0.0f;
    float t = v[0];
#pragma unroll
    for (int z = 1; z < DX_MAX_SPLITS; ++z)
        if (z < S) t += v[z];
    dX[m * lddx + k] = *gamma_p * t;
}

// ---------------------------------------------------------------------------
// dW = dY^T @ Xhat.  Workgroup: 64 rows n x 64 columns k of dW, 4 waves of
// 32 x 32 (2 x 2 MFMA tiles); the contraction runs over the tokens, 4 per
// MFMA, 4 MFMA k-steps (16 tokens) per loop trip with all their loads issued
// first.  A = dY^T[16 rows x 4 tokens] (lane l: row l%16, token l/16),
// B = Xhat[4 tokens x 16 columns] (lane l: token l/16, column l%16), with
// Xhat = float(q) * r_m and r_m = beta_m / 127 rounded to binary32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_dw_few(const int8_t *__restrict__ Xq, int64_t ldq,
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

// ---------------------------------------------------------------------------
// dW for one token (the kernel takes up to 4; at 4 tokens it was slower
// than k_bwd_dw_few, 19 against 12.4 us for the 3B q layer): a rank-M outer
// product, bound by its N x K fp32 writes (3B q 12.6 -> 12.1 us, 70B gate
// 186 -> 166 us).  Workgroup: 4 rows n (blockIdx.x) x 1024 columns k (blockIdx.y);
// thread t owns columns k0 + 4 t .. + 3 of the 4 rows, forms Xhat = float(q)
// * r_m for its 4 columns of every token once, and stores dW[n][k..k+3] =
// sum_m dY[m][n] * Xhat[m][k..k+3] (tokens in order) as one 16-byte store
// where the row is 16-byte aligned (vec) and all four columns exist.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_dw_vec(const int8_t *__restrict__ Xq, int64_t ldq,
                                                   const float *__restrict__ beta, const float *__restrict__ dY,
                                                   int64_t lddy, int64_t M, int64_t N, int64_t K,
                                                   float *__restrict__ dW, int64_t lddw, int vec)
{
    const int64_t k = static_cast<int64_t>(blockIdx.y) * 1024 + 4 * threadIdx.x;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 4;
    if (k >= K) return;
    float xh[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float r = m < M ? beta[m] / 127.0f : 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            xh[m][e] = (m < M && k + e < K) ? static_cast<float>(Xq[m * ldq + k + e]) * r : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + i;
        if (n >= N) break;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float t = 0.0f;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if (m < M) t += dY[m * lddy + n] * xh[m][e];
            v[e] = t;
        }
        float *row = dW + n * lddw;
        if (vec && k + 3 < K) {
            *reinterpret_cast<float4 *>(row + k) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k + e < K) row[k + e] = v[e];
        }
    }
}

// The 128 x 128 dX tiles number ceil(M / 128) ceil(K / 128); below one per
// CU the small-batch kernel, whose workgroups cover 16 tokens x 64 columns,
// keeps more of the chip busy.  dW always has ceil(N / 128) ceil(K / 128)
// tiles; its small-batch kernel only avoids staging 32 tokens of which most
// are padding.
static bool bwd_dx_few(int64_t M, int64_t K)
{
    return ((M + MM_T - 1) / MM_T) * ((K + MM_T - 1) / MM_T) < 256;
}

static bool bwd_dw_few(int64_t M) { return M < MM_S; }

// Splits of the weight-row tiles for the small-batch dX: enough workgroups
// for about two per CU, at most 16 splits, at least 8 tiles (one per wave)
// per split.  Splits write partial tiles that k_bwd_dx_sum adds in order.
int64_t bwd_dx_splits(int64_t M, int64_t N, int64_t K)
{
    if (!bwd_dx_few(M, K)) return 1;
    const int64_t wgs = ((K + 63) / 64) * ((M + 15) / 16), NT = (N + 15) / 16;
    int64_t s = (2 * 256 + wgs - 1) / wgs;
    if (s > DX_MAX_SPLITS) s = DX_MAX_SPLITS;
    if (s > NT / 8) s = NT / 8;
    return s < 1 ? 1 : s;
}

int64_t bwd_dx_partial_bytes(int64_t M, int64_t N, int64_t K)
{
    const int64_t s = bwd_dx_splits(M, N, K);
    return s > 1 ? s * M * K * 4 : 0;
}

const char *bwd_kernel_name(bool dx, int64_t M, int64_t K)
{
    if (dx) return !bwd_dx_few(M, K) ? "bl::k_bwd_dx" : (M == 1 ? "bl::k_bwd_dx_vec<1>" : "bl::k_bwd_dx_few");
    return M == 1 ? "bl::k_bwd_dw_vec" : (bwd_dw_few(M) ? "bl::k_bwd_dw_few" : "bl::k_bwd_dw");
}

hipError_t launch_bwd_dx(const uint8_t *P2, const float *gamma, int64_t M, int64_t N, int64_t K, const float *dY,
                         int64_t lddy, float *dX, int64_t lddx, float *part, hipStream_t stream)
{
    const int64_t KB = (K + 63) / 64;
    if (bwd_dx_few(M, K)) {
        const int64_t NT = (N + 15) / 16, S = bwd_dx_splits(M, N, K);
        const int64_t TPS = (NT + S - 1) / S;
        const int64_t nw = TPS < DX_MAX_WAVES ? TPS : DX_MAX_WAVES;
        dim3 grid(static_cast<unsigned>(KB), static_cast<unsigned>((M + 15) / 16), static_cast<unsigned>(S));
        if (M == 1) {
            float *o = S == 1 ? dX : part;
            const int64_t ldo = S == 1 ? lddx : K, zs = S == 1 ? 0 : M * K;
            const int sc = S == 1 ? 1 : 0;
            hipLaunchKernelGGL(k_bwd_dx_vec<1>, grid, dim3(256), 0, stream, P2, KB, NT, TPS, gamma, sc, dY, lddy, M, N,
                               K, o, ldo, zs);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess || S == 1) return e;
            hipLaunchKernelGGL(k_bwd_dx_sum, dim3(static_cast<unsigned>((K + 255) / 256), static_cast<unsigned>(M)),
                               dim3(256), 0, stream, part, static_cast<int>(S), M, K, gamma, dX, lddx);
            return hipGetLastError();
        }
        if (S == 1) {
            hipLaunchKernelGGL(k_bwd_dx_few, grid, dim3(static_cast<unsigned>(64 * nw)), 0, stream, P2, KB, NT, TPS,
                               gamma, 1, dY, lddy, M, N, K, dX, lddx, int64_t(0));
            return hipGetLastError();
        }
        hipLaunchKernelGGL(k_bwd_dx_few, grid, dim3(static_cast<unsigned>(64 * nw)), 0, stream, P2, KB, NT, TPS,
                           gamma, 0, dY, lddy, M, N, K, part, K, M * K);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_bwd_dx_sum, dim3(static_cast<unsigned>((K + 255) / 256), static_cast<unsigned>(M)),
                           dim3(256), 0, stream, part, static_cast<int>(S), M, K, gamma, dX, lddx);
        return hipGetLastError();
    }
    const int64_t mt = (M + MM_T - 1) / MM_T, kt = (K + MM_T - 1) / MM_T;
    dim3 grid(static_cast<unsigned>(kt), static_cast<unsigned>(mt));
    hipLaunchKernelGGL(k_bwd_dx, grid, dim3(256), 0, stream, P2, KB, gamma, dY, lddy, M, N, K, dX, lddx);
    return hipGetLastError();
}

hipError_t launch_bwd_dw(const int8_t *Xq, int64_t ldq, const float *beta, int64_t M, int64_t N, int64_t K,
                         const float *dY, int64_t lddy, float *dW, int64_t lddw, hipStream_t stream)
{
    if (M == 1) {
        const int vec = (reinterpret_cast<uintptr_t>(dW) & 15) == 0 && (lddw & 3) == 0;
        dim3 grid(static_cast<unsigned>((N + 3) / 4), static_cast<unsigned>((K + 1023) / 1024));
        hipLaunchKernelGGL(k_bwd_dw_vec, grid, dim3(256), 0, stream, Xq, ldq, beta, dY, lddy, M, N, K, dW, lddw, vec);
        return hipGetLastError();
    }
    if (bwd_dw_few(M)) {
        dim3 grid(static_cast<unsigned>((K + 63) / 64), static_cast<unsigned>((N + 63) / 64));
        hipLaunchKernelGGL(k_bwd_dw_few, grid, dim3(256), 0, stream, Xq, ldq, beta, dY, lddy, M, N, K, dW, lddw);
        return hipGetLastError();
    }
    dim3 grid(static_cast<unsigned>((K + MM_T - 1) / MM_T), static_cast<unsigned>((N + MM_T - 1) / MM_T));
    hipLaunchKernelGGL(k_bwd_dw, grid, dim3(256), 0, stream, Xq, ldq, beta, dY, lddy, M, N, K, dW, lddw);
    return hipGetLastError();
}

} // namespace bl
