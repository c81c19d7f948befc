// gemv.hip -- the decode product acc[m][n] = sum_k q[m][k] * T[n][k] for a few
// tokens, followed by the rescale y = float(acc) * (gamma * beta_m) / 127.
//
// LIT-380 record (dmarx anthology), Key takeaways, bullet 4: with ternary
// weights the product needs only additions and subtractions.  The same
// record's closing section notes that on stock GPUs the memory saving is what
// survives: this path streams 2 bits (i2) or 1.6 bits (b3) per weight from HBM
// and is bound by it.
//
// Two kernels:
//  * k_gemv_mfma: tiles of 16 tokens x 16 rows on the int8 matrix cores
//    (v_mfma_i32_16x16x64_i8), the packed weights unpacked in registers to
//    signed bytes.  Waves issue all loads of a batch of k-steps before their
//    first MFMA, so many HBM round trips overlap.
//  * k_gemv_addsub: vector-ALU add/subtract.  A lane owns one weight row and
//    the activation words are wave-uniform.  The offset code c = T + 1 in
//    {0, 1, 2} goes through v_dot4_i32_i8: sum_k c*q adds q where T = 0, 2q
//    where T = +1 and nothing where T = -1; subtracting sum_k q leaves
//    sum_{T=+1} q - sum_{T=-1} q exactly.
#include <cstdio>

#include "common.h"
#include "gemv_core.h"
#include "fq_core.h"
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
// MFMA GEMV.  A k-step is 4 consecutive k-blocks (i2: 256 weights, b3: 320).
// In a k-step, lane l (i = l % 16, g = l / 16) holds the 16-byte chunk of row
// 16*tile + i at k-block 4*step + g.  i2: MFMA d (0..3) multiplies word d
// (16 weights) with activations kb*64 + 16d .. +15 of token i; b3: MFMA t
// (0..4) multiplies base-3 digit t of the 16 bytes with activations
// kb*80 + 16t .. +15.
//
// A workgroup owns TW consecutive row tiles and has KS waves; wave w takes
// the k-steps w, w + KS, ... of all TW tiles, SB steps at a time: it issues
// the loads of SB steps (SB activation operands, SB x TW weight chunks) before
// the first MFMA, and reuses each activation operand for the TW tiles.  With
// up to 16 waves per CU this keeps ~100 KB of weights in flight per CU.  The
// KS partial tiles are summed through LDS; wave t < TW writes tile t.
// ---------------------------------------------------------------------------
// Per-token maxima of |Y| as stored, for the next product's quantiser (the
// producer side of the per-token absmax): lm[rr] is this lane's maximum for
// token 4g + rr; the 16 lanes of a group (rows i) combine by shuffles, the
// waves through LDS, and wave 0 writes the workgroup's 16 maxima to
// pmax[blockIdx.x * 16 + token] with plain stores (tokens past M hold 0).
// Every wave of the workgroup must call it (a barrier).
__device__ __forceinline__ void write_token_maxima(float (&lm)[4], float *__restrict__ pmax, float (*pm)[16])
{
    const int wave = wave_id(), lane = lane_id(), KS = blockDim.x >> 6;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) lm[rr] = fmaxf(lm[rr], __shfl_xor(lm[rr], off));
    if ((lane & 15) == 0)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) pm[wave][4 * (lane >> 4) + rr] = lm[rr];
    __syncthreads();
    if (wave == 0 && lane < 16) {
        float mx = pm[0][lane];
        for (int w = 1; w < KS; ++w) mx = fmaxf(mx, pm[w][lane]);
        pmax[static_cast<int64_t>(blockIdx.x) * 16 + lane] = mx;
    }
}

template <int LAYOUT, int TW, int SB, bool TILED>
__global__ __launch_bounds__(1024) void k_gemv_mfma(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                    const float *__restrict__ gamma_p,
                                                    const int8_t *__restrict__ Xq, int64_t ldq,
                                                    const float *__restrict__ beta, int64_t M, int64_t N,
                                                    int64_t K, void *__restrict__ Y, int y_dtype, int64_t ldy,
                                                    float *__restrict__ pmax, int64_t pmax_cols)
{
    using S = StepShape<LAYOUT>;
    constexpr int NMF = S::NMF, KBLK = S::KBLK;
    constexpr int STEP_K = 4 * KBLK; // weights per k-step
    __shared__ v4i red[TW][16][64];
    const int KS = blockDim.x >> 6;
    const int wave = wave_id(), lane = lane_id();
    const int i = lane & 15, g = lane >> 4;
    const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * TW;
    const int64_t nsteps = (KB + 3) / 4;
    // Row-major activations: k-steps whose activations all lie inside K run
    // without bounds checks, the last partial one is checked.  Tiled
    // activations are zero-padded, so every k-step runs unchecked: a weight
    // chunk past the last k-block (address clamped) meets zero activations.
    const int64_t nfull = TILED ? nsteps : K / STEP_K;
    // (b1 has no zero weight: its past-the-end chunk meets zero activations)
    const uint4 zero_chunk = LAYOUT == LAYOUT_I2   ? make_uint4(I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD)
                             : LAYOUT == LAYOUT_B3 ? make_uint4(B3_ZERO_WORD, B3_ZERO_WORD, B3_ZERO_WORD, B3_ZERO_WORD)
                                                   : make_uint4(0u, 0u, 0u, 0u);
    // Tokens past M and tiles past NT read valid rows (clamped); their results are never stored.
    const int64_t m_a = static_cast<int64_t>(blockIdx.y) * 16 + i;
    const int8_t *xrow = TILED ? Xq + (static_cast<int64_t>(blockIdx.y) * nsteps * NMF * 64 + lane) * 16
                               : Xq + (m_a < M ? m_a : M - 1) * ldq + g * KBLK;
    const uint8_t *ptile[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int64_t tt = tile0 + t < NT ? tile0 + t : NT - 1;
        ptile[t] = P + tt * KB * 256;
    }
    const uint32_t lane_off = static_cast<uint32_t>(g) * 256u + static_cast<uint32_t>(i) * 16u;
    const uint32_t last_kb_off = static_cast<uint32_t>(KB - 1) * 256u + static_cast<uint32_t>(i) * 16u;
    // rescale factors of this lane's 4 output tokens, loaded before the product
    // (clamped loads, then selects: no branch, so the four loads overlap)
    float sc[4];
    {
        const float gamma = *gamma_p;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int64_t mm = static_cast<int64_t>(blockIdx.y) * 16 + 4 * g + rr;
            const float v = token_scale(gamma, beta[mm < M ? mm : M - 1]);
            sc[rr] = mm < M ? v : 0.0f;
        }
    }

    v4i acc[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[t] = v4i{0, 0, 0, 0};

    // Software-pipelined: the loads of the next batch are in flight while the
    // current batch is unpacked and multiplied.
    const int64_t stride = static_cast<int64_t>(KS) * SB;
    auto load_batch = [&](int64_t s0, uint4 (&b)[SB][TW], v4i (&a)[SB][NMF]) {
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            int64_t s = s0 + static_cast<int64_t>(j) * KS;
            s = s < nfull ? s : nfull - 1; // (the loop never asks past the last step)
            uint32_t off = static_cast<uint32_t>(s) * 1024u + lane_off;
            if (TILED) off = 4 * s + g < KB ? off : last_kb_off;
#pragma unroll
            for (int t = 0; t < TW; ++t) b[j][t] = *reinterpret_cast<const uint4 *>(ptile[t] + off);
#pragma unroll
            for (int d = 0; d < NMF; ++d)
                a[j][d] = TILED ? *reinterpret_cast<const v4i *>(xrow + (s * NMF + d) * 1024)
                                : *reinterpret_cast<const v4i *>(xrow + s * STEP_K + 16 * d);
        }
    };
    // (SB = 1: the loop below only computes batches that exist)
    static_assert(SB == 1, "one k-step per batch");
    v4i sacc = {0, 0, 0, 0}; // sum_k q of the wave's k-steps (offset codes only)
    auto compute_batch = [&](int64_t, const uint4 (&b)[SB][TW], const v4i (&a)[SB][NMF]) {
        gemv_step<LAYOUT, TW, NMF>(b[0], a[0], acc);
        if constexpr (kOffsetCodes<LAYOUT>) act_sum_step<NMF>(a[0], sacc);
    };
    if (wave < nfull) {
        uint4 b0[SB][TW], b1[SB][TW];
        v4i a0[SB][NMF], a1[SB][NMF];
        const int64_t niter = (nfull - 1 - wave) / stride + 1; // k-steps of this wave
        int64_t s0 = wave, it = 0;
        load_batch(s0, b0, a0);
        // Two steps per trip, each preceded by the unconditional request of the
        // next one: every path through the loop has the same loads outstanding,
        // so the wait before a step's MFMAs covers only that step and the next
        // stays in flight.  The last one or two steps run after the loop, so no
        // request goes past this wave's last step.
        for (; it + 2 < niter; it += 2, s0 += 2 * stride) {
            load_batch(s0 + stride, b1, a1);
            __builtin_amdgcn_sched_barrier(0);
            compute_batch(s0, b0, a0);
            load_batch(s0 + 2 * stride, b0, a0);
            __builtin_amdgcn_sched_barrier(0);
            compute_batch(s0 + stride, b1, a1);
        }
        if (niter - it == 2) {
            load_batch(s0 + stride, b1, a1);
            __builtin_amdgcn_sched_barrier(0);
            compute_batch(s0, b0, a0);
            compute_batch(s0 + stride, b1, a1);
        } else {
            compute_batch(s0, b0, a0);
        }
    }
    // the partial k-step of row-major activations, bounds-checked
    if (!TILED && nfull < nsteps && wave == static_cast<int>(nfull % KS)) {
        const int64_t kb = 4 * nfull + g;
        uint4 b[TW];
        v4i a[NMF];
#pragma unroll
        for (int t = 0; t < TW; ++t)
            b[t] = kb < KB ? *reinterpret_cast<const uint4 *>(ptile[t] + kb * 256 + i * 16) : zero_chunk;
#pragma unroll
        for (int d = 0; d < NMF; ++d) a[d] = load_a16(Xq, ldq, m_a, M, K, kb * KBLK + 16 * d);
        gemv_step<LAYOUT, TW, NMF>(b, a, acc);
        if constexpr (kOffsetCodes<LAYOUT>) act_sum_step<NMF>(a, sacc);
    }

#pragma unroll
    for (int t = 0; t < TW; ++t) red[t][wave][lane] = kOffsetCodes<LAYOUT> ? offset_fix<LAYOUT>(acc[t], sacc) : acc[t];
    __syncthreads();
    // tile t is finished by wave t % KS (KS may be smaller than TW)
    float lm[4] = {0.0f, 0.0f, 0.0f, 0.0f}; // |Y| maxima per token (pmax)
    for (int t = wave; t < TW; t += KS) {
        const int64_t tile = tile0 + t;
        if (tile >= NT) break;
        v4i tot = red[t][0][lane];
        for (int w = 1; w < KS; ++w) tot += red[t][w][lane];
        // D layout: lane l holds tokens 4g + rr of this token group, weight row i of the tile.
        const int64_t n = tile * 16 + i;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int64_t mm = static_cast<int64_t>(blockIdx.y) * 16 + 4 * g + rr;
            if (mm < M && n < N) {
                store_out(Y, y_dtype, ldy, mm, n, tot[rr], sc[rr]);
                if (n < pmax_cols) lm[rr] = fmaxf(lm[rr], stored_abs(y_dtype, tot[rr], sc[rr]));
            }
        }
    }
    if (pmax != nullptr) {
        __shared__ float pm[16][16];
        write_token_maxima(lm, pmax, pm);
    }
}

// One row tile per workgroup (the k_gemv_mfma split, TW = 1), KS <= 10 waves.
template <int LAYOUT, int XDT, int SPW>
__global__ __launch_bounds__(64 * FQ_MAX_WAVES) void k_gemv_fq(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                              const float *__restrict__ gamma_p,
                                                              const void *__restrict__ X, int64_t ldx, int xbytes,
                                                              int64_t M, int64_t N, int64_t K, void *__restrict__ Y,
                                                              int y_dtype, int64_t ldy)
{
    using FU = FqUnits<LAYOUT, XDT, SPW>;
    constexpr int NMF = FU::NMF;
    __shared__ v4i qbuf[FQ_MAX_WAVES][SPW * FU::UNITS];
    __shared__ float wmax[FQ_MAX_WAVES][4];
    __shared__ v4i red[FQ_MAX_WAVES][64];
    const int KS = blockDim.x >> 6;
    const int wave = wave_id(), lane = lane_id();
    const int i = lane & 15, g = lane >> 4;
    const int64_t tile = blockIdx.x;
    const int64_t nsteps = (KB + 3) / 4;
    const uint4 zero_chunk = LAYOUT == LAYOUT_I2   ? make_uint4(I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD)
                             : LAYOUT == LAYOUT_B3 ? make_uint4(B3_ZERO_WORD, B3_ZERO_WORD, B3_ZERO_WORD, B3_ZERO_WORD)
                                                   : make_uint4(0u, 0u, 0u, 0u);
    int nj = 0;
#pragma unroll
    for (int j = 0; j < SPW; ++j) nj += wave + static_cast<int64_t>(j) * KS < nsteps ? 1 : 0;
    const FU U{lane, wave, KS, static_cast<int>(M), nj * static_cast<int>(M) * FU::CH, static_cast<int>(K),
               static_cast<int>(ldx)};

    uint4 xv[FU::NUW][FU::VL];
    fq_load(U, X, xbytes, xv);
    uint4 wb[SPW];
    {
        const uint8_t *pt = P + tile * KB * 256;
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int64_t st = wave + static_cast<int64_t>(j) * KS;
            const int64_t kb = 4 * (st < nsteps ? st : nsteps - 1) + g;
            const uint4 v = *reinterpret_cast<const uint4 *>(pt + (kb < KB ? kb : KB - 1) * 256 + i * 16);
            wb[j] = kb < KB ? v : zero_chunk;
        }
    }
    const float gamma = *gamma_p;
    // keep every load above this point: the compiler would otherwise sink the
    // weight loads below the activation work and serialise the round trips
    __builtin_amdgcn_sched_barrier(0);

    v4i a[SPW][NMF];
    const float beta_lane = fq_quantise<FU, SPW>(U, xv, &qbuf[wave][0], wmax, a);

    v4i acc[1] = {v4i{0, 0, 0, 0}};
    v4i sacc = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        if (j >= nj) break;
        const uint4 b[1] = {wb[j]};
        gemv_step<LAYOUT, 1, NMF>(b, a[j], acc);
        if constexpr (kOffsetCodes<LAYOUT>) act_sum_step<NMF>(a[j], sacc);
    }
    red[wave][lane] = kOffsetCodes<LAYOUT> ? offset_fix<LAYOUT>(acc[0], sacc) : acc[0];
    float sc[4]; // rescale of tokens 4g .. 4g + 3 (shuffled while all lanes are active)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sc[rr] = token_scale(gamma, __shfl(beta_lane, (4 * g + rr) & 3));
    __syncthreads();
    if (wave != 0 || g != 0) return; // tokens 0..3: lanes of g = 0
    v4i tot = red[0][lane];
    for (int w = 1; w < KS; ++w) tot += red[w][lane];
    const int64_t n = tile * 16 + i;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
        if (rr < M && n < N) store_out(Y, y_dtype, ldy, rr, n, tot[rr], sc[rr]);
}

// ---------------------------------------------------------------------------
// Persistent MFMA GEMV for large layers.  About one workgroup per CU, KS
// waves; wave w owns the k-steps w, w + KS, ... (at most SPW of them): it loads
// their activation operands into registers once and then streams the packed
// weights of its workgroup's row tiles blockIdx.x + t * gridDim.x
// (t < TMAX), keeping one accumulator per tile, with a ring of D tiles in
// flight.  No barrier until every tile is done; then the KS partials of every
// tile meet in LDS and the 4 x TMAX output groups are summed by different
// waves.  Activations cross L2 once per CU instead of once per tile.
// ---------------------------------------------------------------------------
template <int LAYOUT, int SPW, int TMAX, bool TILED, bool GUARD>
__global__ __launch_bounds__(1024) void k_gemv_persist(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                       const float *__restrict__ gamma_p,
                                                       const int8_t *__restrict__ Xq, int64_t ldq,
                                                       const float *__restrict__ beta, int64_t M, int64_t N,
                                                       int64_t K, void *__restrict__ Y, int y_dtype, int64_t ldy,
                                                       float *__restrict__ pmax, int64_t pmax_cols)
{
    using S = StepShape<LAYOUT>;
    constexpr int NMF = S::NMF, KBLK = S::KBLK;
    constexpr int D = SPW >= 4 ? 2 : (SPW >= 2 ? 3 : 4);
    extern __shared__ int red_dyn[]; // [TMAX][KS][4][64]
    const int KS = blockDim.x >> 6;
    const int wave = wave_id(), lane = lane_id();
    const int i = lane & 15, g = lane >> 4;
    const int64_t nsteps = (KB + 3) / 4;
    const int64_t m_a = static_cast<int64_t>(blockIdx.y) * 16 + i;
    const int64_t G = gridDim.x;
    const int ntiles = static_cast<int>((NT - blockIdx.x + G - 1) / G); // tiles of this workgroup (<= TMAX)
    // rescale factors of this lane's 4 output tokens, loaded before the product
    // (clamped loads, then selects: no branch, so the four loads overlap)
    float sc[4];
    {
        const float gamma = *gamma_p;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int64_t mm = static_cast<int64_t>(blockIdx.y) * 16 + 4 * g + rr;
            const float v = token_scale(gamma, beta[mm < M ? mm : M - 1]);
            sc[rr] = mm < M ? v : 0.0f;
        }
    }

    uint32_t boff[SPW]; // byte offset of this lane's weight chunk in a tile, per k-step
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int64_t kb = 4 * (wave + static_cast<int64_t>(j) * KS) + g;
        boff[j] = static_cast<uint32_t>(kb < KB ? kb : KB - 1) * 256u + static_cast<uint32_t>(i) * 16u;
    }
    // Ring loads.  Unguarded (many tiles per workgroup): tiles past this
    // workgroup's last one re-read its last tile (just fetched, so from L2)
    // and are never used; the loads are unconditional, every path has the same
    // loads outstanding, and the wait before tile t leaves the next D-1 tiles
    // in flight.  Guarded (a few tiles per workgroup): tiles that do not exist
    // are skipped, which saves the redundant reads when they would be a large
    // share of the work.
    auto load_tile = [&](int t, uint4 (&b)[SPW]) {
        const int64_t tile = blockIdx.x + static_cast<int64_t>(t < ntiles ? t : ntiles - 1) * G;
        const uint8_t *pt = P + tile * KB * 256;
#pragma unroll
        for (int j = 0; j < SPW; ++j) b[j] = *reinterpret_cast<const uint4 *>(pt + boff[j]);
    };

    v4i acc[TMAX];
    uint4 b[D][SPW];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) acc[t] = v4i{0, 0, 0, 0};
    // activation operands of this wave's k-steps, loaded once (zero past K),
    // before the first weight tiles: waits are in issue order, so the wait for
    // tile 0 then leaves tiles 1 .. D-1 in flight
    v4i a[SPW][NMF];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int64_t s = wave + static_cast<int64_t>(j) * KS;
        const int64_t sx = s < nsteps ? s : nsteps - 1;
        const int64_t kb = 4 * sx + g;
#pragma unroll
        for (int d = 0; d < NMF; ++d) {
            v4i v = TILED ? *reinterpret_cast<const v4i *>(
                                Xq + (((static_cast<int64_t>(blockIdx.y) * nsteps + sx) * NMF + d) * 64 + lane) * 16)
                          : load_a16(Xq, ldq, m_a, M, K, kb * KBLK + 16 * d);
            a[j][d] = s < nsteps ? v : v4i{0, 0, 0, 0};
        }
    }

    v4i sacc = {0, 0, 0, 0}; // sum_k q of the wave's k-steps (offset codes only)
    if constexpr (kOffsetCodes<LAYOUT>) {
#pragma unroll
        for (int j = 0; j < SPW; ++j) act_sum_step<NMF>(a[j], sacc);
    }

#pragma unroll
    for (int t = 0; t < D; ++t)
        if (!GUARD || t < ntiles) load_tile(t, b[t]);
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t >= ntiles) break;
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            if (wave + static_cast<int64_t>(j) * KS >= nsteps) break;
            const uint4 bj[1] = {b[t % D][j]};
            v4i accs[1] = {acc[t]};
            gemv_step<LAYOUT, 1, NMF>(bj, a[j], accs);
            acc[t] = accs[0];
        }
        if (!GUARD || t + D < ntiles) load_tile(t + D, b[t % D]);
    }
    int *red = red_dyn;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t >= ntiles) break;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            red[((t * KS + wave) * 4 + rr) * 64 + lane] =
                kOffsetCodes<LAYOUT> ? offset_fix<LAYOUT>(acc[t][rr], sacc[rr]) : acc[t][rr];
    }
    __syncthreads();
    // output group (t, rr): tokens 4g + rr of this token group, weight row i of tile t
    float lm[4] = {0.0f, 0.0f, 0.0f, 0.0f}; // |Y| maxima per token (pmax)
    for (int task = wave; task < ntiles * 4; task += KS) {
        const int t = task >> 2, rr = task & 3;
        int tot = 0;
        for (int w = 0; w < KS; ++w) tot += red[((t * KS + w) * 4 + rr) * 64 + lane];
        const int64_t n = (blockIdx.x + t * G) * 16 + i;
        const int64_t mm = static_cast<int64_t>(blockIdx.y) * 16 + 4 * g + rr;
        float s_rr = sc[0];
        s_rr = rr == 1 ? sc[1] : s_rr;
        s_rr = rr == 2 ? sc[2] : s_rr;
        s_rr = rr == 3 ? sc[3] : s_rr;
        if (mm < M && n < N) {
            store_out(Y, y_dtype, ldy, mm, n, tot, s_rr);
            const float v = n < pmax_cols ? stored_abs(y_dtype, tot, s_rr) : 0.0f;
            lm[0] = rr == 0 ? fmaxf(lm[0], v) : lm[0];
            lm[1] = rr == 1 ? fmaxf(lm[1], v) : lm[1];
            lm[2] = rr == 2 ? fmaxf(lm[2], v) : lm[2];
            lm[3] = rr == 3 ? fmaxf(lm[3], v) : lm[3];
        }
    }
    if (pmax != nullptr) {
        __shared__ float pm[16][16];
        write_token_maxima(lm, pmax, pm);
    }
}

// ---------------------------------------------------------------------------
// k_gemv_persist with the activation quantiser inside (1 to 4 tokens of fp32 /
// bf16 rows; see fq_load / fq_quantise): the wave's activation loads, then
// the first D weight tiles of the ring, then the rounding while those are in
// flight.
// ---------------------------------------------------------------------------
constexpr int FQ_PERSIST_WAVES = 16;

template <int LAYOUT, int XDT, int SPW, int TMAX, bool GUARD>
__global__ __launch_bounds__(1024) void k_gemv_persist_fq(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                          const float *__restrict__ gamma_p,
                                                          const void *__restrict__ X, int64_t ldx, int xbytes,
                                                          int64_t M, int64_t N, int64_t K, void *__restrict__ Y,
                                                          int y_dtype, int64_t ldy)
{
    using FU = FqUnits<LAYOUT, XDT, SPW>;
    constexpr int NMF = FU::NMF;
    constexpr int D = SPW >= 4 ? 2 : (SPW >= 2 ? 3 : 4);
    extern __shared__ int red_dyn[]; // [TMAX][KS][4][64]
    __shared__ v4i qbuf[FQ_PERSIST_WAVES][SPW * FU::UNITS];
    __shared__ float wmax[FQ_PERSIST_WAVES][4];
    const int KS = blockDim.x >> 6;
    const int wave = wave_id(), lane = lane_id();
    const int i = lane & 15, g = lane >> 4;
    const int64_t nsteps = (KB + 3) / 4;
    const int64_t G = gridDim.x;
    const int ntiles = static_cast<int>((NT - blockIdx.x + G - 1) / G); // tiles of this workgroup (<= TMAX)
    int nj = 0;
#pragma unroll
    for (int j = 0; j < SPW; ++j) nj += wave + static_cast<int64_t>(j) * KS < nsteps ? 1 : 0;
    const FU U{lane, wave, KS, static_cast<int>(M), nj * static_cast<int>(M) * FU::CH, static_cast<int>(K),
               static_cast<int>(ldx)};

    uint4 xv[FU::NUW][FU::VL];
    fq_load(U, X, xbytes, xv);

    uint32_t boff[SPW]; // byte offset of this lane's weight chunk in a tile, per k-step
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int64_t kb = 4 * (wave + static_cast<int64_t>(j) * KS) + g;
        boff[j] = static_cast<uint32_t>(kb < KB ? kb : KB - 1) * 256u + static_cast<uint32_t>(i) * 16u;
    }
    auto load_tile = [&](int t, uint4 (&b)[SPW]) {
        const int64_t tile = blockIdx.x + static_cast<int64_t>(t < ntiles ? t : ntiles - 1) * G;
        const uint8_t *pt = P + tile * KB * 256;
#pragma unroll
        for (int j = 0; j < SPW; ++j) b[j] = *reinterpret_cast<const uint4 *>(pt + boff[j]);
    };
    v4i acc[TMAX];
    uint4 b[D][SPW];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) acc[t] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < D; ++t)
        if (!GUARD || t < ntiles) load_tile(t, b[t]);
    const float gamma = *gamma_p;
    // keep every load above this point (see k_gemv_fq)
    __builtin_amdgcn_sched_barrier(0);

    v4i a[SPW][NMF];
    const float beta_lane = fq_quantise<FU, SPW>(U, xv, &qbuf[wave][0], wmax, a);
    float sc[4]; // rescale of tokens 4g .. 4g + 3 (shuffled while all lanes are active)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sc[rr] = token_scale(gamma, __shfl(beta_lane, (4 * g + rr) & 3));
    v4i sacc = {0, 0, 0, 0}; // sum_k q of the wave's k-steps (offset codes only)
    if constexpr (kOffsetCodes<LAYOUT>) {
#pragma unroll
        for (int j = 0; j < SPW; ++j)
            if (j < nj) act_sum_step<NMF>(a[j], sacc);
    }

#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t >= ntiles) break;
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            if (j >= nj) break;
            const uint4 bj[1] = {b[t % D][j]};
            v4i accs[1] = {acc[t]};
            gemv_step<LAYOUT, 1, NMF>(bj, a[j], accs);
            acc[t] = accs[0];
        }
        if (!GUARD || t + D < ntiles) load_tile(t + D, b[t % D]);
    }
    int *red = red_dyn;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t >= ntiles) break;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            red[((t * KS + wave) * 4 + rr) * 64 + lane] =
                kOffsetCodes<LAYOUT> ? offset_fix<LAYOUT>(acc[t][rr], sacc[rr]) : acc[t][rr];
    }
    __syncthreads();
    // output group (t, rr): token 4g + rr, weight row i of tile t (tokens < 4: g = 0)
    for (int task = wave; task < ntiles * 4; task += KS) {
        const int t = task >> 2, rr = task & 3;
        int tot = 0;
        for (int w = 0; w < KS; ++w) tot += red[((t * KS + w) * 4 + rr) * 64 + lane];
        const int64_t n = (blockIdx.x + t * G) * 16 + i;
        float s_rr = sc[0];
        s_rr = rr == 1 ? sc[1] : s_rr;
        s_rr = rr == 2 ? sc[2] : s_rr;
        s_rr = rr == 3 ? sc[3] : s_rr;
        if (g == 0 && rr < M && n < N) store_out(Y, y_dtype, ldy, rr, n, tot, s_rr);
    }
}

// ---------------------------------------------------------------------------
// Add/subtract GEMV: a workgroup owns 64 weight rows (4 tiles), lane l owns
// row 16*(4*blockIdx.x + l/16) + l%16; wave w of W takes k-blocks w, w+W, ...,
// loading up to 4 of them before it computes.  For a k-block the 16 code
// words of the lane's row are formed once and dotted with the 16 activation
// words of each token, which are the same for the whole wave.
// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(1024) void k_gemv_addsub(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                                      const float *__restrict__ gamma_p,
                                                      const int8_t *__restrict__ Xq, int64_t ldq,
                                                      const float *__restrict__ beta, int64_t M, int64_t N,
                                                      int64_t K, void *__restrict__ Y, int y_dtype, int64_t ldy)
{
    constexpr int DEPTH = 4;
    __shared__ int red[16][MT][64];
    __shared__ int qsum_part[16][MT];
    const int W = blockDim.x >> 6;
    const int wave = wave_id(), lane = lane_id();
    const int64_t tile = 4 * static_cast<int64_t>(blockIdx.x) + (lane >> 4);
    const int r = lane & 15;

    // sum_k q[m][k], for the correction of the offset codes
    {
        int part[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) part[t] = 0;
        const int64_t nwords = (K + 3) / 4;
        for (int64_t wi = threadIdx.x; wi < nwords; wi += blockDim.x) {
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

    float sc[MT]; // rescale factors, loaded before the product
    {
        const float gamma = *gamma_p;
#pragma unroll
        for (int t = 0; t < MT; ++t) sc[t] = t < M ? token_scale(gamma, beta[t]) : 0.0f;
    }
    int acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0;
    const int64_t KBF = K / 64; // k-blocks whose 64 activations are all in range
    const uint8_t *prow = P + tile * KB * 256 + r * 16;
    for (int64_t kb0 = wave; kb0 < KB; kb0 += static_cast<int64_t>(W) * DEPTH) {
        uint4 wv[DEPTH];
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
            const int64_t kb = kb0 + static_cast<int64_t>(j) * W;
            wv[j] = (tile < NT && kb < KB) ? *reinterpret_cast<const uint4 *>(prow + kb * 256)
                                           : make_uint4(I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD, I2_ZERO_WORD);
        }
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
            const int64_t kb = kb0 + static_cast<int64_t>(j) * W;
            if (kb >= KB) break;
            const uint32_t wd[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
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
                        for (int jj = 0; jj < 4; ++jj) {
                            int64_t k = kb * 64 + 4 * v + jj;
                            if (k < K) word |= (static_cast<uint32_t>(qp[4 * v + jj]) & 0xffu) << (8 * jj);
                        }
                        qd[v] = word;
                    }
                }
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
                    acc[t] = __builtin_amdgcn_sdot4(static_cast<int>(c[jj]), static_cast<int>(qd[jj]), acc[t], false);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
    const int64_t n = tile * 16 + r;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t >= M) break;
        int total = 0, qs = 0;
        for (int w = 0; w < W; ++w) {
            total += red[w][t][lane];
            qs += qsum_part[w][t];
        }
        if (n < N) store_out(Y, y_dtype, ldy, t, n, total - qs, sc[t]);
    }
}

// Shape choice of the MFMA GEMV: TW tiles per workgroup (reuse of each
// activation operand, worth it when many tokens make the activations a large
// share of the L2 -> CU traffic) and KS waves per workgroup (enough waves to
// cover the chip: about 16 per CU).
template <int LAYOUT, int TW>
static void launch_mfma_tw(const GemvArgs &a, int64_t KB, int64_t NT, int64_t nsteps, hipStream_t stream)
{
    const int64_t groups = (NT + TW - 1) / TW;
    const int64_t tgroups = (a.M + 15) / 16;
    const int64_t want_waves = 256 * 16;
    int64_t KS = (want_waves + groups * tgroups - 1) / (groups * tgroups);
    KS = KS < 1 ? 1 : KS;
    // at most 10 waves: with fewer, larger waves the cross-wave reduction is
    // shorter (measured 5-9 % faster than 13-16 waves on 3200- and 1024-row
    // layers, K = 3200 to 8640)
    KS = KS > 10 ? 10 : KS;
    KS = KS > nsteps ? nsteps : KS;
    dim3 grid(static_cast<unsigned>(groups), static_cast<unsigned>(tgroups));
    dim3 block(static_cast<unsigned>(KS * 64));
    constexpr int SB = 1;
    if (a.tiled)
        hipLaunchKernelGGL((k_gemv_mfma<LAYOUT, TW, SB, true>), grid, block, 0, stream, a.P, KB, NT, a.gamma, a.Xq,
                           a.ldq, a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy, a.pmax, a.pmax_cols);
    else
        hipLaunchKernelGGL((k_gemv_mfma<LAYOUT, TW, SB, false>), grid, block, 0, stream, a.P, KB, NT, a.gamma, a.Xq,
                           a.ldq, a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy, a.pmax, a.pmax_cols);
}

// Which matrix-core GEMV kernel runs for a shape.  Large layers: persistent
// workgroups with register-resident activations, when every CU gets at least
// two row tiles and the k-steps fit 16 waves x 4 (about one workgroup per CU
// in total, at most TMAX tiles each; the weight ring is guarded when a
// workgroup has only a few tiles).  Otherwise one workgroup per TW row tiles,
// reusing each activation operand over several tiles when there are many
// tokens (the activations are then a large share of the L2 -> CU traffic)
// and enough tiles to keep every CU busy.
struct GemvPlan {
    bool persist;
    int spw;     // persistent: k-steps per wave (1, 2 or 4)
    int tmax;    // persistent: most tiles per workgroup
    bool guard;  // persistent: ring loads skipped past the workgroup's tiles
    int64_t KS;  // persistent: waves per workgroup
    int64_t wgs; // persistent: workgroups per token group
    int tw;      // per-tile kernel: row tiles per workgroup (1, 2 or 4)
};

static GemvPlan gemv_plan(int layout, int64_t M, int64_t N, int64_t K)
{
    const int64_t NT = (N + 15) / 16;
    const int64_t KB = layout == LAYOUT_I2 ? (K + 63) / 64 : (layout == LAYOUT_B3 ? (K + 79) / 80 : (K + 127) / 128);
    const int64_t nsteps = (KB + 3) / 4;
    const int64_t tgroups = (M + 15) / 16;
    GemvPlan p{false, 0, 0, false, 0, 0, 1};
    // (b1 keeps 8 activation operands per k-step: four k-steps per wave would
    // not fit the registers, so it goes persistent only up to two)
    if (NT >= 512 * tgroups && nsteps <= (layout == LAYOUT_B1 ? 32 : 64)) {
        p.persist = true;
        p.KS = nsteps < 16 ? nsteps : 16;
        const int64_t spw = (nsteps + p.KS - 1) / p.KS;
        p.spw = spw <= 1 ? 1 : (spw <= 2 ? 2 : 4);
        p.tmax = p.spw >= 4 ? 4 : 8;
        int64_t wgs = 256 / tgroups;
        const int64_t min_wgs = (NT + p.tmax - 1) / p.tmax;
        wgs = wgs < min_wgs ? min_wgs : wgs;
        p.wgs = wgs > NT ? NT : wgs;
        p.guard = (NT + p.wgs - 1) / p.wgs <= 5;
        return p;
    }
    p.tw = (M > 4 && NT >= 1024) ? 4 : ((M > 4 && NT >= 512) ? 2 : 1);
    if (layout == LAYOUT_B1) p.tw = 1; // (operands of several tiles would spill)
    return p;
}

template <int LAYOUT, int SPW, int TMAX, bool TILED, bool GUARD>
static void launch_persist_kernel(const GemvArgs &a, int64_t KB, int64_t NT, dim3 grid, dim3 block, size_t lds,
                                  hipStream_t stream)
{
    auto *f = &k_gemv_persist<LAYOUT, SPW, TMAX, TILED, GUARD>;
    // more than 64 KiB of dynamic LDS must be allowed explicitly (a host-side
    // function attribute; nothing is enqueued)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(lds));
    hipLaunchKernelGGL(f, grid, block, lds, stream, a.P, KB, NT, a.gamma, a.Xq, a.ldq, a.beta, a.M, a.N, a.K, a.Y,
                       a.y_dtype, a.ldy, a.pmax, a.pmax_cols);
}

template <int LAYOUT, int SPW>
static void launch_persist(const GemvArgs &a, const GemvPlan &p, int64_t KB, int64_t NT, hipStream_t stream)
{
    constexpr int TMAX = SPW >= 4 ? 4 : 8;
    const int64_t tgroups = (a.M + 15) / 16;
    const size_t lds = static_cast<size_t>(TMAX) * p.KS * 4 * 64 * sizeof(int);
    dim3 grid(static_cast<unsigned>(p.wgs), static_cast<unsigned>(tgroups)), block(static_cast<unsigned>(p.KS * 64));
    if (a.tiled) {
        if (p.guard) launch_persist_kernel<LAYOUT, SPW, TMAX, true, true>(a, KB, NT, grid, block, lds, stream);
        else launch_persist_kernel<LAYOUT, SPW, TMAX, true, false>(a, KB, NT, grid, block, lds, stream);
    } else {
        if (p.guard) launch_persist_kernel<LAYOUT, SPW, TMAX, false, true>(a, KB, NT, grid, block, lds, stream);
        else launch_persist_kernel<LAYOUT, SPW, TMAX, false, false>(a, KB, NT, grid, block, lds, stream);
    }
}

int64_t gemv_mfma_parts(int layout, int64_t M, int64_t N, int64_t K)
{
    const GemvPlan p = gemv_plan(layout, M, N, K);
    const int64_t NT = (N + 15) / 16;
    return p.persist ? p.wgs : (NT + p.tw - 1) / p.tw;
}

template <int LAYOUT>
static void launch_mfma_layout(const GemvArgs &a, hipStream_t stream)
{
    const int64_t NT = (a.N + 15) / 16;
    const int64_t KB = (a.K + StepShape<LAYOUT>::KBLK - 1) / StepShape<LAYOUT>::KBLK;
    const int64_t nsteps = (KB + 3) / 4;
    const GemvPlan p = gemv_plan(LAYOUT, a.M, a.N, a.K);
    if (p.persist) {
        if (p.spw == 1) launch_persist<LAYOUT, 1>(a, p, KB, NT, stream);
        else if (p.spw == 2) launch_persist<LAYOUT, 2>(a, p, KB, NT, stream);
        else launch_persist<LAYOUT, 4>(a, p, KB, NT, stream);
        return;
    }
    if (p.tw == 4) launch_mfma_tw<LAYOUT, 4>(a, KB, NT, nsteps, stream);
    else if (p.tw == 2) launch_mfma_tw<LAYOUT, 2>(a, KB, NT, nsteps, stream);
    else launch_mfma_tw<LAYOUT, 1>(a, KB, NT, nsteps, stream);
}

// The GEMV with the quantiser inside: 1 to 4 tokens of fp32 / bf16 input,
// on the shapes and launch geometry of the kernel the int8 path would run:
// the per-tile kernel with one tile per workgroup (k_gemv_fq, at most 10
// waves, or up to FQ_MAX_WAVES where that shortens the per-wave template, at
// most FQ_MAX_SPW k-steps per wave, b1 2) or the persistent one
// (k_gemv_persist_fq, at most 2 k-steps per wave, b1 1), so that nothing
// spills, and LDS for the rounding areas and the persistent kernel's partial
// sums within the 160 KB of a CU.  Alignment
// is checked separately (gemv_fq_ok).
struct FqPlan {
    bool ok;
    bool persist;
    int64_t KS; // waves per workgroup
    int spw;    // k-steps per wave (1, 2 or 4)
    GemvPlan gp; // the persistent kernel's geometry
};

static FqPlan fq_plan(int layout, int64_t M, int64_t N, int64_t K, int x_dtype)
{
    FqPlan f{false, false, 0, 0, {}};
    // (16-token groups were measured slower than quantiser + GEMV: every
    // workgroup rounds all 16 x K values again; 2x on the 3B q layer)
    if (M < 1 || M > 4 || (x_dtype != DT_F32 && x_dtype != DT_BF16)) return f;
    const GemvPlan gp = gemv_plan(layout, M, N, K);
    const int64_t NT = (N + 15) / 16;
    const int64_t kblk = layout == LAYOUT_I2 ? 64 : (layout == LAYOUT_B3 ? 80 : 128);
    const int64_t nsteps = ((K + kblk - 1) / kblk + 3) / 4;
    const int64_t units = 4 * (4 * kblk / 16); // rounding units per k-step
    const int64_t max_spw = layout == LAYOUT_B1 ? 2 : FQ_MAX_SPW;
    if (gp.persist) {
        // (the weight ring and TMAX accumulators leave registers for at
        // most two k-steps per wave, one for b1)
        if (gp.spw > (layout == LAYOUT_B1 ? 1 : 2)) return f;
        const int64_t lds = static_cast<int64_t>(gp.tmax) * gp.KS * 4 * 64 * 4 +
                            FQ_PERSIST_WAVES * gp.spw * units * 16 + FQ_PERSIST_WAVES * 4 * 4;
        if (lds > 160 * 1024) return f;
        f.ok = true;
        f.persist = true;
        f.KS = gp.KS;
        f.spw = gp.spw;
        f.gp = gp;
        return f;
    }
    if (gp.tw != 1) return f;
    // About 16 waves per CU, at most 10 per workgroup; up to FQ_MAX_WAVES
    // where that moves the waves to a shorter template (SPW 4 -> 2 or 2 -> 1:
    // measured 5.64 -> 5.43 us on the 3B q layer, 9.7 -> 9.2 us on the b3
    // down layer; 16 waves that still need SPW 4 were slower, 8.0 -> 9.6 us).
    auto tmpl = [](int64_t spw) -> int64_t { return spw <= 1 ? 1 : (spw <= 2 ? 2 : 4); };
    const int64_t want = (256 * 16 + NT - 1) / NT;
    auto waves = [&](int64_t cap) {
        int64_t ks = want < 1 ? 1 : (want > cap ? cap : want);
        return ks > nsteps ? nsteps : ks;
    };
    int64_t KS = waves(10);
    const int64_t KSw = waves(FQ_MAX_WAVES);
    if (tmpl((nsteps + KSw - 1) / KSw) < tmpl((nsteps + KS - 1) / KS)) KS = KSw;
    const int64_t spw = (nsteps + KS - 1) / KS;
    if (spw > max_spw) return f;
    f.ok = true;
    f.KS = KS;
    f.spw = static_cast<int>(tmpl(spw));
    return f;
}

bool gemv_fq_shape(int layout, int64_t M, int64_t N, int64_t K, int x_dtype)
{
    return fq_plan(layout, M, N, K, x_dtype).ok;
}

bool gemv_fq_ok(int layout, int64_t M, int64_t N, int64_t K, int x_dtype, const void *X, int64_t ldx)
{
    if (!gemv_fq_shape(layout, M, N, K, x_dtype)) return false;
    const int64_t es = x_dtype == DT_F32 ? 4 : 2;
    if ((reinterpret_cast<uintptr_t>(X) & 15u) || (ldx * es) % 16) return false;
    return ((M - 1) * ldx + K) * es + 15 <= 0x7fffffff; // the buffer resource's byte range
}

template <int LAYOUT, int XDT, int SPW, int TMAX, bool GUARD>
static void launch_persist_fq_kernel(const GemvArgs &a, const void *X, int64_t ldx, int xbytes, int64_t KB,
                                     int64_t NT, const FqPlan &f, hipStream_t stream)
{
    auto *fn = &k_gemv_persist_fq<LAYOUT, XDT, SPW, TMAX, GUARD>;
    const size_t lds = static_cast<size_t>(TMAX) * f.KS * 4 * 64 * sizeof(int);
    // more than 64 KiB of LDS must be allowed explicitly (a host-side function
    // attribute; nothing is enqueued)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(lds));
    dim3 grid(static_cast<unsigned>(f.gp.wgs)), block(static_cast<unsigned>(f.KS * 64));
    hipLaunchKernelGGL(fn, grid, block, lds, stream, a.P, KB, NT, a.gamma, X, ldx, xbytes, a.M, a.N, a.K, a.Y,
                       a.y_dtype, a.ldy);
}

template <int LAYOUT, int XDT, int SPW>
static void launch_persist_fq(const GemvArgs &a, const void *X, int64_t ldx, int xbytes, int64_t KB, int64_t NT,
                              const FqPlan &f, hipStream_t stream)
{
    constexpr int TMAX = SPW >= 4 ? 4 : 8;
    if (f.gp.guard) launch_persist_fq_kernel<LAYOUT, XDT, SPW, TMAX, true>(a, X, ldx, xbytes, KB, NT, f, stream);
    else launch_persist_fq_kernel<LAYOUT, XDT, SPW, TMAX, false>(a, X, ldx, xbytes, KB, NT, f, stream);
}

template <int LAYOUT, int XDT>
static void launch_fq_x(const GemvArgs &a, const void *X, int64_t ldx, const FqPlan &f, hipStream_t stream)
{
    const int64_t NT = (a.N + 15) / 16;
    const int64_t KB = (a.K + StepShape<LAYOUT>::KBLK - 1) / StepShape<LAYOUT>::KBLK;
    constexpr int64_t ES = XDT == DT_F32 ? 4 : 2;
    const int xbytes = static_cast<int>((((a.M - 1) * ldx + a.K) * ES + 15) & ~int64_t(15));
    if (f.persist) {
        if (f.spw == 1) launch_persist_fq<LAYOUT, XDT, 1>(a, X, ldx, xbytes, KB, NT, f, stream);
        else if constexpr (LAYOUT != LAYOUT_B1) launch_persist_fq<LAYOUT, XDT, 2>(a, X, ldx, xbytes, KB, NT, f, stream);
        return;
    }
    dim3 grid(static_cast<unsigned>(NT)), block(static_cast<unsigned>(f.KS * 64));
    if (f.spw == 1) {
        hipLaunchKernelGGL((k_gemv_fq<LAYOUT, XDT, 1>), grid, block, 0, stream, a.P, KB, NT, a.gamma, X, ldx, xbytes,
                           a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy);
    } else if (f.spw == 2) {
        hipLaunchKernelGGL((k_gemv_fq<LAYOUT, XDT, 2>), grid, block, 0, stream, a.P, KB, NT, a.gamma, X, ldx, xbytes,
                           a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy);
    } else if constexpr (LAYOUT != LAYOUT_B1) {
        hipLaunchKernelGGL((k_gemv_fq<LAYOUT, XDT, 4>), grid, block, 0, stream, a.P, KB, NT, a.gamma, X, ldx, xbytes,
                           a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy);
    }
}

template <int LAYOUT>
static void launch_fq_layout(const GemvArgs &a, const void *X, int x_dtype, int64_t ldx, const FqPlan &f,
                             hipStream_t stream)
{
    if (x_dtype == DT_F32) launch_fq_x<LAYOUT, DT_F32>(a, X, ldx, f, stream);
    else launch_fq_x<LAYOUT, DT_BF16>(a, X, ldx, f, stream);
}

hipError_t launch_gemv_fq(const GemvArgs &a, const void *X, int x_dtype, int64_t ldx, hipStream_t stream)
{
    const FqPlan f = fq_plan(a.layout, a.M, a.N, a.K, x_dtype);
    if (!f.ok) return hipErrorInvalidValue;
    if (a.layout == LAYOUT_I2) launch_fq_layout<LAYOUT_I2>(a, X, x_dtype, ldx, f, stream);
    else if (a.layout == LAYOUT_B3) launch_fq_layout<LAYOUT_B3>(a, X, x_dtype, ldx, f, stream);
    else launch_fq_layout<LAYOUT_B1>(a, X, x_dtype, ldx, f, stream);
    return hipGetLastError();
}

void gemv_fq_kernel_name(int layout, int64_t M, int64_t N, int64_t K, int x_dtype, char *buf, size_t n)
{
    const FqPlan f = fq_plan(layout, M, N, K, x_dtype);
    if (f.persist)
        snprintf(buf, n, "bl::k_gemv_persist_fq<%d, %d, %d, %d, %s>", layout, x_dtype, f.spw, f.gp.tmax,
                 f.gp.guard ? "true" : "false");
    else
        snprintf(buf, n, "bl::k_gemv_fq<%d, %d, %d>", layout, x_dtype, f.spw);
}

void gemv_kernel_name(int layout, int64_t M, int64_t N, int64_t K, bool tiled, char *buf, size_t n)
{
    const GemvPlan p = gemv_plan(layout, M, N, K);
    if (p.persist)
        snprintf(buf, n, "bl::k_gemv_persist<%d, %d, %d, %s, %s>", layout, p.spw, p.tmax, tiled ? "true" : "false",
                 p.guard ? "true" : "false");
    else
        snprintf(buf, n, "bl::k_gemv_mfma<%d, %d, 1, %s>", layout, p.tw, tiled ? "true" : "false");
}

void gemv_addsub_kernel_name(int64_t M, char *buf, size_t n)
{
    snprintf(buf, n, "bl::k_gemv_addsub<%d>", M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 8 ? 8 : 16))));
}

hipError_t launch_gemv_mfma(const GemvArgs &a, hipStream_t stream)
{
    if (a.layout == LAYOUT_I2)
        launch_mfma_layout<LAYOUT_I2>(a, stream);
    else if (a.layout == LAYOUT_B3)
        launch_mfma_layout<LAYOUT_B3>(a, stream);
    else
        launch_mfma_layout<LAYOUT_B1>(a, stream);
    return hipGetLastError();
}

template <int MT>
static void launch_addsub_mt(const GemvArgs &a, int64_t KB, int64_t NT, hipStream_t stream)
{
    int64_t W = (KB + 3) / 4;
    W = W < 1 ? 1 : (W > 16 ? 16 : W);
    dim3 grid(static_cast<unsigned>((NT + 3) / 4));
    hipLaunchKernelGGL(k_gemv_addsub<MT>, grid, dim3(static_cast<unsigned>(W * 64)), 0, stream, a.P, KB, NT, a.gamma,
                       a.Xq, a.ldq, a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy);
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
