// act.hip -- per-token absmax int8 quantisation of BitLinear activations.
//
// LIT-380 record (dmarx anthology), Key takeaways, bullet 1: activations are
// 8-bit.  Reading: per token m, beta_m = max_k |x_mk| and
// q_mk = clamp(rint(x_mk * (127 / beta_m)), -127, 127) with ties to even, in
// binary32 with the row taken to the power-of-two scale where beta_m lies in
// [1, 2) (token_quant in common.h: one correctly rounded division per token,
// one rounding of each product; q = 0 for an all-zero row).
#include "common.h"
#include "launch.h"

namespace bl {

// Maximum of non-negative values over the workgroup (whole waves, every lane
// active): DPP within each wave, then LDS across the waves.
__device__ __forceinline__ float block_max(float v, float *red)
{
    v = wave_max_nonneg(v);
    const int nw = blockDim.x >> 6;
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < nw; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
}

// Generic path: one workgroup per token row; a thread handles groups of 4
// consecutive elements and writes them as one 32-bit word.
template <int XDT>
__global__ __launch_bounds__(256) void k_quant_act(const void *__restrict__ X, int64_t K, int64_t ldx,
                                                   int8_t *__restrict__ Xq, int64_t ldq,
                                                   float *__restrict__ beta)
{
    __shared__ float red[16];
    const int64_t m = blockIdx.x;
    const int64_t base = m * ldx;
    float amax = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += blockDim.x) amax = fmaxf(amax, fabsf(load_x<XDT>(X, base + k)));
    const float b = block_max(amax, red);
    const TokenQuant s = token_quant(b);
    uint32_t *qrow = reinterpret_cast<uint32_t *>(Xq + m * ldq);
    const int64_t nwords = ldq / 4;
    for (int64_t w = threadIdx.x; w < nwords; w += blockDim.x) {
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t k = 4 * w + j;
            uint32_t q = k < K ? quant_one(load_x<XDT>(X, base + k), s) : 0u;
            packed |= q << (8 * j);
        }
        qrow[w] = packed;
    }
    if (threadIdx.x == 0) beta[m] = b;
}

// Vector path (16-byte aligned rows, K a multiple of the vector width): every
// thread issues all its 16-byte loads of the row first (one memory round
// trip), keeps them in registers for the max and for the rounding.
template <int XDT, int VPT>
__global__ __launch_bounds__(1024) void k_quant_act_vec(const void *__restrict__ X, int64_t K, int64_t ldx,
                                                       int8_t *__restrict__ Xq, int64_t ldq,
                                                       float *__restrict__ beta)
{
    constexpr int EPV = XDT == DT_F32 ? 4 : 8; // elements per 16-byte vector
    __shared__ float red[16];
    const int64_t m = blockIdx.x;
    const int64_t nvec = K / EPV;
    const uint4 *row = reinterpret_cast<const uint4 *>(static_cast<const char *>(X) +
                                                       m * ldx * (XDT == DT_F32 ? 4 : 2));
    uint4 v[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int64_t vi = threadIdx.x + static_cast<int64_t>(j) * blockDim.x;
        v[j] = vi < nvec ? row[vi] : make_uint4(0u, 0u, 0u, 0u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (XDT == DT_F32) {
                amax = fmaxf(amax, fabsf(__uint_as_float(u[e])));
            } else {
                amax = fmaxf(amax, fabsf(__uint_as_float(u[e] << 16)));
                amax = fmaxf(amax, fabsf(__uint_as_float(u[e] & 0xffff0000u)));
            }
        }
    }
    const float b = block_max(amax, red);
    const TokenQuant s = token_quant(b);
    int8_t *qrow = Xq + m * ldq;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int64_t vi = threadIdx.x + static_cast<int64_t>(j) * blockDim.x;
        if (vi >= nvec) continue;
        const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        if constexpr (XDT == DT_F32) {
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) w |= quant_one(__uint_as_float(u[e]), s) << (8 * e);
            reinterpret_cast<uint32_t *>(qrow)[vi] = w;
        } else {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                w0 |= quant_one(__uint_as_float(u[e] << 16), s) << (16 * e);
                w0 |= quant_one(__uint_as_float(u[e] & 0xffff0000u), s) << (16 * e + 8);
                w1 |= quant_one(__uint_as_float(u[e + 2] << 16), s) << (16 * e);
                w1 |= quant_one(__uint_as_float(u[e + 2] & 0xffff0000u), s) << (16 * e + 8);
            }
            reinterpret_cast<uint2 *>(qrow)[vi] = make_uint2(w0, w1);
        }
    }
    // zero the row padding [K, ldq)
    for (int64_t k = K + 4 * threadIdx.x; k < ldq; k += 4 * blockDim.x)
        *reinterpret_cast<uint32_t *>(qrow + k) = 0u;
    if (threadIdx.x == 0) beta[m] = b;
}

// Many tokens (prefill): one wave per token row, 4 rows per workgroup.  A
// lane issues all its 16-byte loads of the row (VPL of them) first, the row
// maximum is a DPP reduction inside the wave (no barrier), and the lane
// rounds and stores its own vectors.  Many more rows are in flight per CU
// than with a workgroup per row.  Same arithmetic as k_quant_act_vec.
constexpr int ROWS_WAVES = 4;
template <int XDT, int VPL>
__global__ __launch_bounds__(64 * ROWS_WAVES) void k_quant_act_rows(const void *__restrict__ X, int64_t M, int64_t K,
                                                                    int64_t ldx, int8_t *__restrict__ Xq, int64_t ldq,
                                                                    float *__restrict__ beta)
{
    constexpr int EPV = XDT == DT_F32 ? 4 : 8; // elements per 16-byte vector
    const int64_t m = static_cast<int64_t>(blockIdx.x) * ROWS_WAVES + wave_id();
    if (m >= M) return; // (whole wave: the reduction below stays within one row)
    const int lane = lane_id();
    const int64_t nvec = K / EPV;
    const uint4 *row = reinterpret_cast<const uint4 *>(static_cast<const char *>(X) +
                                                       m * ldx * (XDT == DT_F32 ? 4 : 2));
    uint4 v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int64_t vi = lane + 64 * static_cast<int64_t>(j);
        v[j] = vi < nvec ? row[vi] : make_uint4(0u, 0u, 0u, 0u);
    }
    // |x| as bit patterns: non-negative binary32 / bfloat16 values order like
    // their bits, so the maximum is an unsigned integer maximum (bf16: two
    // halves at a time), with no unpacking to floats
    float amax;
    if constexpr (XDT == DT_F32) {
        uint32_t mb = 0;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) mb = max(mb, u[e] & 0x7fffffffu);
        }
        amax = __uint_as_float(mb);
    } else {
        typedef unsigned short us2 __attribute__((ext_vector_type(2)));
        us2 mb = {0, 0};
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) mb = __builtin_elementwise_max(mb, __builtin_bit_cast(us2, u[e] & 0x7fff7fffu));
        }
        amax = __uint_as_float(static_cast<uint32_t>(mb[0] > mb[1] ? mb[0] : mb[1]) << 16);
    }
    const float b = wave_max_nonneg(amax);
    const TokenQuant s = token_quant(b);
    int8_t *qrow = Xq + m * ldq;
    // every |x| <= b, the row's own maximum: the bounded rounding applies
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int64_t vi = lane + 64 * static_cast<int64_t>(j);
        if (vi >= nvec) continue;
        const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        if constexpr (XDT == DT_F32) {
            reinterpret_cast<uint32_t *>(qrow)[vi] = quant4_bounded(__uint_as_float(u[0]), __uint_as_float(u[1]),
                                                                    __uint_as_float(u[2]), __uint_as_float(u[3]), s);
        } else {
            auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
            auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
            reinterpret_cast<uint2 *>(qrow)[vi] =
                make_uint2(quant4_bounded(lo(u[0]), hi(u[0]), lo(u[1]), hi(u[1]), s),
                           quant4_bounded(lo(u[2]), hi(u[2]), lo(u[3]), hi(u[3]), s));
        }
    }
    // zero the row padding [K, ldq)
    for (int64_t k = K + 4 * lane; k < ldq; k += 4 * 64) *reinterpret_cast<uint32_t *>(qrow + k) = 0u;
    if (lane == 0) beta[m] = b;
}

template <int XDT>
static bool launch_vec(const void *X, int64_t M, int64_t K, int64_t ldx, int8_t *Xq, int64_t ldq, float *beta,
                       hipStream_t stream)
{
    constexpr int EPV = XDT == DT_F32 ? 4 : 8;
    constexpr int ES = XDT == DT_F32 ? 4 : 2;
    if (K % EPV || (ldx * ES) % 16 || (reinterpret_cast<uintptr_t>(X) & 15)) return false;
    const int64_t nvec = K / EPV;
    // many tokens: a wave per row, when a lane's share of the row fits its
    // registers (K up to 6144 fp32 / 12288 bf16)
    if (M >= 64 && nvec <= 64 * 24) {
        const int64_t vpl = (nvec + 63) / 64;
        dim3 grid(static_cast<unsigned>((M + ROWS_WAVES - 1) / ROWS_WAVES)), block(64 * ROWS_WAVES);
        if (vpl <= 4) hipLaunchKernelGGL((k_quant_act_rows<XDT, 4>), grid, block, 0, stream, X, M, K, ldx, Xq, ldq, beta);
        else if (vpl <= 8) hipLaunchKernelGGL((k_quant_act_rows<XDT, 8>), grid, block, 0, stream, X, M, K, ldx, Xq, ldq, beta);
        else if (vpl <= 12) hipLaunchKernelGGL((k_quant_act_rows<XDT, 12>), grid, block, 0, stream, X, M, K, ldx, Xq, ldq, beta);
        else if (vpl <= 16) hipLaunchKernelGGL((k_quant_act_rows<XDT, 16>), grid, block, 0, stream, X, M, K, ldx, Xq, ldq, beta);
        else if (vpl <= 20) hipLaunchKernelGGL((k_quant_act_rows<XDT, 20>), grid, block, 0, stream, X, M, K, ldx, Xq, ldq, beta);
        else hipLaunchKernelGGL((k_quant_act_rows<XDT, 24>), grid, block, 0, stream, X, M, K, ldx, Xq, ldq, beta);
        return true;
    }
    // about one 16-byte vector per thread (up to 1024 threads): the row's
    // loads all go out at once and each thread rounds only a few elements
    const int64_t threads = nvec <= 64 ? 64 : (nvec >= 1024 ? 1024 : (nvec + 63) / 64 * 64);
    const int64_t vpt = (nvec + threads - 1) / threads;
    dim3 grid(static_cast<unsigned>(M)), block(static_cast<unsigned>(threads));
    if (vpt <= 1) hipLaunchKernelGGL((k_quant_act_vec<XDT, 1>), grid, block, 0, stream, X, K, ldx, Xq, ldq, beta);
    else if (vpt <= 2) hipLaunchKernelGGL((k_quant_act_vec<XDT, 2>), grid, block, 0, stream, X, K, ldx, Xq, ldq, beta);
    else if (vpt <= 4) hipLaunchKernelGGL((k_quant_act_vec<XDT, 4>), grid, block, 0, stream, X, K, ldx, Xq, ldq, beta);
    else if (vpt <= 8) hipLaunchKernelGGL((k_quant_act_vec<XDT, 8>), grid, block, 0, stream, X, K, ldx, Xq, ldq, beta);
    else if (vpt <= 16) hipLaunchKernelGGL((k_quant_act_vec<XDT, 16>), grid, block, 0, stream, X, K, ldx, Xq, ldq, beta);
    else return false;
    return true;
}

hipError_t launch_quant_act(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t *Xq,
                            int64_t ldq, float *beta, hipStream_t stream)
{
    bool done = x_dtype == DT_F32 ? launch_vec<DT_F32>(X, M, K, ldx, Xq, ldq, beta, stream)
                                  : launch_vec<DT_BF16>(X, M, K, ldx, Xq, ldq, beta, stream);
    if (!done) {
        if (x_dtype == DT_F32)
            hipLaunchKernelGGL(k_quant_act<DT_F32>, dim3(static_cast<unsigned>(M)), dim3(256), 0, stream, X, K, ldx,
                               Xq, ldq, beta);
        else
            hipLaunchKernelGGL(k_quant_act<DT_BF16>, dim3(static_cast<unsigned>(M)), dim3(256), 0, stream, X, K, ldx,
                               Xq, ldq, beta);
    }
    return hipGetLastError();
}

} // namespace bl

namespace bl {

// Tiled activation layout (bitlinear.h): one workgroup per token row m of the
// G*16 padded rows, up to 1024 threads.  A thread owns whole 16-element
// pieces of the row (16 consecutive k: one 16-byte operand slice; about one
// piece per thread), loads them all before the max, then quantises from
// registers and stores each piece with one 16-byte store.
template <int XDT, int PPT>
__device__ __forceinline__ void quant_tiled_row(const void *__restrict__ X, int64_t M, int64_t K, int64_t ldx,
                                                int layout, int64_t nsteps, int8_t *__restrict__ Xt,
                                                float *__restrict__ beta, int64_t m, float *red,
                                                const float *__restrict__ pmax = nullptr, int64_t nparts = 0)
{
    constexpr int ES = XDT == DT_F32 ? 4 : 2;
    const int64_t step_k = layout == LAYOUT_I2 ? 256 : (layout == LAYOUT_B3 ? 320 : 512), kblk = step_k / 4;
    const int64_t nmf = layout == LAYOUT_I2 ? 4 : (layout == LAYOUT_B3 ? 5 : 8);
    const int64_t npieces = nsteps * step_k / 16;
    const int64_t tg = m / 16, i = m % 16;
    const bool live_row = m < M;
    const char *row = static_cast<const char *>(X) + (live_row ? m : 0) * ldx * ES;
    const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
    float v[PPT][16];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int64_t p = threadIdx.x + static_cast<int64_t>(j) * blockDim.x;
        const int64_t k0 = 16 * p;
        if (live_row && p < npieces && k0 + 16 <= K && vec) {
            if constexpr (XDT == DT_F32) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 u = reinterpret_cast<const uint4 *>(row + k0 * 4)[q];
                    v[j][4 * q] = __uint_as_float(u.x); v[j][4 * q + 1] = __uint_as_float(u.y);
                    v[j][4 * q + 2] = __uint_as_float(u.z); v[j][4 * q + 3] = __uint_as_float(u.w);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint4 u = reinterpret_cast<const uint4 *>(row + k0 * 2)[q];
                    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[j][8 * q + 2 * e] = __uint_as_float(w[e] << 16);
                        v[j][8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                    }
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                v[j][e] = (live_row && p < npieces && k0 + e < K) ? load_x<XDT>(X, m * ldx + k0 + e) : 0.0f;
        }
        if (pmax == nullptr) {
#pragma unroll
            for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
        }
    }
    // producer-side maxima (the previous product's epilogue wrote each of its
    // workgroups' maximum of |x| per token over exactly these K columns): the
    // row maximum without a pass over the values
    if (pmax != nullptr && live_row)
        for (int64_t p = threadIdx.x; p < nparts; p += blockDim.x) amax = fmaxf(amax, pmax[p * 16 + i]);
    const float b = block_max(amax, red);
    const TokenQuant s = token_quant(b);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int64_t p = threadIdx.x + static_cast<int64_t>(j) * blockDim.x;
        if (p >= npieces) break;
        const int64_t k0 = 16 * p;
        const int64_t st = k0 / step_k, r = k0 % step_k, g = r / kblk, d = (r % kblk) / 16;
        uint32_t w[4] = {0, 0, 0, 0};
        if (pmax == nullptr) {
            // beta is this row's own maximum, so every |x| <= beta: the
            // bounded rounding gives the same bytes
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = quant4_bounded(v[j][4 * q], v[j][4 * q + 1], v[j][4 * q + 2], v[j][4 * q + 3], s);
        } else {
            // beta from the producer's maxima: the clamped form
#pragma unroll
            for (int e = 0; e < 16; ++e) w[e / 4] |= quant_one(v[j][e], s) << (8 * (e % 4));
        }
        const int64_t off = (((tg * nsteps + st) * nmf + d) * 64 + g * 16 + i) * 16;
        *reinterpret_cast<uint4 *>(Xt + off) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (threadIdx.x == 0 && live_row) beta[m] = b;
}

template <int XDT, int PPT>
__global__ __launch_bounds__(1024) void k_quant_act_tiled(const void *__restrict__ X, int64_t M, int64_t K,
                                                         int64_t ldx, int layout, int64_t nsteps,
                                                         int8_t *__restrict__ Xt, float *__restrict__ beta,
                                                         const float *__restrict__ pmax, int64_t nparts)
{
    __shared__ float red[16];
    quant_tiled_row<XDT, PPT>(X, M, K, ldx, layout, nsteps, Xt, beta, blockIdx.x, red, pmax, nparts);
}

// Several inputs in one launch (the grouped forward): workgroup (m, u)
// quantises real token row m of input u (no padding rows: the grouped GEMV
// never reads tokens past M), as k_quant_act_tiled quantises it.
template <int XDT, int PPT>
__global__ __launch_bounds__(1024) void k_group_quant_tiled(const GroupQuantArgs args)
{
    __shared__ float red[16];
    const GroupInput &in = args.in[blockIdx.y];
    if (static_cast<int>(blockIdx.x) >= in.M) return; // (whole workgroup)
    quant_tiled_row<XDT, PPT>(in.X, in.M, in.K, in.ldx, args.layout, in.nsteps, in.Xt, in.beta, blockIdx.x, red);
}

template <int XDT>
static bool launch_group_quant_x(const GroupQuantArgs &args, int max_m, int64_t max_npieces, hipStream_t stream)
{
    const int64_t threads = max_npieces >= 1024 ? 1024 : (max_npieces + 63) / 64 * 64;
    const int64_t ppt = (max_npieces + threads - 1) / threads;
    dim3 grid(static_cast<unsigned>(max_m), static_cast<unsigned>(args.ninputs)), block(static_cast<unsigned>(threads));
    if (ppt <= 1) hipLaunchKernelGGL((k_group_quant_tiled<XDT, 1>), grid, block, 0, stream, args);
    else if (ppt <= 2) hipLaunchKernelGGL((k_group_quant_tiled<XDT, 2>), grid, block, 0, stream, args);
    else if (ppt <= 4) hipLaunchKernelGGL((k_group_quant_tiled<XDT, 4>), grid, block, 0, stream, args);
    else if (ppt <= 8) hipLaunchKernelGGL((k_group_quant_tiled<XDT, 8>), grid, block, 0, stream, args);
    else return false;
    return true;
}

hipError_t launch_group_quant(const GroupQuantArgs &args, int x_dtype, hipStream_t stream)
{
    int max_m = 1;
    int64_t max_np = 1;
    for (int u = 0; u < args.ninputs; ++u) {
        max_m = args.in[u].M > max_m ? args.in[u].M : max_m;
        const int64_t np = args.in[u].nsteps * tiled_step_k(args.layout) / 16;
        max_np = np > max_np ? np : max_np;
    }
    const bool ok = x_dtype == DT_F32 ? launch_group_quant_x<DT_F32>(args, max_m, max_np, stream)
                                      : launch_group_quant_x<DT_BF16>(args, max_m, max_np, stream);
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

template <int XDT>
static bool launch_tiled_ppt(const void *X, int64_t M, int64_t K, int64_t ldx, int layout, int8_t *Xt, float *beta,
                             const float *pmax, int64_t nparts, hipStream_t stream)
{
    const int64_t nsteps = tiled_nsteps(K, layout);
    const int64_t npieces = nsteps * tiled_step_k(layout) / 16;
    const int64_t threads = npieces >= 1024 ? 1024 : (npieces + 63) / 64 * 64;
    const int64_t ppt = (npieces + threads - 1) / threads;
    dim3 grid(static_cast<unsigned>((M + 15) / 16 * 16)), block(static_cast<unsigned>(threads));
#define BL_TILED(N) hipLaunchKernelGGL((k_quant_act_tiled<XDT, N>), grid, block, 0, stream, X, M, K, ldx, layout, nsteps, Xt, beta, pmax, nparts)
    // (K <= 65536 for the tiled layout: at most 4096 pieces for i2 and b1,
    // 4100 for b3, whose last few take the 8-piece variant)
    if (ppt <= 1) BL_TILED(1);
    else if (ppt <= 2) BL_TILED(2);
    else if (ppt <= 4) BL_TILED(4);
    else if (ppt <= 8) BL_TILED(8);
    else return false;
#undef BL_TILED
    return true;
}

hipError_t launch_quant_act_tiled(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int layout,
                                  int8_t *Xt, float *beta, hipStream_t stream, const float *pmax, int64_t nparts)
{
    const bool ok = x_dtype == DT_F32 ? launch_tiled_ppt<DT_F32>(X, M, K, ldx, layout, Xt, beta, pmax, nparts, stream)
                                      : launch_tiled_ppt<DT_BF16>(X, M, K, ldx, layout, Xt, beta, pmax, nparts, stream);
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

} // namespace bl
