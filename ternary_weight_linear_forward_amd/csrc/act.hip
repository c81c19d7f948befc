// act.hip -- per-token absmax int8 quantisation of BitLinear activations.
//
// LIT-380 record (dmarx anthology), Key takeaways, bullet 1: activations are
// 8-bit.  Reading: per token m, beta_m = max_k |x_mk|, s_m = 127 / beta_m
// (correctly rounded binary32 division; s_m = 0 when beta_m = 0), and
// q_mk = clamp(rint(x_mk * s_m), -127, 127) with ties to even.
#include "common.h"
#include "launch.h"

namespace bl {

template <int XDT>
__device__ __forceinline__ float load_x(const void *X, int64_t idx)
{
    if constexpr (XDT == DT_F32)
        return static_cast<const float *>(X)[idx];
    else
        return bf16_bits_to_float(static_cast<const uint16_t *>(X)[idx]);
}

__device__ __forceinline__ float block_max_256(float v, float *red)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}

__device__ __forceinline__ int quant_one(float x, float s)
{
    float r = __builtin_rintf(x * s);
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return static_cast<int>(r);
}

// One workgroup of 256 threads per token row; a thread handles groups of
// 4 consecutive elements and writes them as one 32-bit word.
template <int XDT>
__global__ __launch_bounds__(256) void k_quant_act(const void *__restrict__ X, int64_t K, int64_t ldx,
                                                   int8_t *__restrict__ Xq, int64_t ldq,
                                                   float *__restrict__ beta)
{
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const int64_t base = m * ldx;
    float amax = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += 256) amax = fmaxf(amax, fabsf(load_x<XDT>(X, base + k)));
    const float b = block_max_256(amax, red);
    const float s = b > 0.0f ? 127.0f / b : 0.0f;
    uint32_t *qrow = reinterpret_cast<uint32_t *>(Xq + m * ldq);
    const int64_t nwords = ldq / 4;
    for (int64_t w = threadIdx.x; w < nwords; w += 256) {
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t k = 4 * w + j;
            int q = k < K ? quant_one(load_x<XDT>(X, base + k), s) : 0;
            packed |= (static_cast<uint32_t>(q) & 0xffu) << (8 * j);
        }
        qrow[w] = packed;
    }
    if (threadIdx.x == 0) beta[m] = b;
}

hipError_t launch_quant_act(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t *Xq,
                            int64_t ldq, float *beta, hipStream_t stream)
{
    if (x_dtype == DT_F32)
        hipLaunchKernelGGL(k_quant_act<DT_F32>, dim3(static_cast<unsigned>(M)), dim3(256), 0, stream, X, K, ldx, Xq,
                           ldq, beta);
    else
        hipLaunchKernelGGL(k_quant_act<DT_BF16>, dim3(static_cast<unsigned>(M)), dim3(256), 0, stream, X, K, ldx, Xq,
                           ldq, beta);
    return hipGetLastError();
}

} // namespace bl
