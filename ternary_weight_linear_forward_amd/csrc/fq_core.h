// fq_core.h -- the per-token activation quantiser inside the decode GEMVs
// (1 to 4 tokens of fp32 / bf16 rows), shared by the single-layer GEMVs
// (gemv.hip) and the grouped one (group.hip).
#pragma once

#include "common.h"
#include "gemv_core.h"

namespace bl {

// ---------------------------------------------------------------------------
// The per-token quantiser inside the decode GEMVs, for 1 to 4 tokens given as
// fp32 or bf16 rows (16-byte aligned): every workgroup quantises the few KB of
// activations itself, so the forward is one launch instead of quantiser +
// GEMV.  In each wave (owning k-steps wave + j KS, j < nj):
//  1. fq_load issues the loads of the wave's own activations (4 tokens x
//     STEP_K values per k-step, as 16-value units: unit u = (j M + token) CH
//     + chunk, dealt to lane u % 64), then the caller issues its weight
//     loads, all before the first wait.  Waits count loads in issue order,
//     so the activations are waited for without waiting for the weights.
//  2. fq_quantise: beta_m = max |x_mk| of the wave's values, across the wave
//     by DPP and across the waves through LDS (one barrier); the values are
//     rounded exactly as the quantiser rounds them (bit-identical to
//     bitlinear_quantize_act) and pass through a per-wave LDS area into the
//     MFMA operand layout: lane (i, g), operand d takes token i's 16 values
//     at chunk NMF g + d of the k-step.
//  3. The kernel's own products, cross-wave sum and rescale.
// ---------------------------------------------------------------------------
constexpr int FQ_MAX_WAVES = 16; // per-tile kernel (10 unless more waves shorten the per-wave template)
constexpr int FQ_MAX_SPW = 4;

__device__ __forceinline__ uint4 buffer_load_16(const void *base, int nbytes, int voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nbytes, 0x00020000);
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
#else
    (void)base, (void)nbytes, (void)voff;
    return make_uint4(0u, 0u, 0u, 0u);
#endif
}

// This lane's activation units (see above) and their geometry.
template <int LAYOUT, int XDT, int SPW>
struct FqUnits {
    static constexpr int NMF = StepShape<LAYOUT>::NMF;
    static constexpr int STEP_K = 4 * StepShape<LAYOUT>::KBLK;
    static constexpr int CH = STEP_K / 16;               // 16-value chunks per token per k-step (i2 16, b3 20, b1 32)
    static constexpr int UNITS = 4 * CH;                 // units per k-step (4 tokens)
    static constexpr int NUW = (SPW * UNITS + 63) / 64;  // unit slots per lane
    static constexpr int ES = XDT == DT_F32 ? 4 : 2;     // bytes per value
    static constexpr int VL = ES;                        // 16-byte loads per unit (16 values)
    int lane, wave, KS, mtok, nunits, K32, ldx32;

    struct Unit {
        int j, tok, c, k0, nv; // k-step slot, token, chunk, first k, values before K (0: dead slot)
    };
    // recomputed where needed rather than kept in registers
    __device__ __forceinline__ Unit unit(int n) const
    {
        Unit r;
        const int u = lane + 64 * n;
        const bool live = u < nunits;
        const int uu = live ? u : 0;
        const int t = uu / CH; // t = j M + token
        r.c = uu - t * CH;
        // t / M for M = 1..4 without a division ((t * 0xAAAB) >> 17 is t / 3 below 2^15)
        r.j = mtok == 1 ? t : (mtok == 2 ? t >> 1 : (mtok == 4 ? t >> 2 : static_cast<int>((t * 0xAAABu) >> 17)));
        r.tok = t - r.j * mtok;
        r.k0 = (wave + r.j * KS) * STEP_K + 16 * r.c;
        const int left = K32 - r.k0;
        r.nv = live ? (left <= 0 ? 0 : (left < 16 ? left : 16)) : 0;
        return r;
    }
};

// Issue this lane's activation loads.  Dead unit slots and values past K read
// an in-bounds place (zeroed later); the resource ends at the last row's value
// K rounded up to 16 bytes (xbytes), and reads past it return zeros.
template <class FU>
__device__ __forceinline__ void fq_load(const FU &U, const void *X, int xbytes, uint4 (&xv)[FU::NUW][FU::VL])
{
#pragma unroll
    for (int n = 0; n < FU::NUW; ++n) {
        const auto un = U.unit(n);
        const int off = (un.tok * U.ldx32 + (un.k0 < U.K32 ? un.k0 : 0)) * FU::ES;
#pragma unroll
        for (int v = 0; v < FU::VL; ++v) xv[n][v] = buffer_load_16(X, xbytes, off + 16 * v);
    }
}

// Absmax, rounding and regroup (every wave of the workgroup must call it: it
// holds a barrier).  qbuf: this wave's LDS area, SPW x UNITS units; wmax:
// [waves][4].  Fills a[j][d] for the wave's k-steps j < nj and returns, in lane
// t, beta of token t % 4 (a lane shuffle of the result gives any token's).
// after_barrier() runs in every wave right after the barrier (the grouped GEMV
// issues its weight loads there, once every wave of the workgroup holds its
// activations).
struct FqNoHook {
    __device__ void operator()() const {}
};

template <class FU, int SPW, class Hook = FqNoHook>
__device__ __forceinline__ float fq_quantise(const FU &U, uint4 (&xv)[FU::NUW][FU::VL], v4i *qbuf, float (*wmax)[4],
                                             v4i (&a)[SPW][FU::NMF], const Hook &after_barrier = Hook())
{
    constexpr int XF32 = FU::ES == 4;
    const int lane = U.lane, wave = U.wave;
    // the 16-value unit as 16 binary32 bit patterns (bf16: value e is the
    // upper or lower half of dword e / 2)
    auto bits = [&](int n, int e) -> uint32_t {
        const uint4 q = xv[n][XF32 ? e / 4 : e / 8];
        const int w = XF32 ? e % 4 : (e % 8) / 2;
        const uint32_t d = w == 0 ? q.x : (w == 1 ? q.y : (w == 2 ? q.z : q.w));
        if constexpr (XF32) return d;
        else return (e & 1) ? (d & 0xffff0000u) : (d << 16);
    };
    // zero the values at or past K of the unit that holds K, and whole dead
    // slots (a lane-divergent branch, taken by few lanes)
#pragma unroll
    for (int n = 0; n < FU::NUW; ++n) {
        const int nv = U.unit(n).nv;
        if (nv < 16) {
#pragma unroll
            for (int v = 0; v < FU::VL; ++v) {
                uint32_t w4[4] = {xv[n][v].x, xv[n][v].y, xv[n][v].z, xv[n][v].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int e0 = (XF32 ? 4 : 8) * v + (XF32 ? 1 : 2) * w; // first value of the dword
                    uint32_t keep;
                    if constexpr (XF32) keep = e0 < nv ? 0xffffffffu : 0u;
                    else keep = (e0 < nv ? 0x0000ffffu : 0u) | (e0 + 1 < nv ? 0xffff0000u : 0u);
                    w4[w] &= keep;
                }
                xv[n][v] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            }
        }
    }
    float amax[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int n = 0; n < FU::NUW; ++n) {
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(__uint_as_float(bits(n, e))));
        const int tok = U.unit(n).tok;
#pragma unroll
        for (int t = 0; t < 4; ++t) amax[t] = tok == t ? fmaxf(amax[t], m) : amax[t];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float b = wave_max_nonneg(amax[t]);
        if (lane == t) wmax[wave][t] = b;
    }
    __syncthreads();
    after_barrier();
    float beta_lane;
    {
        const int t = lane & 3;
        float b = wmax[0][t];
        for (int w = 1; w < U.KS; ++w) b = fmaxf(b, wmax[w][t]);
        beta_lane = b;
    }
    // q = rint(fl32(x pre s)) as quant_one computes it: every |x| <= beta, so
    // |fl32(x pre s)| <= 127 (1 + 2^-24)^2 < 127.5 and the clamp never acts
    // (s is finite for every beta: token_quant);
    // adding 1.5 * 2^23 (a separate, correctly rounded add: the build does
    // not contract) rounds to an integer with ties to even, which then sits
    // in the low bits of the sum (two's complement in its low byte).
#pragma unroll
    for (int n = 0; n < FU::NUW; ++n) {
        const auto un = U.unit(n);
        const TokenQuant st = token_quant(__shfl(beta_lane, un.tok)); // (every lane active here)
        if (lane + 64 * n >= U.nunits) continue;
        uint32_t w4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = token_scaled(__uint_as_float(bits(n, 4 * q + e)), st);
                b[e] = __float_as_uint(v + 12582912.0f);
            }
            const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
            const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
            w4[q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
        qbuf[un.j * FU::UNITS + un.tok * FU::CH + un.c] = v4i{static_cast<int>(w4[0]), static_cast<int>(w4[1]),
                                                             static_cast<int>(w4[2]), static_cast<int>(w4[3])};
    }
    // the other lanes of this wave read what it wrote: order the LDS accesses
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // operand d of lane (i, g): token i's chunk NMF g + d (tokens past M and
    // 4..15 read copies or stale data: their outputs are never stored)
    const int i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
        for (int d = 0; d < FU::NMF; ++d) a[j][d] = qbuf[j * FU::UNITS + (i & 3) * FU::CH + FU::NMF * g + d];
    return beta_lane;
}

} // namespace bl
