// group.hip -- many decode BitLinears (at most 16 tokens each) in one product
// launch.
//
// LIT-380 record (dmarx anthology), closing section: on stock GPUs the memory
// saving of ternary weights is what survives, so a decode product is an HBM
// stream of packed weights.  One BitLinear of a 3B layer is only 2.6-6.9 MB
// of weights: alone it cannot fill the chip before its launch ends.  Here
// every layer of a group (e.g. the q, k, v, o, gate, up and down projections
// of a decode step) is one job of a single persistent launch, so the whole
// group streams as one.
//
// Layout of the launch: the workgroups are dealt to the jobs in proportion to
// their weight bytes (plan below).  A workgroup serves one job: it takes the
// job's 16-row tiles lb, lb + nwg, lb + 2 nwg, ... (lb its index among the
// job's nwg workgroups, so that the job's workgroups stream neighbouring tiles
// at the same time), and its waves split the job's k-steps (wave w takes steps
// w, w + KS, ...).  Each wave loads the int8 activation operands of its
// k-steps once (the tiled layout, token group 0) and keeps them in registers,
// then streams its chunk of every tile through a ring of D tiles of weight
// loads in flight.  The waves never wait for each other while they stream:
// each adds its partial 16 x 16 result of a tile into the tile's int32 sums in
// LDS with integer atomics (exact in any order), and after one barrier at the
// end the tiles are rescaled and stored, so no store interleaves with the ring
// loads.
#include <cstdio>
#include <type_traits>

#include "common.h"
#include "gemv_core.h"
#include "launch.h"

namespace bl {

namespace {
constexpr int GROUP_WAVES = 16; // most waves per workgroup (the plan's limit)

// s_waitcnt immediate: every LDS access of this wave done (lgkmcnt 0), vector
// memory and export counters left alone (gfx9 encoding).
constexpr int kLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// f(integral_constant<int, T>) for T = T0, T0 + 1, ... while it returns true
// (below T1), as straight-line code.
template <int T0, int T1, class F>
__device__ __forceinline__ void unroll_while(F &&f)
{
    if constexpr (T0 < T1) {
        if (f(std::integral_constant<int, T0>{})) unroll_while<T0 + 1, T1>(f);
    }
}

__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
} // namespace

// Weight tiles in flight per wave for a job of SPW k-steps per wave: as many
// as the registers left next to the activation operands hold without
// spilling (about 8-12 KB per wave).
constexpr int group_depth(int layout, int spw)
{
    return layout == LAYOUT_I2 ? (spw == 1 ? 10 : (spw == 2 ? 5 : 3))
           : layout == LAYOUT_B3 ? (spw == 1 ? 8 : (spw == 2 ? 4 : 2))
                                 : (spw == 1 ? 5 : 2);
}

// One job's share of a workgroup: this wave's k-steps (nj of them, at most
// SPW) of the row tiles lb, lb + nwg, ... (ntiles of them), D tiles of weight
// loads in flight; each tile's partial sums go into sums[t] by LDS atomics.
template <int LAYOUT, int SPW, int D, class Z>
__device__ __forceinline__ void group_job_tiles(const GroupJob &J, int KS, int wave, int lane, int nj, int lb,
                                                int ntiles, int (*sums)[4][64], const Z &zero_sums)
{
    using S = StepShape<LAYOUT>;
    constexpr int NMF = S::NMF;
    const int M = J.M, KB = J.KB, nsteps = J.nsteps;
    const int i = lane & 15, g = lane >> 4;
    // activation operands of this wave's k-steps, once.  Lanes of tokens
    // past M read token 0's bytes (the same cache lines) and drop them.
    v4i a[SPW][NMF];
    const int lane_a = i < M ? lane : (lane & ~15);
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int s = wave + j * KS;
        const int sx = s < nsteps ? s : nsteps - 1;
#pragma unroll
        for (int d = 0; d < NMF; ++d) {
            const v4i v = *reinterpret_cast<const v4i *>(J.Xt + ((static_cast<int64_t>(sx) * NMF + d) * 64 + lane_a) * 16);
            a[j][d] = (s < nsteps && i < M) ? v : v4i{0, 0, 0, 0};
        }
    }
    // weight chunk offsets in a tile, per k-step (a chunk past the last
    // k-block re-reads the last one: it meets zero activations)
    uint32_t boff[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int s = wave + j * KS;
        const int kb = 4 * (s < nsteps ? s : nsteps - 1) + g;
        boff[j] = static_cast<uint32_t>(kb < KB ? kb : KB - 1) * 256u + static_cast<uint32_t>(i) * 16u;
    }
    const int64_t tile_bytes = static_cast<int64_t>(KB) * 256;
    const uint8_t *P0 = J.P + static_cast<int64_t>(lb) * tile_bytes;
    const int64_t stride_bytes = static_cast<int64_t>(J.nwg) * tile_bytes;
    // Ring loads are unconditional (tiles past the workgroup's last re-read
    // that one, just fetched): every path has the same loads outstanding, so
    // the wait before tile t's products leaves the next D - 1 in flight.
    auto load_tile = [&](int t, uint4 (&b)[SPW]) {
        const uint8_t *pt = P0 + static_cast<int64_t>(t < ntiles ? t : ntiles - 1) * stride_bytes;
#pragma unroll
        for (int j = 0; j < SPW; ++j) b[j] = *reinterpret_cast<const uint4 *>(pt + boff[j]);
    };
    uint4 b[D][SPW];
#pragma unroll
    for (int d = 0; d < D; ++d) load_tile(d, b[d]);
    // with the first loads in flight: clear the tile sums (every wave of the
    // workgroup takes this barrier once before its first atomic)
    zero_sums();

    v4i sacc = {0, 0, 0, 0}; // sum_k q of the wave's k-steps (offset codes only)
    if constexpr (kOffsetCodes<LAYOUT>) {
#pragma unroll
        for (int j = 0; j < SPW; ++j)
            if (j < nj) act_sum_step<NMF>(a[j], sacc);
    }
    // Unrolled over the most tiles a workgroup takes (a compile-time
    // recursion, so no loop is left): a loop back-edge would make the
    // compiler wait for every load in flight at each trip (it moves ring
    // registers across the edge), draining the ring.
    unroll_while<0, GROUP_STAGE_TILES>([&](auto tc) -> bool {
        constexpr int t = decltype(tc)::value;
        if (t >= ntiles) return false;
        v4i acc[1] = {v4i{0, 0, 0, 0}};
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            if (j >= nj) break;
            const uint4 bj[1] = {b[t % D][j]};
            gemv_step<LAYOUT, 1, NMF>(bj, a[j], acc);
        }
        if constexpr (t + D < GROUP_STAGE_TILES) load_tile(t + D, b[t % D]);
        const v4i part = kOffsetCodes<LAYOUT> ? offset_fix<LAYOUT>(acc[0], sacc) : acc[0];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            __hip_atomic_fetch_add(&sums[t][rr][lane], part[rr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return true;
    });
}

template <int LAYOUT>
__global__ __launch_bounds__(1024) void k_group_gemv(const GroupGemvArgs args)
{
    // int32 sums of the workgroup's tiles: [tile][token sub-row rr][lane]
    // (lane (i, g) of tile t: token 4g + rr, weight row i)
    __shared__ int sums[GROUP_STAGE_TILES][4][64];

    // this workgroup's job (one scalar load of the index table, then one
    // batch for the job's fields) and its index among the job's workgroups
    const int jx = (args.jobidx[blockIdx.x >> 2] >> (8 * (blockIdx.x & 3))) & 0xff;
    const GroupJob J = args.job[jx]; // (a copy: all fields in one batch of scalar loads)
    const int lb = static_cast<int>(blockIdx.x) - J.wg0;
    const int M = J.M, N = J.N, nsteps = J.nsteps;
    const int KS = blockDim.x >> 6;
    const int wave = wave_id(), lane = lane_id();
    const int i = lane & 15, g = lane >> 4;
    const int NT = (N + 15) >> 4;
    const int ntiles = (NT - lb + J.nwg - 1) / J.nwg; // tiles lb, lb + nwg, ...
    const int spw = (nsteps + KS - 1) / KS;           // the job's k-steps per wave (uniform)
    const int nj = wave < nsteps ? (nsteps - 1 - wave) / KS + 1 : 0; // this wave's

    // gamma and beta of this lane's output tokens 4g .. 4g+3: loaded first,
    // used only after the product (so no wait on them delays the stream)
    // (a vector load: a scalar one would be waited for at the first barrier)
    const float gamma = __hip_atomic_load(J.gamma, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float bt[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int m = 4 * g + rr;
        bt[rr] = J.beta[m < M ? m : M - 1];
    }
    auto zero_sums = [&]() {
        for (int e = threadIdx.x; e < ntiles * 4 * 64; e += blockDim.x) (&sums[0][0][0])[e] = 0;
        lds_barrier();
    };
    if (nj > 0) {
        if (spw <= 1) group_job_tiles<LAYOUT, 1, group_depth(LAYOUT, 1)>(J, KS, wave, lane, nj, lb, ntiles, sums, zero_sums);
        else if (spw == 2) group_job_tiles<LAYOUT, 2, group_depth(LAYOUT, 2)>(J, KS, wave, lane, nj, lb, ntiles, sums, zero_sums);
        else if (LAYOUT == LAYOUT_I2 && spw == 3) group_job_tiles<LAYOUT, LAYOUT == LAYOUT_I2 ? 3 : 2, group_depth(LAYOUT, 3)>(J, KS, wave, lane, nj, lb, ntiles, sums, zero_sums);
        else zero_sums(); // (not reached: the plan keeps spw within the templates)
    } else {
        zero_sums();
    }
    lds_barrier();
    float sc[4]; // rescale factors of tokens 4g .. 4g+3
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sc[rr] = 4 * g + rr < M ? token_scale(gamma, bt[rr]) : 0.0f;
    // rescale and store tile t (weight rows 16 (lb + t nwg) + i)
    for (int t = wave; t < ntiles; t += KS) {
        const int64_t n = static_cast<int64_t>(lb + t * J.nwg) * 16 + i;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = 4 * g + rr;
            if (m < M && n < N) store_out(J.Y, args.y_dtype, J.ldy, m, n, sums[t][rr][lane], sc[rr]);
        }
    }
}

int group_max_nsteps(int layout)
{
    // k-steps per wave the registers hold next to the weight ring: 3 for i2,
    // 2 for b3 (5 activation operands per k-step and the digit decode) and b1
    // (8 operands per k-step)
    return GROUP_WAVES * (layout == LAYOUT_I2 ? 3 : 2);
}

GroupPlan group_plan(GroupGemvArgs &args, int layout)
{
    GroupPlan p{1, 1, 0};
    int max_steps = 1;
    double total = 0.0;
    for (int j = 0; j < args.njobs; ++j) {
        const GroupJob &J = args.job[j];
        max_steps = J.nsteps > max_steps ? J.nsteps : max_steps;
        total += static_cast<double>((J.N + 15) / 16) * J.KB;
    }
    p.waves = max_steps < GROUP_WAVES ? max_steps : GROUP_WAVES;
    const int spw = (max_steps + p.waves - 1) / p.waves;
    p.spw = spw <= 1 ? 1 : (spw <= 2 ? 2 : 3);
    (void)layout;
    // one workgroup per CU in all, dealt by weight bytes; at least one per
    // GROUP_STAGE_TILES tiles (the LDS staging of a workgroup's outputs) and
    // at most one per tile
    constexpr double kCUs = 256.0;
    int wg = 0;
    for (int j = 0; j < args.njobs; ++j) {
        GroupJob &J = args.job[j];
        const int NT = (J.N + 15) / 16;
        int n = static_cast<int>(kCUs * NT * J.KB / total + 0.5);
        const int min_n = (NT + GROUP_STAGE_TILES - 1) / GROUP_STAGE_TILES;
        n = n < min_n ? min_n : n;
        n = n > NT ? NT : n;
        n = n < 1 ? 1 : n;
        J.wg0 = wg;
        J.nwg = n;
        for (int b = wg; b < wg + n && b < GROUP_MAX_WGS; ++b) {
            if ((b & 3) == 0) args.jobidx[b >> 2] = 0;
            args.jobidx[b >> 2] |= static_cast<uint32_t>(j) << (8 * (b & 3));
        }
        wg += n;
    }
    p.wgs = wg <= GROUP_MAX_WGS ? wg : 0;
    return p;
}

template <int LAYOUT>
static void launch_group_layout(const GroupGemvArgs &args, const GroupPlan &plan, hipStream_t stream)
{
    hipLaunchKernelGGL((k_group_gemv<LAYOUT>), dim3(static_cast<unsigned>(plan.wgs)),
                       dim3(static_cast<unsigned>(plan.waves * 64)), 0, stream, args);
}

hipError_t launch_group_gemv(const GroupGemvArgs &args, const GroupPlan &plan, int layout, hipStream_t stream)
{
    if (plan.wgs < 1 || plan.spw > 3 || (layout != LAYOUT_I2 && plan.spw > 2)) return hipErrorInvalidValue;
    if (layout == LAYOUT_I2) launch_group_layout<LAYOUT_I2>(args, plan, stream);
    else if (layout == LAYOUT_B3) launch_group_layout<LAYOUT_B3>(args, plan, stream);
    else launch_group_layout<LAYOUT_B1>(args, plan, stream);
    return hipGetLastError();
}

void group_gemv_kernel_name(int layout, int spw, char *buf, size_t n)
{
    (void)spw;
    snprintf(buf, n, "bl::k_group_gemv<%d>", layout);
}

} // namespace bl
