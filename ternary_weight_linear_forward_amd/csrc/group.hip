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
// their weight bytes (plan below).  A workgroup serves one job: it owns a
// contiguous range of the job's 16-row tiles, and its waves split the job's
// k-steps (wave w takes steps w, w + KS, ...).  Each wave loads the int8
// activation operands of its k-steps once (the tiled layout, token group 0)
// and keeps them in registers, then streams its chunk of every tile through a
// ring of D tiles of weight loads in flight.  Per tile the KS partial 16 x 16
// results meet in LDS (double-buffered, one barrier per tile); one wave adds
// them and parks the tile in LDS, and the tiles are rescaled and stored at the
// end, so no store interleaves with the ring loads.
#include <cstdio>

#include "common.h"
#include "gemv_core.h"
#include "launch.h"

namespace bl {

namespace {
constexpr int GROUP_WAVES = 16; // most waves per workgroup

// s_waitcnt immediate: every LDS access of this wave done (lgkmcnt 0), vector
// memory and export counters left alone (gfx9 encoding).
constexpr int kLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
} // namespace

template <int LAYOUT, int SPW, int D>
__global__ __launch_bounds__(1024) void k_group_gemv(const GroupGemvArgs args)
{
    using S = StepShape<LAYOUT>;
    constexpr int NMF = S::NMF;
    __shared__ v4i red[2][GROUP_WAVES][64];
    __shared__ v4i stage[GROUP_STAGE_TILES][64];

    // this workgroup's job (wave-uniform scan of the kernel arguments)
    int jx = 0;
    for (int t = 1; t < args.njobs; ++t) jx = static_cast<int>(blockIdx.x) >= args.job[t].wg0 ? t : jx;
    const GroupJob &J = args.job[jx];
    const int M = J.M, N = J.N, KB = J.KB, nsteps = J.nsteps;
    const int KS = blockDim.x >> 6;
    const int wave = wave_id(), lane = lane_id();
    const int i = lane & 15, g = lane >> 4;
    const int NT = (N + 15) >> 4;
    const int lb = static_cast<int>(blockIdx.x) - J.wg0;
    const int t_begin = static_cast<int>(static_cast<int64_t>(lb) * NT / J.nwg);
    const int ntiles = static_cast<int>(static_cast<int64_t>(lb + 1) * NT / J.nwg) - t_begin;
    int nj = 0; // this wave's k-steps in this job
#pragma unroll
    for (int j = 0; j < SPW; ++j) nj += wave + j * KS < nsteps ? 1 : 0;

    // rescale factors of this lane's output tokens 4g .. 4g+3
    float sc[4];
    {
        const float gamma = *J.gamma;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = 4 * g + rr;
            const float v = token_scale(gamma, J.beta[m < M ? m : M - 1]);
            sc[rr] = m < M ? v : 0.0f;
        }
    }

    if (nj > 0) {
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
        const uint8_t *P0 = J.P + static_cast<int64_t>(t_begin) * KB * 256;
        const int64_t tile_bytes = static_cast<int64_t>(KB) * 256;
        // Ring loads are unconditional (tiles past the range re-read the last
        // one, just fetched): every path has the same loads outstanding, so
        // the wait before tile t's products leaves the next D - 1 in flight.
        auto load_tile = [&](int t, uint4 (&b)[SPW]) {
            const uint8_t *pt = P0 + static_cast<int64_t>(t < ntiles ? t : ntiles - 1) * tile_bytes;
#pragma unroll
            for (int j = 0; j < SPW; ++j) b[j] = *reinterpret_cast<const uint4 *>(pt + boff[j]);
        };
        uint4 b[D][SPW];
#pragma unroll
        for (int d = 0; d < D; ++d) load_tile(d, b[d]);

        v4i sacc = {0, 0, 0, 0}; // sum_k q of the wave's k-steps (offset codes only)
        if constexpr (kOffsetCodes<LAYOUT>) {
#pragma unroll
            for (int j = 0; j < SPW; ++j)
                if (j < nj) act_sum_step<NMF>(a[j], sacc);
        }
        for (int t0 = 0; t0 < ntiles; t0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int t = t0 + d;
                if (t >= ntiles) break;
                v4i acc[1] = {v4i{0, 0, 0, 0}};
#pragma unroll
                for (int j = 0; j < SPW; ++j) {
                    if (j >= nj) break;
                    const uint4 bj[1] = {b[d][j]};
                    gemv_step<LAYOUT, 1, NMF>(bj, a[j], acc);
                }
                load_tile(t + D, b[d]);
                red[t & 1][wave][lane] = kOffsetCodes<LAYOUT> ? offset_fix<LAYOUT>(acc[0], sacc) : acc[0];
                lds_barrier();
                if (wave == t % KS) {
                    v4i tot = red[t & 1][0][lane];
                    for (int w = 1; w < KS; ++w) tot += red[t & 1][w][lane];
                    stage[t][lane] = tot;
                }
            }
        }
    } else {
        // no k-step of this job for this wave: it only takes its share of
        // the per-tile barriers and reductions
        for (int t = 0; t < ntiles; ++t) {
            red[t & 1][wave][lane] = v4i{0, 0, 0, 0};
            lds_barrier();
            if (wave == t % KS) {
                v4i tot = red[t & 1][0][lane];
                for (int w = 1; w < KS; ++w) tot += red[t & 1][w][lane];
                stage[t][lane] = tot;
            }
        }
    }
    lds_barrier();
    // rescale and store: lane (i, g) of tile t holds tokens 4g .. 4g+3 of
    // weight row 16 (t_begin + t) + i
    for (int t = wave; t < ntiles; t += KS) {
        const v4i tot = stage[t][lane];
        const int64_t n = static_cast<int64_t>(t_begin + t) * 16 + i;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = 4 * g + rr;
            if (m < M && n < N) store_out(J.Y, args.y_dtype, J.ldy, m, n, tot[rr], sc[rr]);
        }
    }
}

int group_max_nsteps(int layout)
{
    // k-steps per wave the registers hold next to the weight ring: 3 (i2,
    // b3), 2 (b1, whose k-step has 8 activation operands)
    return GROUP_WAVES * (layout == LAYOUT_B1 ? 2 : 3);
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
        wg += n;
    }
    p.wgs = wg;
    return p;
}

// Weight tiles in flight per wave: as many as the registers left next to the
// activation operands hold without spilling.
constexpr int group_depth(int layout, int spw)
{
    return layout == LAYOUT_I2 ? (spw == 1 ? 8 : (spw == 2 ? 4 : 3))
           : layout == LAYOUT_B3 ? (spw == 1 ? 8 : (spw == 2 ? 4 : 2))
                                 : (spw == 1 ? 6 : 3);
}

template <int LAYOUT, int SPW>
static void launch_group_spw(const GroupGemvArgs &args, const GroupPlan &plan, hipStream_t stream)
{
    constexpr int D = group_depth(LAYOUT, SPW);
    hipLaunchKernelGGL((k_group_gemv<LAYOUT, SPW, D>), dim3(static_cast<unsigned>(plan.wgs)),
                       dim3(static_cast<unsigned>(plan.waves * 64)), 0, stream, args);
}

template <int LAYOUT>
static void launch_group_layout(const GroupGemvArgs &args, const GroupPlan &plan, hipStream_t stream)
{
    if (plan.spw == 1) launch_group_spw<LAYOUT, 1>(args, plan, stream);
    else if (plan.spw == 2) launch_group_spw<LAYOUT, 2>(args, plan, stream);
    else if constexpr (LAYOUT != LAYOUT_B1) launch_group_spw<LAYOUT, 3>(args, plan, stream);
}

hipError_t launch_group_gemv(const GroupGemvArgs &args, const GroupPlan &plan, int layout, hipStream_t stream)
{
    if (plan.spw > 3 || (layout == LAYOUT_B1 && plan.spw > 2)) return hipErrorInvalidValue;
    if (layout == LAYOUT_I2) launch_group_layout<LAYOUT_I2>(args, plan, stream);
    else if (layout == LAYOUT_B3) launch_group_layout<LAYOUT_B3>(args, plan, stream);
    else launch_group_layout<LAYOUT_B1>(args, plan, stream);
    return hipGetLastError();
}

void group_gemv_kernel_name(int layout, int spw, char *buf, size_t n)
{
    const int d = group_depth(layout, spw);
    snprintf(buf, n, "bl::k_group_gemv<%d, %d, %d>", layout, spw, d);
}

} // namespace bl
