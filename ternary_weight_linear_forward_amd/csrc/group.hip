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
#include "fq_core.h"
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

// Settle loaded registers: the compiler waits for their loads here (and only
// here), and later code sees the values of this empty statement, with no
// load pending behind them.  Without it, code that uses them after the
// weight ring has been issued may be given waits that also count ring loads.
__device__ __forceinline__ void settle(uint4 &x)
{
    asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}
__device__ __forceinline__ void settle(v4i &x) { asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])); }

__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
} // namespace

// Weight tiles in flight per wave for a job of SPW k-steps per wave: at most
// what the registers left next to the activation operands hold without
// spilling.  i2 with one k-step per wave keeps 6 of the 10 that would fit:
// with every tile of a workgroup asked for at once the 3B calls took 13.1 us
// (one token) against 12.5 us with 5 or 6 in flight, refilled as tiles finish.
constexpr int group_depth(int layout, int spw)
{
    return layout == LAYOUT_I2 ? (spw == 1 ? 6 : (spw == 2 ? 4 : 2))
           : layout == LAYOUT_B3 ? (spw == 1 ? 8 : (spw == 2 ? 4 : 2))
                                 : (spw == 1 ? 5 : 2);
}

// Raw buffer load of 16 bytes at byte voff of [base, base + nbytes): reads at
// or past nbytes return zeros without touching memory.  base and nbytes are
// wave-uniform.
__device__ __forceinline__ uint4 group_buffer_load(const void *base, int nbytes, uint32_t voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nbytes, 0x00020000);
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
#else
    (void)base, (void)nbytes, (void)voff;
    return make_uint4(0u, 0u, 0u, 0u);
#endif
}

// i2 k-step with the 2-bit codes c = T + 1 masked in place.  Word d of the
// lane's chunk holds weight 16d + 4s + j at bits 8j + 2s, so (w & 0x03030303)
// are the codes of weights 16d + j, (w & 0x0c0c0c0c) 4 x the codes of weights
// 16d + 4 + j, (w & 0x30303030) 16 x those of 16d + 8 + j and ((w >> 2) &
// 0x30303030) 16 x those of 16d + 12 + j: 5 instructions per word, with no
// conversion to signed bytes.  MFMA s multiplies the four words' field s with
// the activations of the same weights (operand at[s], dword d = activations
// 16d + 4s .. 16d + 4s + 3, a transpose of the natural operands) into an
// accumulator of its own scale: sum_k q c = acc1 + acc4 / 4 + acc16 / 16,
// every quotient exact, and sum_k q T = that - sum_k q.
struct I2ScaledAcc {
    v4i a1, a4, a16a, a16b;
};

__device__ __forceinline__ void i2_scaled_step(const uint4 &w, const v4i (&at)[4], I2ScaledAcc &acc)
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    v4i b0, b1, b2, b3;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        b0[d] = static_cast<int>(wd[d] & 0x03030303u);
        b1[d] = static_cast<int>(wd[d] & 0x0c0c0c0cu);
        b2[d] = static_cast<int>(wd[d] & 0x30303030u);
        b3[d] = static_cast<int>((wd[d] >> 2) & 0x30303030u);
    }
    acc.a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(at[0], b0, acc.a1, 0, 0, 0);
    acc.a4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(at[1], b1, acc.a4, 0, 0, 0);
    acc.a16a = __builtin_amdgcn_mfma_i32_16x16x64_i8(at[2], b2, acc.a16a, 0, 0, 0);
    acc.a16b = __builtin_amdgcn_mfma_i32_16x16x64_i8(at[3], b3, acc.a16b, 0, 0, 0);
}

// The same i2 k-step on the vector ALU for one token (the add/subtract form:
// no multiplier sees a weight other than 0, 1, 2 or 3 times a power of two).
// ab[d] holds the token's activations of the lane's k-block in the natural
// operand layout (dword s of operand d = activations 16d + 4s .. 16d + 4s + 3),
// the same in every lane of a row; field s of word d pairs with dword s of
// operand d, one v_dot4 each, into accumulators of three scales as above.
struct I2DotAcc {
    int p1, p4, p16;
};

__device__ __forceinline__ void i2_dot_step(const uint4 &w, const v4i (&ab)[4], I2DotAcc &acc)
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        acc.p1 = __builtin_amdgcn_sdot4(static_cast<int>(wd[d] & 0x03030303u), ab[d][0], acc.p1, false);
        acc.p4 = __builtin_amdgcn_sdot4(static_cast<int>(wd[d] & 0x0c0c0c0cu), ab[d][1], acc.p4, false);
        acc.p16 = __builtin_amdgcn_sdot4(static_cast<int>(wd[d] & 0x30303030u), ab[d][2], acc.p16, false);
        acc.p16 = __builtin_amdgcn_sdot4(static_cast<int>((wd[d] >> 2) & 0x30303030u), ab[d][3], acc.p16, false);
    }
}

// b3 k-step with the digit subtraction moved into the matrix cores.  The
// fixed-point byte u of five digits (c_0 most significant) gives the levels
// X_t = floor(u 3^t / 256) (t = 1..5; X_5 is the base-3 value itself) and
// digit t is X_(t+1) - 3 X_t (b3_word_digits).  Instead of forming the digits,
// MFMA t multiplies the activations of digit t with X_(t+1) into acc_p and,
// for t >= 1, with X_t into acc_m: sum_k q c = acc_p - 3 acc_m.  X_5 (up to
// 242) does not fit a signed byte, so it enters as X_5 - 128 (bit 7 flipped)
// and 128 times the sum of digit 4's activations is added back (b3_level_fix).
// Per 4-byte word: 17 instructions (the 16-bit products and one v_perm_b32
// per level, one xor) instead of 25, and 9 MFMAs per k-step instead of 5.
struct B3LevelAcc {
    v4i p, m;
};

__device__ __forceinline__ void b3_level_step(const uint4 &w, const v4i (&a)[5], B3LevelAcc &acc)
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    v4i X[6];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t even = wd[q] & 0x00ff00ffu;                         // bytes 0 and 2
        const uint32_t odd = __builtin_amdgcn_perm(0u, wd[q], 0x0c030c01u); // bytes 1 and 3
        uint32_t p3 = 1;
#pragma unroll
        for (int t = 1; t <= 5; ++t) {
            p3 *= 3;
            const uint32_t ze = pk_mul_u16(even, p3 * 0x00010001u), zo = pk_mul_u16(odd, p3 * 0x00010001u);
            const uint32_t x = __builtin_amdgcn_perm(zo, ze, 0x07030501u); // high byte of each lane, in order
            X[t][q] = static_cast<int>(t == 5 ? x ^ 0x80808080u : x);
        }
    }
#pragma unroll
    for (int t = 0; t < 5; ++t) {
        acc.p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], X[t + 1], acc.p, 0, 0, 0);
        if (t >= 1) acc.m = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], X[t], acc.m, 0, 0, 0);
    }
}

// 128 sum_k q over digit 4's activations minus sum_k q over all (the offset
// codes c = T + 1), for the wave's k-steps, in the MFMA output layout.
template <int SPW>
__device__ __forceinline__ v4i b3_level_fix(const v4i (&a)[SPW][5], int nj)
{
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    v4i s4 = {0, 0, 0, 0}, all = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < SPW; ++j)
        if (j < nj) {
            s4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j][4], ones, s4, 0, 0, 0);
            act_sum_step<5>(a[j], all);
        }
    return 128 * s4 - all;
}

// LDS of the workgroup: the tile sums, and for the quantiser inside (1 to 4
// tokens of fp32 / bf16 input) the per-wave rounding areas and maxima.
struct GroupLds {
    int (*sums)[4][64]; // [GROUP_STAGE_TILES][rr][lane]
    v4i *qbuf;          // [waves][SPW * units per k-step] (quantiser inside)
    float (*wmax)[4];   // [waves][4] (quantiser inside)
};

// One job's share of a workgroup: this wave's k-steps (nj of them, at most
// SPW; 0 for a wave without one) of the row tiles lb, lb + nwg, ... (ntiles
// of them), D tiles of weight loads in flight; each tile's partial sums go
// into sums[t] by LDS atomics.  XDT: DT_I8 reads the activations quantised
// by k_group_quant_tiled (tiled layout, beta given); DT_F32 / DT_BF16 reads
// the job's 1 to 4 tokens of X and quantises them inside (fq_quantise: beta
// across the waves, exactly as the quantiser) and returns beta of token
// lane % 4 in every lane.  Every wave of the workgroup calls this once: it
// holds one barrier.
template <int LAYOUT, int SPW, int D, int XDT, bool ADDSUB>
__device__ __forceinline__ float group_job_tiles(const GroupJob &J, int KS, int wave, int lane, int nj, int lb,
                                                 int ntiles, const GroupLds &L)
{
    static_assert(!ADDSUB || LAYOUT == LAYOUT_I2, "the vector-ALU product is written for i2");
    using S = StepShape<LAYOUT>;
    constexpr int NMF = S::NMF;
    const int M = J.M, KB = J.KB, nsteps = J.nsteps;
    const int i = lane & 15, g = lane >> 4;

    // weight chunk offsets in a tile, per k-step (a chunk past the last
    // k-block re-reads the last one: it meets zero activations)
    uint32_t boff[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int s = wave + j * KS;
        const int kb = 4 * (s < nsteps ? s : nsteps - 1) + g;
        boff[j] = static_cast<uint32_t>(kb < KB ? kb : KB - 1) * 256u + static_cast<uint32_t>(i) * 16u;
    }
    const uint32_t tile_bytes = static_cast<uint32_t>(KB) * 256u;
    const uint32_t stride_bytes = static_cast<uint32_t>(J.nwg) * tile_bytes;
    const int job_bytes = static_cast<int>(static_cast<int64_t>((J.N + 15) >> 4) * tile_bytes);
    // Ring loads are unconditional, so every path has the same loads
    // outstanding and the wait before tile t's products leaves the next D - 1
    // in flight.  Tiles past the workgroup's last and k-steps past the wave's
    // last ask for bytes past the job's end: the buffer returns zeros without
    // touching memory.
    auto load_tile = [&](int t, uint4 (&b)[SPW]) {
        const uint32_t toff = t < ntiles ? static_cast<uint32_t>(lb) * tile_bytes + static_cast<uint32_t>(t) * stride_bytes
                                         : 0x80000000u;
#pragma unroll
        for (int j = 0; j < SPW; ++j) b[j] = group_buffer_load(J.P, job_bytes, j < nj ? toff + boff[j] : 0x80000000u);
    };
    uint4 b[D][SPW];
    v4i a[SPW][NMF];
    float beta_lane = 0.0f;
    auto zero_sums = [&]() {
        for (int e = threadIdx.x; e < ntiles * 4 * 64; e += blockDim.x) (&L.sums[0][0][0])[e] = 0;
    };
    if constexpr (XDT == DT_I8) {
        // activation operands of this wave's k-steps, once.  Lanes of tokens
        // past M read token 0's bytes (the same cache lines) and drop them.
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
        // Every wave of the workgroup asks for its activations before any wave
        // asks for weights: the loads of one CU are served in order, and
        // activations asked for after another wave's weight ring would wait
        // behind it.  The barrier also orders the clearing of the sums before
        // the first atomic.  One weight tile goes out before the wait for the
        // activations, the rest of the ring after it (measured: faster than
        // the whole ring on either side of the wait).
        zero_sums();
        lds_barrier();
        load_tile(0, b[0]);
#pragma unroll
        for (int j = 0; j < SPW; ++j)
#pragma unroll
            for (int d = 0; d < NMF; ++d) settle(a[j][d]);
#pragma unroll
        for (int d = 1; d < D; ++d) load_tile(d, b[d]);
    } else {
        // The wave's own activations, asked for by every wave of the
        // workgroup before any wave asks for weights (as above), then one
        // weight tile, the wait for the activations, and the quantiser; the
        // rest of the ring goes out right after the quantiser's barrier, and
        // the rounding runs while it is in flight.  (Measured at the 3B
        // layers, one token: the whole ring after that barrier 12.5 us per
        // call, one tile before it 11.9 us, two 12.5 us, the whole ring
        // before the wait 14.0 us.)  The first barrier also orders the
        // clearing of the sums before the first atomic.
        using FU = FqUnits<LAYOUT, XDT, SPW>;
        const FU U{lane, wave, KS, M, nj * M * FU::CH, J.K, static_cast<int>(J.ldx)};
        constexpr int ES = XDT == DT_F32 ? 4 : 2;
        const int xbytes = static_cast<int>((((static_cast<int64_t>(M) - 1) * J.ldx + J.K) * ES + 15) & ~int64_t(15));
        uint4 xv[FU::NUW][FU::VL];
        fq_load(U, J.X, xbytes, xv);
        zero_sums();
        lds_barrier();
        load_tile(0, b[0]);
#pragma unroll
        for (int n = 0; n < FU::NUW; ++n)
#pragma unroll
            for (int v = 0; v < FU::VL; ++v) settle(xv[n][v]);
        beta_lane = fq_quantise<FU, SPW>(U, xv, L.qbuf + wave * SPW * FU::UNITS, L.wmax, a, [&]() {
#pragma unroll
            for (int d = 1; d < D; ++d) load_tile(d, b[d]);
        });
    }
    if constexpr (ADDSUB) {
        // one token (M = 1): every lane of row g takes lane (0, g)'s operands,
        // token 0's activations of k-block g (DPP row_newbcast:0, lane 0 of
        // each 16-lane row to the whole row)
#pragma unroll
        for (int j = 0; j < SPW; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int w = 0; w < 4; ++w) a[j][d][w] = __builtin_amdgcn_update_dpp(0, a[j][d][w], 0x150, 0xf, 0xf, false);
    } else if constexpr (LAYOUT == LAYOUT_I2) {
        // i2: the operands transposed for the masked codes (i2_scaled_step)
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            v4i t[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int d = 0; d < 4; ++d) t[q][d] = a[j][d][q];
#pragma unroll
            for (int q = 0; q < 4; ++q) a[j][q] = t[q];
        }
    }
    if (nj == 0) return beta_lane;

    v4i sacc = {0, 0, 0, 0}; // sum_k q of the wave's k-steps (offset codes); b3: b3_level_fix
    int qsum = 0;             // add/sub: sum_k q of the lane's k-blocks
    if constexpr (ADDSUB) {
#pragma unroll
        for (int j = 0; j < SPW; ++j)
            if (j < nj)
#pragma unroll
                for (int d = 0; d < 4; ++d)
#pragma unroll
                    for (int w = 0; w < 4; ++w) qsum = __builtin_amdgcn_sdot4(a[j][d][w], 0x01010101, qsum, false);
    } else if constexpr (LAYOUT == LAYOUT_B3) {
        sacc = b3_level_fix<SPW>(a, nj);
    } else {
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
        v4i part;
        if constexpr (ADDSUB) {
            I2DotAcc acc{0, 0, 0};
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                if (j >= nj) break;
                i2_dot_step(b[t % D][j], a[j], acc);
            }
            // row i, k-block lane g: summed over the waves in sums[t][0][lane]
            // (the four k-block lanes of a row are added at the store)
            const int p = acc.p1 + (acc.p4 >> 2) + (acc.p16 >> 4) - qsum;
            if constexpr (t + D < GROUP_STAGE_TILES) load_tile(t + D, b[t % D]);
            __hip_atomic_fetch_add(&L.sums[t][0][lane], p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return true;
        } else if constexpr (LAYOUT == LAYOUT_I2) {
            I2ScaledAcc acc{{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                if (j >= nj) break;
                i2_scaled_step(b[t % D][j], a[j], acc);
            }
            part = acc.a1 + (acc.a4 >> 2) + ((acc.a16a + acc.a16b) >> 4) - sacc;
        } else if constexpr (LAYOUT == LAYOUT_B3) {
            B3LevelAcc acc{{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                if (j >= nj) break;
                b3_level_step(b[t % D][j], a[j], acc);
            }
            part = acc.p - 3 * acc.m + sacc;
        } else {
            v4i acc[1] = {v4i{0, 0, 0, 0}};
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                if (j >= nj) break;
                const uint4 bj[1] = {b[t % D][j]};
                gemv_step<LAYOUT, 1, NMF>(bj, a[j], acc);
            }
            part = offset_fix<LAYOUT>(acc[0], sacc);
        }
        if constexpr (t + D < GROUP_STAGE_TILES) load_tile(t + D, b[t % D]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            __hip_atomic_fetch_add(&L.sums[t][rr][lane], part[rr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return true;
    });
    return beta_lane;
}

// k-steps per wave the fused-quantiser kernel takes for a layout (its
// rounding area and staged activations share the registers with the ring)
constexpr int group_fq_max_spw(int layout) { return layout == LAYOUT_I2 ? 3 : 2; }

// The grouped launch's workgroup: its job, the products (matrix cores, or the
// vector ALU for ADDSUB), the rescale and the stores.  L.sums: the int32 sums
// of the workgroup's tiles, [tile][token sub-row rr][lane] (lane (i, g) of
// tile t: token 4g + rr, weight row i).
template <int LAYOUT, int XDT, bool ADDSUB>
__device__ __forceinline__ void group_gemv_body(const GroupGemvArgs &args, const GroupLds &L)
{
    int (*const sums)[4][64] = L.sums;

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

    // gamma and (tiled input) beta of this lane's output tokens 4g .. 4g+3:
    // loaded first, used only after the product (so no wait on them delays
    // the stream; gamma by a vector load: a scalar one would be waited for at
    // the first barrier)
    const float gamma = __hip_atomic_load(J.gamma, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float bt[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (XDT == DT_I8) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = 4 * g + rr;
            bt[rr] = J.beta[m < M ? m : M - 1];
        }
    }
    float beta_lane = 0.0f;
    if (XDT != DT_I8 || nj > 0) {
        if (spw <= 1) beta_lane = group_job_tiles<LAYOUT, 1, group_depth(LAYOUT, 1), XDT, ADDSUB>(J, KS, wave, lane, nj, lb, ntiles, L);
        else if (spw == 2) beta_lane = group_job_tiles<LAYOUT, 2, group_depth(LAYOUT, 2), XDT, ADDSUB>(J, KS, wave, lane, nj, lb, ntiles, L);
        else if (LAYOUT == LAYOUT_I2 && spw == 3) beta_lane = group_job_tiles<LAYOUT, LAYOUT == LAYOUT_I2 ? 3 : 2, group_depth(LAYOUT, 3), XDT, ADDSUB>(J, KS, wave, lane, nj, lb, ntiles, L);
        else lds_barrier(); // (not reached: the plan keeps spw within the templates)
    } else {
        for (int e = threadIdx.x; e < ntiles * 4 * 64; e += blockDim.x) (&sums[0][0][0])[e] = 0;
        lds_barrier();
    }
    if constexpr (XDT != DT_I8) {
        // beta of tokens 4g + rr < 4 (every lane active for the shuffles)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) bt[rr] = __shfl(beta_lane, rr);
    }
    lds_barrier();
    float sc[4]; // rescale factors of tokens 4g .. 4g+3
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sc[rr] = 4 * g + rr < M ? token_scale(gamma, bt[rr]) : 0.0f;
    // rescale and store tile t (weight rows 16 (lb + t nwg) + i)
    for (int t = wave; t < ntiles; t += KS) {
        const int64_t n = static_cast<int64_t>(lb + t * J.nwg) * 16 + i;
        if constexpr (ADDSUB) { // one token: row i's four k-block lanes
            if (g == 0 && n < N)
                store_out(J.Y, args.y_dtype, J.ldy, 0, n, sums[t][0][i] + sums[t][0][i + 16] + sums[t][0][i + 32] + sums[t][0][i + 48], sc[0]);
            continue;
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = 4 * g + rr;
            if (m < M && n < N) store_out(J.Y, args.y_dtype, J.ldy, m, n, sums[t][rr][lane], sc[rr]);
        }
    }
}

template <int LAYOUT, int XDT>
__global__ __launch_bounds__(1024) void k_group_gemv(const GroupGemvArgs args)
{
    __shared__ int sums[GROUP_STAGE_TILES][4][64];
    __shared__ float wmax[16][4];
    extern __shared__ v4i qbuf_dyn[]; // quantiser inside: [waves][spw * units]
    group_gemv_body<LAYOUT, XDT, false>(args, GroupLds{sums, qbuf_dyn, wmax});
}

// The same launch with the i2 products on the vector ALU (i2_dot_step), for
// jobs of one token each.
template <int XDT>
__global__ __launch_bounds__(1024) void k_group_gemv_addsub(const GroupGemvArgs args)
{
    __shared__ int sums[GROUP_STAGE_TILES][4][64];
    __shared__ float wmax[16][4];
    extern __shared__ v4i qbuf_dyn[];
    group_gemv_body<LAYOUT_I2, XDT, true>(args, GroupLds{sums, qbuf_dyn, wmax});
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
    {
        // the fewest waves that leave every job's k-steps per wave as they are
        // with GROUP_WAVES (3B layers: 13, not 16 -- the 13-step jobs' other
        // three waves would idle): fewer waves to dispatch and to meet at the
        // barriers, 0.1-0.25 us per call
        int ks = 1;
        for (int j = 0; j < args.njobs; ++j) {
            const int ns = args.job[j].nsteps;
            const int spw16 = (ns + GROUP_WAVES - 1) / GROUP_WAVES;
            const int need = (ns + spw16 - 1) / spw16;
            ks = need > ks ? need : ks;
        }
        p.waves = ks < p.waves ? ks : p.waves;
    }
    const int spw = (max_steps + p.waves - 1) / p.waves;
    p.spw = spw <= 1 ? 1 : (spw <= 2 ? 2 : 3);
    (void)layout;
    (void)total;
    // One workgroup per CU in all (256), at least one per GROUP_STAGE_TILES
    // tiles of a job (the LDS staging of a workgroup's outputs) and at most
    // one per tile.  The launch lasts as long as its most loaded workgroup,
    // so the workgroups are dealt one at a time to the job whose workgroups
    // hold the most weight bytes each (ceil(tiles / n) tiles of KB k-blocks):
    // that minimises the largest share.  (Shares proportional to the bytes
    // leave whole tiles over in some workgroups: at the 3B layers the
    // largest share was 1.14 times the mean, at the 70B q/k/v/o/gate/up 1.19
    // times (k and v: 3 workgroups of 22 tiles); dealt this way 1.06 and
    // 1.03 times.)
    constexpr int kCUs = 256;
    int nwg[GROUP_MAX_JOBS];
    int sum = 0;
    for (int j = 0; j < args.njobs; ++j) {
        const int NT = (args.job[j].N + 15) / 16;
        nwg[j] = (NT + GROUP_STAGE_TILES - 1) / GROUP_STAGE_TILES;
        sum += nwg[j];
    }
    for (; sum < kCUs; ++sum) {
        int best = -1;
        int64_t best_bytes = 0;
        for (int j = 0; j < args.njobs; ++j) {
            const int NT = (args.job[j].N + 15) / 16;
            if (nwg[j] >= NT) continue;
            const int64_t b = static_cast<int64_t>((NT + nwg[j] - 1) / nwg[j]) * args.job[j].KB;
            if (b > best_bytes) {
                best_bytes = b;
                best = j;
            }
        }
        if (best < 0) break;
        ++nwg[best];
    }
    int wg = 0;
    for (int j = 0; j < args.njobs; ++j) {
        GroupJob &J = args.job[j];
        const int n = nwg[j];
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

template <int LAYOUT, int XDT>
static void launch_group_x(const GroupGemvArgs &args, const GroupPlan &plan, bool addsub, hipStream_t stream)
{
    auto *f = addsub && LAYOUT == LAYOUT_I2 ? &k_group_gemv_addsub<XDT> : &k_group_gemv<LAYOUT, XDT>;
    // the rounding areas of the quantiser inside: waves x k-steps x 4 tokens
    // x the k-step's 16-value chunks, 16 bytes each
    const size_t lds = XDT == DT_I8 ? 0
                                    : static_cast<size_t>(plan.waves) * plan.spw * 4 * (4 * StepShape<LAYOUT>::KBLK / 16) * 16;
    if (lds > 0)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  static_cast<int>(lds));
    hipLaunchKernelGGL(f, dim3(static_cast<unsigned>(plan.wgs)), dim3(static_cast<unsigned>(plan.waves * 64)), lds,
                       stream, args);
}

template <int LAYOUT>
static void launch_group_layout(const GroupGemvArgs &args, const GroupPlan &plan, int x_dtype, bool addsub,
                                hipStream_t stream)
{
    if (x_dtype == DT_BF16) launch_group_x<LAYOUT, DT_BF16>(args, plan, addsub, stream);
    else if (x_dtype == DT_F32) launch_group_x<LAYOUT, DT_F32>(args, plan, addsub, stream);
    else launch_group_x<LAYOUT, DT_I8>(args, plan, addsub, stream);
}

bool group_addsub_ok(const GroupGemvArgs &args, int layout)
{
    if (layout != LAYOUT_I2) return false;
    for (int j = 0; j < args.njobs; ++j)
        if (args.job[j].M != 1) return false;
    return true;
}

hipError_t launch_group_gemv(const GroupGemvArgs &args, const GroupPlan &plan, int layout, int x_dtype,
                             hipStream_t stream, bool addsub)
{
    if (plan.wgs < 1 || plan.spw > 3 || (layout != LAYOUT_I2 && plan.spw > 2)) return hipErrorInvalidValue;
    if (addsub && !group_addsub_ok(args, layout)) return hipErrorInvalidValue;
    if (layout == LAYOUT_I2) launch_group_layout<LAYOUT_I2>(args, plan, x_dtype, addsub, stream);
    else if (layout == LAYOUT_B3) launch_group_layout<LAYOUT_B3>(args, plan, x_dtype, false, stream);
    else launch_group_layout<LAYOUT_B1>(args, plan, x_dtype, false, stream);
    return hipGetLastError();
}

void group_gemv_kernel_name(int layout, int x_dtype, bool addsub, char *buf, size_t n)
{
    if (addsub) snprintf(buf, n, "bl::k_group_gemv_addsub<%d>", x_dtype);
    else snprintf(buf, n, "bl::k_group_gemv<%d, %d>", layout, x_dtype);
}

} // namespace bl
