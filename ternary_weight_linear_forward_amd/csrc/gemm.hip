// gemm.hip -- the prefill product for many tokens on the int8 matrix cores.
//
// At large M the BitLinear product (LIT-380 record, Key takeaways, bullet 4:
// integer additions of activations selected by ternary weights) is a dense
// contraction whose arithmetic, not HBM, is the bound: every packed weight is
// used by hundreds of tokens.  So it runs as v_mfma_i32_32x32x32_i8 on int8
// activation tiles and signed-byte weight operands unpacked from the 2-bit
// codes in registers.  The epilogue applies y = float(acc) * (gamma*beta_m)/127.
//
// Workgroup tile: BM tokens x BN weight rows, 4 waves in a 2 x 2 grid, each
// (BM/2) x (BN/2) = MI x NI MFMA tiles of 32 x 32.  A stage covers 128 k (two
// 64-weight k-blocks).  Both operands of a stage go from global memory
// straight to LDS (global_load_lds_dwordx4: no registers, no LDS write
// instructions), into a ring of NST stage buffers; the loads of stage s+NST-1
// are issued while stage s is multiplied, so NST-1 stages of memory latency
// are hidden.
//  * Activations: BM rows of 128 bytes per stage.  The 16-byte unit g of row r
//    sits at slot g ^ swz(r), so the 32 rows read by one MFMA operand load
//    spread over all LDS banks.
//  * Weights: the packed 256-byte chunks (16 rows x 64 weights) of the stage,
//    copied as they are (BN/16 tiles x 2 k-blocks = BN * 32 bytes).  Each lane
//    reads the one 32-bit word holding its 16 weights of an operand and
//    unpacks it with four v_perm_b32.
//
// Base-3 weights (k_gemm_mfma_b3) are decoded in the same place, so the GEMM
// reads the 20 % smaller b3 bytes and nothing is rewritten first.  A stage
// covers two 80-weight k-blocks (160 k) and lane half kh (lanes 32 kh ..
// 32 kh + 31) owns block kh of it: the lane reads its weight row's 16-byte
// chunk row with one 128-bit LDS read, and digit t of those 16 bytes is the
// 16 consecutive weights of MFMA k-step t (t = 0..4), in natural k order.  So
// the activations stay row-major: 160 bytes per row per stage, copied as
// consecutive 16-byte units (row stride 160 bytes spreads a 32-row operand
// read over the banks without a swizzle), and lane (token, kh) takes unit
// 5 kh + t of its row at k-step t.  Digits come from the fixed-point byte
// (H_t = floor(u 3^t / 256), digit t = H_(t+1) - 3 H_t) and become signed
// bytes with one v_perm_b32 each.
//
// Binary weights (k_gemm_mfma_b1) take the i2 activation staging (128 k per
// stage) with one 128-weight k-block of 16 bytes per row: the lane reads its
// row's 16 bytes at once, word kk holds the 32 weights of MFMA k-step kk, and
// half kh of them (bits 4 kh + s of each byte, s = 0..3) become signed bytes
// with one v_perm_b32 per dword.  Pad weights are -1, not 0, so the last
// stage masks the operand bytes at or past K.
// Only s_barrier (no memory fence) separates the stages; the explicit vmcnt
// wait before it covers this wave's own copies of the stage, and the barrier
// then covers every wave's.
#include <cstdio>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace bl {

namespace {
constexpr int KSTEP = 128;              // k per stage half: two 64-weight k-blocks
constexpr int B3_ROW = 160;             // b3: k per stage, two 80-weight k-blocks
constexpr int LDS_RING_BYTES = 150 * 1024; // LDS given to the stage ring (of 160 KB)
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
// Word 3 of a raw buffer resource on gfx9 parts: 32-bit data format, no swizzle.
constexpr int BUF_RSRC_WORD3 = 0x00020000;

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and lgkmcnt at max).
constexpr int vmcnt_only(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }
// ... and also for every LDS read of this wave (lgkmcnt 0)
constexpr int vmcnt_lgkm0(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }
} // namespace

__device__ __forceinline__ int a_swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ v4i gemm_i2_word_signed(uint32_t w)
{
    v4i r;
    r[0] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, w & 0x03030303u));
    r[1] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, (w >> 2) & 0x03030303u));
    r[2] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, (w >> 4) & 0x03030303u));
    r[3] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, (w >> 6) & 0x03030303u));
    return r;
}

// One wave-wide copy into LDS through a raw buffer resource over [base,
// base + nbytes): lane i's SZ bytes at byte voff land at dst + SZ * i; reads
// at or past nbytes return zeros without touching memory.  (The buffer
// builtins exist only in the device pass.)
template <int SZ>
__device__ __forceinline__ void buffer_copy_to_lds(const void *base, int nbytes, lds_void_t *dst, int voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    // base and nbytes are wave-uniform; say so, so that the resource stays in
    // scalar registers
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t bu = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32))) << 32) |
                        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(bu), 0, __builtin_amdgcn_readfirstlane(nbytes), BUF_RSRC_WORD3);
    if constexpr (SZ == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, 0, 0, 0);
#endif
}

__device__ __forceinline__ void stage_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int LAYOUT, int BM, int BN, int WM, int WN, int S>
__device__ __forceinline__ void gemm_body(const uint8_t *__restrict__ P, int64_t KB, int64_t NT,
                                          const float *__restrict__ gamma_p, const int8_t *__restrict__ Xq,
                                          int64_t ldq, const float *__restrict__ beta, int64_t M, int64_t N,
                                          int64_t K, void *__restrict__ Y, int y_dtype, int64_t ldy, int n_major)
{
    constexpr bool B3 = LAYOUT == LAYOUT_B3, B1 = LAYOUT == LAYOUT_B1;
    static_assert(LAYOUT == LAYOUT_I2 || ((B3 || B1) && S == 1), "i2 with S halves of 128 k, b3 with 160 k, b1 with 128 k");
    constexpr int NW = WM * WN;                // waves
    constexpr int MI = BM / WM / 32;           // 32-token MFMA tiles per wave
    constexpr int NI = BN / WN / 32;           // 32-row MFMA tiles per wave
    constexpr int ROW = B3 ? B3_ROW : KSTEP;   // activation bytes per row per stage half
    constexpr int KS_ = ROW * S;               // k per stage
    constexpr int KK = B3 ? 5 : 4 * S;         // 32-k MFMA steps per stage
    constexpr int NWORD = B3 ? 4 : KK;         // packed words per weight operand row per stage
    constexpr int A_BYTES = BM * KS_;          // activation bytes per stage: [S][BM][ROW]
    constexpr int KBS = B1 ? 1 : 2 * S;        // k-blocks per stage
    constexpr int B_BYTES = BN * 16 * KBS;     // packed weight bytes per stage
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_ROWS_W = BM / NW;          // i2: activation rows copied by one wave
    constexpr int A_RB = A_ROWS_W / 8;         // i2: 1 KB copies (8 rows of 128 B) per wave per half
    constexpr int A_COPIES = A_BYTES / 1024;   // b3: 1 KB copies per stage, dealt round-robin
    constexpr int A_INST = B3 ? (A_COPIES + NW - 1) / NW : A_RB * S; // copies per wave per stage
    // weight copies: 16 bytes per lane when every wave gets whole 1 KB copies, else 4
    constexpr int B_CP = (B_BYTES % (1024 * NW) == 0) ? 16 : 4;
    constexpr int B_INST = B_BYTES / (64 * B_CP) / NW;
    constexpr int NST = LDS_RING_BYTES / STAGE < 8 ? LDS_RING_BYTES / STAGE : 8; // ring depth
    constexpr int LOADS = A_INST + B_INST;     // copies per wave per stage
    static_assert(MI >= 1 && NI >= 1 && A_INST >= 1 && B_INST >= 1 && NST >= 3, "tile shape");
    static_assert(!B3 || A_COPIES * 1024 == A_BYTES, "b3 activation stage in whole 1 KB copies");
    static_assert(B_INST * NW * 64 * B_CP == B_BYTES && (NST - 1) * LOADS < 64, "copy plan");
    __shared__ __attribute__((aligned(16))) int8_t lds[NST * STAGE];

    const int wave = wave_id(), lane = lane_id();
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, kh = lane >> 5;

    // XCD-aware tile order.  Workgroup ids are dealt round-robin to the 8 XCDs
    // (each with its own L2), so id L runs on XCD L % 8, and XCD x takes the
    // contiguous range of tile numbers [x * W/8, (x+1) * W/8).  Tiles are
    // numbered M-block-major (t = mb * nN + nb: the workgroups sharing an XCD
    // work on the same activation rows and find them in its L2) or, with
    // n_major, N-block-major (t = nb * nM + mb: they share weight tiles, which
    // then cross HBM once; the host picks whichever operand is larger per XCD).
    const int64_t nN = gridDim.x, nM = gridDim.y, W = nN * nM;
    const int64_t L = blockIdx.x + nN * blockIdx.y;
    int64_t t;
    {
        const int64_t per = W / 8, rem = W % 8, x = L % 8, j = L / 8;
        t = x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
    }
    const int64_t m0 = (n_major ? t % nM : t / nN) * BM;
    const int64_t n0 = (n_major ? t / nM : t % nN) * BN;
    const int64_t nstages = (KB + KBS - 1) / KBS;

    // ---- copy sources, fixed for the whole loop ------------------------------
    // The copies are buffer loads.  The hardware range check of a buffer
    // resource turns every read past its end into zeros without touching
    // memory, so rows past M, tiles past NT and the k tail need no clamping.
    // Rows and tiles that do not exist only feed outputs that are never
    // stored, and k positions past K meet zero weights (pad codes, or words
    // replaced in the last stage), so whatever they read is harmless.
    //
    // Activation copy j of this wave: k-half h = j / A_RB, row
    // wave*A_ROWS_W + 8 (j % A_RB) + lane/8, LDS slot lane%8 of the half's
    // 128-byte row, which holds the row's 16-byte unit (lane%8) ^ swz(row).
    //
    // b3: copy c (c = wave * A_INST + j, taken modulo A_COPIES: the last waves
    // repeat a few copies, which write the same bytes again) moves units
    // 64 c + lane of the stage, unit U = 10 row + g holding bytes 16 g .. 16 g
    // + 15 of the row's 160.
    int a_voff[A_INST], a_dst[A_INST];
#pragma unroll
    for (int j = 0; j < A_INST; ++j) {
        if constexpr (B3) {
            const int c = (wave * A_INST + j) % A_COPIES;
            const int u = c * 64 + lane;
            a_voff[j] = static_cast<int>((u / 10) * ldq) + (u % 10) * 16;
            a_dst[j] = c * 1024;
        } else {
            const int row = wave * A_ROWS_W + 8 * (j % A_RB) + (lane >> 3);
            a_voff[j] = static_cast<int>(row * ldq) + (j / A_RB) * KSTEP + ((lane & 7) ^ a_swz(row)) * 16;
            a_dst[j] = (j / A_RB) * BM * KSTEP + (wave * A_ROWS_W + 8 * (j % A_RB)) * KSTEP;
        }
    }
    // Weight copy j of this wave covers stage chunk c (c = kb2 * BN/16 + tile,
    // 256 bytes = 16 rows x 16 bytes): with 16-byte copies chunks
    // 4 (wave*B_INST + j) + lane/16, row lane%16; with 4-byte copies chunk
    // wave*B_INST + j, row lane/4, word lane%4.
    int b_voff[B_INST];
#pragma unroll
    for (int j = 0; j < B_INST; ++j) {
        const int c = B_CP == 16 ? (wave * B_INST + j) * 4 + (lane >> 4) : wave * B_INST + j;
        const int in_chunk = B_CP == 16 ? (lane & 15) * 16 : (lane >> 2) * 16 + (lane & 3) * 4;
        b_voff[j] = static_cast<int>((c % (BN / 16)) * KB * 256 + (c / (BN / 16)) * 256 + in_chunk);
    }
    // Bytes the resources cover from the block's first row / tile: rows m0 ..
    // min(M, m0+BM)-1, the last one up to column K rounded up to 16 (the range
    // check drops whole dwords, and the 16-byte-aligned unit holding the row's
    // last byte never crosses a page); tiles n0/16 .. min(NT, (n0+BN)/16)-1.
    const int64_t rows = (M - m0 < BM ? M - m0 : BM);
    const int64_t a_bytes = (rows - 1) * ldq + ((K + 15) & ~int64_t(15));
    const int64_t tiles = (NT - n0 / 16 < BN / 16 ? NT - n0 / 16 : BN / 16);
    const int64_t b_bytes = tiles * KB * 256;
    const int8_t *a_base = Xq + m0 * ldq;
    const uint8_t *b_base = P + (n0 / 16) * KB * 256;

    // Issue the copies of stage st into ring slot buf.  Stages past the last
    // read nothing (their resources are empty) and are never used.
    auto issue = [&](int64_t st, int buf) {
        int8_t *sbase = lds + buf * STAGE;
        const int64_t ka = st * KS_, kb = st * KBS * 256;
        const int na = static_cast<int>(a_bytes > ka ? a_bytes - ka : 0);
        const int nb = static_cast<int>(b_bytes > kb ? b_bytes - kb : 0);
#pragma unroll
        for (int j = 0; j < A_INST; ++j)
            buffer_copy_to_lds<16>(a_base + ka, na, (lds_void_t *)(sbase + a_dst[j]), a_voff[j]);
#pragma unroll
        for (int j = 0; j < B_INST; ++j)
            buffer_copy_to_lds<B_CP>(b_base + kb, nb, (lds_void_t *)(sbase + A_BYTES + (wave * B_INST + j) * 64 * B_CP),
                                     b_voff[j]);
    };

    // ---- operand read offsets within a stage ---------------------------------
    int a_off[MI][KK];
#pragma unroll
    for (int a = 0; a < MI; ++a) {
        const int row = wm * (BM / WM) + a * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            a_off[a][kk] = B3 ? (row * 10 + 5 * kh + kk) * 16
                              : (kk / 4) * BM * KSTEP + row * KSTEP + (((2 * (kk % 4) + kh) ^ a_swz(row)) * 16);
    }
    // i2: word (kk % 2) * 2 + kh of the row in k-block kk / 2 (added in
    // read_ops); b3: the whole chunk row of k-block kh; b1: the whole chunk row
    int b_off[NI];
#pragma unroll
    for (int b = 0; b < NI; ++b) {
        const int nl = wn * (BN / WN) + b * 32 + l32;
        b_off[b] = B3 ? A_BYTES + (kh * (BN / 16) + nl / 16) * 256 + (nl % 16) * 16
                      : A_BYTES + (nl / 16) * 256 + (nl % 16) * 16 + (B1 ? 0 : 4 * kh);
    }

    // A wave with fewer than 4 output tiles keeps SPLIT accumulators per tile
    // (k-step kk adds into copy kk % SPLIT), so that consecutive MFMAs of a
    // stage do not wait on each other's results; the copies are summed at the
    // end (exact: integer sums).
    constexpr int SPLIT = MI * NI >= 4 ? 1 : 4 / (MI * NI);
    v16i acc[MI][NI][SPLIT];
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NI; ++b)
#pragma unroll
            for (int c = 0; c < SPLIT; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[a][b][c][r] = 0;

    // Operands of one stage, read from LDS one stage ahead of their MFMAs so
    // that LDS latency overlaps the matrix work of the stage before.
    struct Ops {
        v4i a[MI][KK];         // activation operand of tile a, k-step kk
        uint32_t w[NI][NWORD]; // i2: packed word of B tile b, k-step kk; b3, b1: the chunk row's words
    };
    auto read_ops = [&](int buf, Ops &o) {
        const int8_t *sbase = lds + buf * STAGE;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int a = 0; a < MI; ++a) o.a[a][kk] = *reinterpret_cast<const v4i *>(sbase + a_off[a][kk]);
        if constexpr (B3 || B1) {
#pragma unroll
            for (int b = 0; b < NI; ++b) {
                const uint4 v = *reinterpret_cast<const uint4 *>(sbase + b_off[b]);
                o.w[b][0] = v.x;
                o.w[b][1] = v.y;
                o.w[b][2] = v.z;
                o.w[b][3] = v.w;
            }
        } else {
            // word of k-block kk/2, 16-weight group (kk % 2) * 2 + kh
#pragma unroll
            for (int b = 0; b < NI; ++b)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    o.w[b][kk] = *reinterpret_cast<const uint32_t *>(sbase + b_off[b] + (kk / 2) * (BN / 16) * 256 +
                                                                     (kk % 2) * 8);
        }
    };
    // kb_left: k-blocks of the stage that exist (>= 2S except in the last
    // stage); the words of the others become T = 0.  b1: k_left, the k of the
    // stage before K (>= 128 except in the last stage).
    auto mma = [&](const Ops &o, int kb_left, auto last) {
        if constexpr (B1) {
            // weights 32 kk + 16 kh + 4 q + j (byte j of dword q) exist when
            // below k_left; only the last stage (peeled off the loop, so the
            // loop body holds the plain decode alone) masks
            const int k_left = kb_left;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int nv = k_left - 32 * kk - 16 * kh;
                v4i bf[NI];
#pragma unroll
                for (int b = 0; b < NI; ++b)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t bits = (o.w[b][kk] >> (4 * kh + q)) & 0x01010101u;
                        uint32_t v = __builtin_amdgcn_perm(0u, 0x000001ffu, bits);
                        if constexpr (decltype(last)::value) {
                            const int e = nv - 4 * q; // bytes of this dword that exist
                            v &= e >= 4 ? 0xffffffffu : (e <= 0 ? 0u : (1u << (8 * e)) - 1u);
                        }
                        bf[b][q] = static_cast<int>(v);
                    }
#pragma unroll
                for (int a = 0; a < MI; ++a)
#pragma unroll
                    for (int b = 0; b < NI; ++b)
                        acc[a][b][kk % SPLIT] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            o.a[a][kk], bf[b], acc[a][b][kk % SPLIT], 0, 0, 0);
            }
        } else if constexpr (B3) {
            // k-block kh exists unless kb_left == 1; a missing block's words
            // become the all-zero-weight word before decoding
            v4i bf[NI][5];
#pragma unroll
            for (int b = 0; b < NI; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const B3Digits dg = b3_word_digits(kh < kb_left ? o.w[b][q] : B3_ZERO_WORD);
#pragma unroll
                    for (int t = 0; t < 5; ++t)
                        bf[b][t][q] = static_cast<int>(__builtin_amdgcn_perm(0u, 0x000100ffu, dg.d[t]));
                }
#pragma unroll
            for (int t = 0; t < 5; ++t)
#pragma unroll
                for (int a = 0; a < MI; ++a)
#pragma unroll
                    for (int b = 0; b < NI; ++b)
                        acc[a][b][t % SPLIT] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[a][t], bf[b][t],
                                                                                     acc[a][b][t % SPLIT], 0, 0, 0);
        } else {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                v4i bf[NI];
#pragma unroll
                for (int b = 0; b < NI; ++b)
                    bf[b] = gemm_i2_word_signed((kk < 2 || kk / 2 < kb_left) ? o.w[b][kk] : I2_ZERO_WORD);
#pragma unroll
                for (int a = 0; a < MI; ++a)
#pragma unroll
                    for (int b = 0; b < NI; ++b)
                        acc[a][b][kk % SPLIT] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[a][kk], bf[b],
                                                                                      acc[a][b][kk % SPLIT], 0, 0, 0);
            }
        }
    };

    // The ring holds NST stages.  Before the MFMAs of stage st: stage st's
    // operands are in registers, stage st+1 has landed in LDS (waited for and
    // read into the other register set in this step), and stages st+2 ..
    // st+NST are in flight; stage st+NST goes into the slot stage st has left.
#pragma unroll
    for (int s = 0; s < NST; ++s) issue(s, s);
    __builtin_amdgcn_s_waitcnt(vmcnt_only((NST - 1) * LOADS));
    stage_barrier();
    Ops o0, o1;
    read_ops(0, o0);
    int slot = 0; // ring slot of stage st
    auto step = [&](int64_t st, const Ops &cur, Ops &nxt, auto last) {
        const int nslot = slot == NST - 1 ? 0 : slot + 1;
        // this wave's copies of stage st+1 are done once at most NST-2 later
        // stages' copies are outstanding, and its reads of stage st are back;
        // the barrier extends both to every wave
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0((NST - 2) * LOADS));
        stage_barrier();
        issue(st + NST, slot);
        read_ops(nslot, nxt);
        if constexpr (B1) {
            const int64_t left = K - KS_ * st;
            mma(cur, static_cast<int>(left < KS_ ? left : KS_), last);
        } else {
            const int64_t left = KB - KBS * st;
            mma(cur, static_cast<int>(left < KBS ? left : KBS), last);
        }
        slot = nslot;
    };
    int64_t st = 0;
    if constexpr (B1) {
        // the last stage, the only one that can hold pad weights, on its own
        const std::false_type body{};
        const std::true_type last{};
        for (; st + 2 < nstages; st += 2) {
            step(st, o0, o1, body);
            step(st + 1, o1, o0, body);
        }
        if (st + 1 < nstages) {
            step(st, o0, o1, body);
            step(st + 1, o1, o0, last);
        } else {
            step(st, o0, o1, last);
        }
    } else {
        const std::false_type any{};
        for (; st + 1 < nstages; st += 2) {
            step(st, o0, o1, any);
            step(st + 1, o1, o0, any);
        }
        if (st < nstages) step(st, o0, o1, any);
    }

    // ---- epilogue ------------------------------------------------------------
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NI; ++b)
#pragma unroll
            for (int c = 1; c < SPLIT; ++c) acc[a][b][0] += acc[a][b][c];
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0)); // the clamped tail copies still land in LDS
    stage_barrier();
    float *scale = reinterpret_cast<float *>(lds);
    for (int i = threadIdx.x; i < BM; i += 64 * NW) {
        const int64_t m = m0 + i;
        scale[i] = m < M ? token_scale(*gamma_p, beta[m]) : 0.0f;
    }
    __syncthreads();

    // 32 x 32 output layout: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
    auto store_all = [&](auto put) {
#pragma unroll
        for (int a = 0; a < MI; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lrow = wm * (BM / WM) + a * 32 + 8 * (r / 4) + 4 * kh + (r % 4);
                const int64_t m = m0 + lrow;
                if (m >= M) continue;
                const float sc = scale[lrow];
#pragma unroll
                for (int b = 0; b < NI; ++b) {
                    const int64_t n = n0 + wn * (BN / WN) + b * 32 + l32;
                    if (n < N) put(m * ldy + n, acc[a][b][0][r], sc);
                }
            }
    };
    if (y_dtype == DT_F32)
        store_all([&](int64_t i, int v, float sc) { static_cast<float *>(Y)[i] = static_cast<float>(v) * sc; });
    else if (y_dtype == DT_BF16)
        store_all([&](int64_t i, int v, float sc) {
            static_cast<uint16_t *>(Y)[i] = float_to_bf16_rne(static_cast<float>(v) * sc);
        });
    else
        store_all([&](int64_t i, int v, float) { static_cast<int *>(Y)[i] = v; });
}

template <int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_mfma_i2(const uint8_t *__restrict__ P, int64_t KB,
                                                               int64_t NT, const float *__restrict__ gamma_p,
                                                               const int8_t *__restrict__ Xq, int64_t ldq,
                                                               const float *__restrict__ beta, int64_t M,
                                                               int64_t N, int64_t K, void *__restrict__ Y,
                                                               int y_dtype, int64_t ldy, int n_major)
{
    gemm_body<LAYOUT_I2, BM, BN, WM, WN, S>(P, KB, NT, gamma_p, Xq, ldq, beta, M, N, K, Y, y_dtype, ldy, n_major);
}

template <int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_mfma_b1(const uint8_t *__restrict__ P, int64_t KB,
                                                               int64_t NT, const float *__restrict__ gamma_p,
                                                               const int8_t *__restrict__ Xq, int64_t ldq,
                                                               const float *__restrict__ beta, int64_t M,
                                                               int64_t N, int64_t K, void *__restrict__ Y,
                                                               int y_dtype, int64_t ldy, int n_major)
{
    gemm_body<LAYOUT_B1, BM, BN, WM, WN, S>(P, KB, NT, gamma_p, Xq, ldq, beta, M, N, K, Y, y_dtype, ldy, n_major);
}

template <int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_mfma_b3(const uint8_t *__restrict__ P, int64_t KB,
                                                               int64_t NT, const float *__restrict__ gamma_p,
                                                               const int8_t *__restrict__ Xq, int64_t ldq,
                                                               const float *__restrict__ beta, int64_t M,
                                                               int64_t N, int64_t K, void *__restrict__ Y,
                                                               int y_dtype, int64_t ldy, int n_major)
{
    gemm_body<LAYOUT_B3, BM, BN, WM, WN, S>(P, KB, NT, gamma_p, Xq, ldq, beta, M, N, K, Y, y_dtype, ldy, n_major);
}

namespace {
template <int LAYOUT, int BM, int BN, int WM, int WN, int S>
hipError_t launch_tile(const GemvArgs &a, hipStream_t stream)
{
    const int64_t NT = (a.N + 15) / 16;
    const int64_t KB = LAYOUT == LAYOUT_B3 ? (a.K + 79) / 80 : (LAYOUT == LAYOUT_B1 ? (a.K + 127) / 128 : (a.K + 63) / 64);
    const int64_t nN = (a.N + BN - 1) / BN, nM = (a.M + BM - 1) / BM;
    dim3 grid(static_cast<unsigned>(nN), static_cast<unsigned>(nM));
    // bytes one XCD reads per tile order: M-block-major: its share of the
    // activation row blocks plus every weight tile; N-block-major: its share of
    // the weight tiles plus every activation row
    const double act = static_cast<double>(a.M) * a.K,
                 wts = static_cast<double>(a.N) * a.K / (LAYOUT == LAYOUT_B3 ? 5 : (LAYOUT == LAYOUT_B1 ? 8 : 4));
    const double m_major = act / 8 + wts, n_major = wts / 8 + act;
    const int nmaj = (nM > 1 && n_major < m_major) ? 1 : 0;
    if constexpr (LAYOUT == LAYOUT_B3)
        hipLaunchKernelGGL((k_gemm_mfma_b3<BM, BN, WM, WN, S>), grid, dim3(64 * WM * WN), 0, stream, a.P, KB, NT,
                           a.gamma, a.Xq, a.ldq, a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy, nmaj);
    else if constexpr (LAYOUT == LAYOUT_B1)
        hipLaunchKernelGGL((k_gemm_mfma_b1<BM, BN, WM, WN, S>), grid, dim3(64 * WM * WN), 0, stream, a.P, KB, NT,
                           a.gamma, a.Xq, a.ldq, a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy, nmaj);
    else
        hipLaunchKernelGGL((k_gemm_mfma_i2<BM, BN, WM, WN, S>), grid, dim3(64 * WM * WN), 0, stream, a.P, KB, NT,
                           a.gamma, a.Xq, a.ldq, a.beta, a.M, a.N, a.K, a.Y, a.y_dtype, a.ldy, nmaj);
    return hipGetLastError();
}
} // namespace

namespace {
// Tile shapes on offer, with their sustained rates relative to each other
// (measured; for the small tiles, fitted to 32-176-token products of the
// 70B layers, where latency or the b3 decode rather than the matrix cores
// bounds a tile).  A launch costs about ceil(tiles / 256 CUs) rounds of one
// tile each.  The 64 x 128 tile serves b3 only: at 64 tokens it decodes each
// weight tile once instead of twice.  The 160 x 256 tile (4 waves of 160 x
// 64, one wave per SIMD) is slower per tile but packs 2048 x 8640 into two
// full rounds (442 tiles) where 128 x 256 needs a third, one-eighth full
// (544 tiles): 86 -> 76 us there, and the cost model keeps 128 x 256 where
// the tile count fits one round either way.
struct GemmTile {
    int bm, bn, wm, wn, s; // tile, wave grid, k halves (of 128) per stage
    double rate;
    bool i2, b3, b1; // offered for these weights (the b3 decode, and the b1 tail mask, of a 128 x 128 wave
                     // tile spill registers)
};
constexpr GemmTile kTiles[] = {{256, 256, 2, 2, 1, 2.1, true, false, false},
                               {128, 256, 2, 4, 1, 1.95, true, true, true},
                               {128, 128, 2, 2, 1, 1.5, true, true, true},
                               {32, 128, 1, 4, 1, 1.1, true, true, true},
                               {64, 128, 1, 4, 1, 1.3, false, true, false},
                               {160, 256, 1, 4, 1, 1.85, true, false, false}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
constexpr int64_t kCUs = 256;

int best_tile(int layout, int64_t M, int64_t N)
{
    int best = -1;
    double best_cost = 0;
    for (int i = 0; i < kNumTiles; ++i) {
        if (layout == LAYOUT_B3 ? !kTiles[i].b3 : (layout == LAYOUT_B1 ? !kTiles[i].b1 : !kTiles[i].i2)) continue;
        const int64_t t = ((M + kTiles[i].bm - 1) / kTiles[i].bm) * ((N + kTiles[i].bn - 1) / kTiles[i].bn);
        const double cost = static_cast<double>((t + kCUs - 1) / kCUs) * kTiles[i].bm * kTiles[i].bn / kTiles[i].rate;
        if (best < 0 || cost < best_cost) best = i, best_cost = cost;
    }
    return best;
}

template <int I>
hipError_t launch_entry(const GemvArgs &a, hipStream_t stream)
{
    constexpr GemmTile t = kTiles[I];
    if constexpr (t.b3)
        if (a.layout == LAYOUT_B3) return launch_tile<LAYOUT_B3, t.bm, t.bn, t.wm, t.wn, t.s>(a, stream);
    if constexpr (t.b1)
        if (a.layout == LAYOUT_B1) return launch_tile<LAYOUT_B1, t.bm, t.bn, t.wm, t.wn, t.s>(a, stream);
    if constexpr (t.i2) return launch_tile<LAYOUT_I2, t.bm, t.bn, t.wm, t.wn, t.s>(a, stream);
    return hipErrorInvalidValue; // not reached: best_tile offers the tile only for its layouts
}
} // namespace

int64_t gemm_tiles(int64_t M, int64_t N)
{
    // in units of 64 x 128 (the GEMV / GEMM crossover was measured in these)
    return ((M + 63) / 64) * ((N + 127) / 128);
}

void gemm_kernel_name(int layout, int64_t M, int64_t N, char *buf, size_t n)
{
    const GemmTile &t = kTiles[best_tile(layout, M, N)];
    snprintf(buf, n, "bl::k_gemm_mfma_%s<%d, %d, %d, %d, %d>",
             layout == LAYOUT_B3 ? "b3" : (layout == LAYOUT_B1 ? "b1" : "i2"), t.bm, t.bn, t.wm, t.wn, t.s);
}

hipError_t launch_gemm_mfma(const GemvArgs &a, hipStream_t stream)
{
    static_assert(kNumTiles == 6, "one case per tile shape");
    switch (best_tile(a.layout, a.M, a.N)) {
    case 0: return launch_entry<0>(a, stream);
    case 1: return launch_entry<1>(a, stream);
    case 2: return launch_entry<2>(a, stream);
    case 3: return launch_entry<3>(a, stream);
    case 4: return launch_entry<4>(a, stream);
    default: return launch_entry<5>(a, stream);
    }
}

} // namespace bl
