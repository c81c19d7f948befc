// api.cpp -- the C ABI of libbitlinear (declared in include/bitlinear.h).
// Validates every argument on the host, then enqueues the kernels.  Nothing is
// launched when validation fails.  No allocation, no synchronisation, no
// mutable global state.
#include "bitlinear.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

#include <atomic>

// Allocation-free forwards (bitlinear_forward_noalloc): the workspace is this
// file-scope device array, one per GPU the library runs on, held until the
// process ends.  In host code 'scratch' is only a stand-in for the symbol;
// its device address comes from hipGetSymbolAddress (scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[BITLINEAR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40; // keeps per-exponent sums of |W| below 2^64
// Largest M the single-layer add/subtract GEMV (k_gemv_addsub) takes when the
// kernel is chosen automatically.  Measured on MI355X the single-layer
// matrix-core GEMVs are faster at every M (the vector ALU reaches 4 int8 MACs
// per lane-cycle, the matrix core takes the MACs off it), so automatic
// dispatch of bitlinear_forward never picks it; it stays available as
// BITLINEAR_ALGO_GEMV_ADDSUB.  (The grouped forward's add/sub products are
// another kernel: group_algo.)
constexpr int64_t kAddSubMaxM = 0;
// Fewest GEMM workgroup tiles for which the GEMM beats the matrix-core GEMV
// (token groups of 16) when there are more than 16 tokens: with fewer tiles
// most CUs idle (measured on the 70B k/v and q layers at 64 and 176 tokens).
constexpr int64_t kGemmMinTiles = 128;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

int dtype_size(int dt)
{
    switch (dt) {
    case BITLINEAR_F32: return 4;
    case BITLINEAR_BF16: return 2;
    case BITLINEAR_I8: return 1;
    case BITLINEAR_I32: return 4;
    case BITLINEAR_I8_TILED: return 1;
    default: return 0;
    }
}

struct Span {
    uintptr_t lo, hi; // [lo, hi)
};

Span span_of(const void *p, int64_t rows, int64_t ld, int64_t cols, int elem)
{
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    uintptr_t bytes = static_cast<uintptr_t>(((rows - 1) * ld + cols) * elem);
    return {lo, lo + bytes};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Row strides are bounded so that no offset (rows - 1) * ld * 4 bytes, on the
// host or in a kernel, can overflow 64 bits: ld <= 2^40 elements and the
// rows span at most 2^44 elements.
constexpr int64_t kMaxLd = int64_t(1) << 40, kMaxSpan = int64_t(1) << 44;
bool stride_ok(int64_t rows, int64_t ld) { return ld <= kMaxLd && rows - 1 <= kMaxSpan / ld; }

int status_of(hipError_t e) { return e == hipSuccess ? BITLINEAR_OK : BITLINEAR_ERR_LAUNCH; }

bool valid_layout(int layout)
{
    return layout == BITLINEAR_LAYOUT_I2 || layout == BITLINEAR_LAYOUT_B3 || layout == BITLINEAR_LAYOUT_B1;
}

// Staged activations of the fused quantiser: row-major Xq [M x round_up(K, 64)]
// or the tiled layout, whichever is larger, then beta [M].
int64_t staged_ldq(int64_t K) { return round_up(K, 64); }
constexpr int64_t kTiledMaxK = 65536; // the tiled quantiser keeps a row's pieces in registers
int64_t staged_xq_bytes(int64_t M, int64_t K, int layout)
{
    int64_t rm = M * staged_ldq(K);
    int64_t tl = K <= kTiledMaxK ? bl::tiled_bytes(M, K, layout) : 0;
    return round_up(rm > tl ? rm : tl, 256);
}

// Workspace of one forward: the quantised activations and beta (bf16/fp32
// input).  Every product reads the caller's packed weights in their own
// layout (the GEMM decodes b3 and b1 itself): no forward writes weights.
int64_t staging_bytes(int64_t M, int64_t K, int layout, int x_dtype)
{
    if (x_dtype == BITLINEAR_I8 || x_dtype == BITLINEAR_I8_TILED) return 0;
    return staged_xq_bytes(M, K, layout) + round_up(4 * M, 256);
}

// The GEMM addresses the activation rows of one workgroup tile (at most 256
// rows) with 32-bit offsets from the tile's first row (buffer resources), so
// those rows must span less than 2^31 bytes.  Staged activations always do;
// caller-quantised rows with a huge stride may not.
constexpr int64_t kGemmMaxTileRows = 256;
bool gemm_offsets_fit(int64_t M, int64_t K, int64_t ldq)
{
    const int64_t rows = M < kGemmMaxTileRows ? M : kGemmMaxTileRows;
    return (rows - 1) * ldq + round_up(K, 16) <= int64_t(INT32_MAX);
}

// The product kernel of algo AUTO (sizes already validated).
int auto_algo(int64_t M, int64_t N, int layout, int x_dtype)
{
    if (x_dtype == BITLINEAR_I8_TILED) return BITLINEAR_ALGO_GEMV_MFMA;
    if (M <= 16)
        return (layout == BITLINEAR_LAYOUT_I2 && M <= kAddSubMaxM) ? BITLINEAR_ALGO_GEMV_ADDSUB
                                                                   : BITLINEAR_ALGO_GEMV_MFMA;
    return bl::gemm_tiles(M, N) >= kGemmMinTiles ? BITLINEAR_ALGO_GEMM_MFMA : BITLINEAR_ALGO_GEMV_MFMA;
}

} // namespace

extern "C" {

const char *bitlinear_status_string(int status)
{
    switch (status) {
    case BITLINEAR_OK: return "ok";
    case BITLINEAR_ERR_INVALID_ARG: return "invalid argument";
    case BITLINEAR_ERR_UNSUPPORTED: return "unsupported combination of arguments";
    case BITLINEAR_ERR_WORKSPACE: return "workspace missing or too small";
    case BITLINEAR_ERR_LAUNCH: return "kernel launch failed";
    case BITLINEAR_ERR_DEVICE: return "no usable gfx950 device";
    case BITLINEAR_ERR_SCRATCH: return "request needs more than the allocation-free scratch (BITLINEAR_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

int bitlinear_version(void) { return 101; }

int64_t bitlinear_packed_bytes(int64_t N, int64_t K, int layout)
{
    if (N < 1 || K < 1 || K > BITLINEAR_MAX_K || N > kMaxElems || !valid_layout(layout)) return -1;
    const int64_t NT = (N + 15) / 16;
    const int64_t KB = layout == BITLINEAR_LAYOUT_I2 ? (K + 63) / 64
                       : layout == BITLINEAR_LAYOUT_B3 ? (K + 79) / 80
                                                       : (K + 127) / 128;
    return NT * KB * 256;
}

int64_t bitlinear_quantize_weights_workspace_bytes(int64_t N, int64_t K)
{
    if (N < 1 || K < 1 || N > kMaxElems / K) return -1;
    return 256 * 8; // 256 per-exponent uint64 sums
}

int64_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K, int layout, int x_dtype)
{
    if (M < 1 || M > BITLINEAR_MAX_M || N < 1 || K < 1 || K > BITLINEAR_MAX_K || !valid_layout(layout))
        return -1;
    if (x_dtype != BITLINEAR_I8 && x_dtype != BITLINEAR_I8_TILED && x_dtype != BITLINEAR_F32 &&
        x_dtype != BITLINEAR_BF16)
        return -1;
    return staging_bytes(M, K, layout, x_dtype);
}

int bitlinear_auto_algo(int64_t M, int64_t N, int64_t K, int layout, int x_dtype)
{
    if (M < 1 || M > BITLINEAR_MAX_M || N < 1 || N > (int64_t(1) << 31) || K < 1 || K > BITLINEAR_MAX_K ||
        !valid_layout(layout))
        return -1;
    if (x_dtype != BITLINEAR_F32 && x_dtype != BITLINEAR_BF16 && x_dtype != BITLINEAR_I8 &&
        x_dtype != BITLINEAR_I8_TILED)
        return -1;
    return auto_algo(M, N, layout, x_dtype);
}

const char *bitlinear_product_kernel(int64_t M, int64_t N, int64_t K, int layout, int x_dtype, int algo)
{
    thread_local char name[96];
    if (bitlinear_auto_algo(M, N, K, layout, x_dtype) < 0 || algo < BITLINEAR_ALGO_AUTO ||
        algo > BITLINEAR_ALGO_GEMM_MFMA)
        return nullptr;
    if (algo == BITLINEAR_ALGO_AUTO) algo = auto_algo(M, N, layout, x_dtype);
    if ((algo == BITLINEAR_ALGO_GEMV_ADDSUB && (M > 16 || layout != BITLINEAR_LAYOUT_I2)) ||
        (x_dtype == BITLINEAR_I8_TILED && algo != BITLINEAR_ALGO_GEMV_MFMA))
        return nullptr;
    if (algo == BITLINEAR_ALGO_GEMV_ADDSUB) {
        bl::gemv_addsub_kernel_name(M, name, sizeof name);
    } else if (algo == BITLINEAR_ALGO_GEMM_MFMA) {
        bl::gemm_kernel_name(layout, M, N, name, sizeof name);
    } else if (algo == BITLINEAR_ALGO_GEMV_MFMA && bl::gemv_fq_shape(layout, M, N, K, x_dtype)) {
        // the quantiser inside the GEMV (for 16-byte aligned rows)
        bl::gemv_fq_kernel_name(layout, M, N, K, x_dtype, name, sizeof name);
    } else {
        // the same choice of activation staging as bitlinear_forward_algo
        const bool tiled = x_dtype == BITLINEAR_I8_TILED ||
                           ((x_dtype == BITLINEAR_F32 || x_dtype == BITLINEAR_BF16) && M > 4 && K <= kTiledMaxK);
        bl::gemv_kernel_name(layout, M, N, K, tiled, name, sizeof name);
    }
    return name;
}

int64_t bitlinear_act_tiled_bytes(int64_t M, int64_t K, int layout)
{
    if (M < 1 || M > BITLINEAR_MAX_M || K < 1 || K > BITLINEAR_MAX_K || !valid_layout(layout)) return -1;
    return bl::tiled_bytes(M, K, layout);
}

// Shared argument checks of the two weight quantisers.
static int check_weight_quant(const float *W, int64_t N, int64_t K, int64_t ldw, const int8_t *T,
                              const float *gamma, const void *ws, int64_t ws_bytes)
{
    if (!W || !T || !gamma) return BITLINEAR_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || ldw < K || N > kMaxElems / K || !stride_ok(N, ldw)) return BITLINEAR_ERR_INVALID_ARG;
    const int64_t need = bitlinear_quantize_weights_workspace_bytes(N, K);
    if (!ws || ws_bytes < need) return BITLINEAR_ERR_WORKSPACE;
    if (!aligned16(ws) || (reinterpret_cast<uintptr_t>(W) & 3u) || (reinterpret_cast<uintptr_t>(gamma) & 3u))
        return BITLINEAR_ERR_INVALID_ARG;
    const Span sw = span_of(W, N, ldw, K, 4), st = span_of(T, N, K, K, 1), sg = span_of(gamma, 1, 1, 1, 4),
               sws = span_of(ws, 1, need, need, 1);
    if (overlap(sw, st) || overlap(sw, sg) || overlap(st, sg) || overlap(sws, sw) || overlap(sws, st) ||
        overlap(sws, sg))
        return BITLINEAR_ERR_INVALID_ARG;
    return BITLINEAR_OK;
}

int bitlinear_binarize_weights(const float *W, int64_t N, int64_t K, int64_t ldw, int8_t *T, float *gamma,
                               void *ws, int64_t ws_bytes, void *stream)
{
    const int st = check_weight_quant(W, N, K, ldw, T, gamma, ws, ws_bytes);
    if (st != BITLINEAR_OK) return st;
    (void)hipGetLastError();
    return status_of(bl::launch_binarize_weights(W, N, K, ldw, T, gamma, ws, as_stream(stream)));
}

int bitlinear_quantize_weights(const float *W, int64_t N, int64_t K, int64_t ldw, int8_t *T, float *gamma,
                               void *ws, int64_t ws_bytes, void *stream)
{
    const int st = check_weight_quant(W, N, K, ldw, T, gamma, ws, ws_bytes);
    if (st != BITLINEAR_OK) return st;
    (void)hipGetLastError();
    return status_of(bl::launch_quantize_weights(W, N, K, ldw, T, gamma, ws, as_stream(stream)));
}

int bitlinear_pack(const int8_t *T, int64_t N, int64_t K, int64_t ldt, int layout, uint8_t *P, void *stream)
{
    if (!T || !P || !valid_layout(layout)) return BITLINEAR_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || K > BITLINEAR_MAX_K || ldt < K || N > kMaxElems / K || !stride_ok(N, ldt))
        return BITLINEAR_ERR_INVALID_ARG;
    if (!aligned16(P)) return BITLINEAR_ERR_INVALID_ARG;
    const int64_t pb = bitlinear_packed_bytes(N, K, layout);
    if (overlap(span_of(T, N, ldt, K, 1), span_of(P, 1, pb, pb, 1))) return BITLINEAR_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return status_of(bl::launch_pack(T, N, K, ldt, layout, P, as_stream(stream)));
}

int bitlinear_transcode_i2(const uint8_t *P, int layout, int64_t N, int64_t K, uint8_t *P2, void *stream)
{
    if (!P || !P2 || (layout != BITLINEAR_LAYOUT_B3 && layout != BITLINEAR_LAYOUT_B1)) return BITLINEAR_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || K > BITLINEAR_MAX_K || N > kMaxElems / K) return BITLINEAR_ERR_INVALID_ARG;
    if (!aligned16(P) || !aligned16(P2)) return BITLINEAR_ERR_INVALID_ARG;
    const int64_t pb = bitlinear_packed_bytes(N, K, layout), p2b = bitlinear_packed_bytes(N, K, BITLINEAR_LAYOUT_I2);
    if (overlap(span_of(P, 1, pb, pb, 1), span_of(P2, 1, p2b, p2b, 1))) return BITLINEAR_ERR_INVALID_ARG;
    (void)hipGetLastError();
    hipStream_t st = as_stream(stream);
    return status_of(layout == BITLINEAR_LAYOUT_B3 ? bl::launch_b3_to_i2(P, N, K, P2, st)
                                                   : bl::launch_b1_to_i2(P, N, K, P2, st));
}

int bitlinear_quantize_act(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t *Xq,
                           int64_t ldq, float *beta, void *stream)
{
    if (!X || !Xq || !beta) return BITLINEAR_ERR_INVALID_ARG;
    if (x_dtype != BITLINEAR_F32 && x_dtype != BITLINEAR_BF16) return BITLINEAR_ERR_INVALID_ARG;
    if (M < 1 || M > BITLINEAR_MAX_M || K < 1 || K > BITLINEAR_MAX_K || ldx < K || ldq < K || ldq % 16 ||
        !stride_ok(M, ldx) || !stride_ok(M, ldq))
        return BITLINEAR_ERR_INVALID_ARG;
    if (!aligned16(Xq) || (reinterpret_cast<uintptr_t>(X) % dtype_size(x_dtype)) ||
        (reinterpret_cast<uintptr_t>(beta) & 3u))
        return BITLINEAR_ERR_INVALID_ARG;
    const Span sx = span_of(X, M, ldx, K, dtype_size(x_dtype)), sq = span_of(Xq, M, ldq, ldq, 1),
               sb = span_of(beta, 1, M, M, 4);
    if (overlap(sx, sq) || overlap(sx, sb) || overlap(sq, sb)) return BITLINEAR_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return status_of(bl::launch_quant_act(X, x_dtype, M, K, ldx, Xq, ldq, beta, as_stream(stream)));
}

int bitlinear_quantize_act_tiled(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int layout,
                                 int8_t *Xt, int64_t xt_bytes, float *beta, void *stream)
{
    if (!X || !Xt || !beta || !valid_layout(layout)) return BITLINEAR_ERR_INVALID_ARG;
    if (x_dtype != BITLINEAR_F32 && x_dtype != BITLINEAR_BF16) return BITLINEAR_ERR_INVALID_ARG;
    if (M < 1 || M > BITLINEAR_MAX_M || K < 1 || K > BITLINEAR_MAX_K || ldx < K || !stride_ok(M, ldx))
        return BITLINEAR_ERR_INVALID_ARG;
    const int64_t need = bl::tiled_bytes(M, K, layout);
    if (xt_bytes < need) return BITLINEAR_ERR_INVALID_ARG;
    if (!aligned16(Xt) || (reinterpret_cast<uintptr_t>(X) % dtype_size(x_dtype)) ||
        (reinterpret_cast<uintptr_t>(beta) & 3u))
        return BITLINEAR_ERR_INVALID_ARG;
    const Span sx = span_of(X, M, ldx, K, dtype_size(x_dtype)), st = span_of(Xt, 1, need, need, 1),
               sb = span_of(beta, 1, M, M, 4);
    if (overlap(sx, st) || overlap(sx, sb) || overlap(st, sb)) return BITLINEAR_ERR_INVALID_ARG;
    if (K > kTiledMaxK) return BITLINEAR_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    return status_of(bl::launch_quant_act_tiled(X, x_dtype, M, K, ldx, layout, Xt, beta, as_stream(stream)));
}

static int forward_impl(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                        const void *X, int x_dtype, int64_t ldx, const float *beta_in, void *Y, int y_dtype,
                        int64_t ldy, void *ws, int64_t ws_bytes, int8_t *Xq_out, int64_t ldxq, float *beta_out,
                        int algo, void *stream, bool check_only = false)
{
    if (!P || !gamma || !X || !Y || !valid_layout(layout)) return BITLINEAR_ERR_INVALID_ARG;
    if (M < 1 || M > BITLINEAR_MAX_M || N < 1 || N > (int64_t(1) << 31) || K < 1 || K > BITLINEAR_MAX_K)
        return BITLINEAR_ERR_INVALID_ARG;
    if (x_dtype != BITLINEAR_F32 && x_dtype != BITLINEAR_BF16 && x_dtype != BITLINEAR_I8 &&
        x_dtype != BITLINEAR_I8_TILED)
        return BITLINEAR_ERR_INVALID_ARG;
    const bool x_int8 = x_dtype == BITLINEAR_I8 || x_dtype == BITLINEAR_I8_TILED;
    if (y_dtype != BITLINEAR_F32 && y_dtype != BITLINEAR_BF16 && y_dtype != BITLINEAR_I32)
        return BITLINEAR_ERR_INVALID_ARG;
    if ((x_dtype != BITLINEAR_I8_TILED && (ldx < K || !stride_ok(M, ldx))) || ldy < N || !stride_ok(M, ldy))
        return BITLINEAR_ERR_INVALID_ARG;
    if (algo < BITLINEAR_ALGO_AUTO || algo > BITLINEAR_ALGO_GEMM_MFMA) return BITLINEAR_ERR_INVALID_ARG;
    if (x_int8 != (beta_in != nullptr)) return BITLINEAR_ERR_INVALID_ARG;
    // quantiser outputs: both or neither, only for fp32 / bf16 input
    const bool q_out = Xq_out != nullptr;
    if (q_out != (beta_out != nullptr) || (q_out && x_int8)) return BITLINEAR_ERR_INVALID_ARG;
    if (q_out && (ldxq < K || ldxq % 16 || !stride_ok(M, ldxq) || !aligned16(Xq_out) ||
                  (reinterpret_cast<uintptr_t>(beta_out) & 3u)))
        return BITLINEAR_ERR_INVALID_ARG;
    if (!aligned16(P) || (reinterpret_cast<uintptr_t>(gamma) & 3u) ||
        (reinterpret_cast<uintptr_t>(X) % dtype_size(x_dtype)) ||
        (reinterpret_cast<uintptr_t>(Y) % dtype_size(y_dtype)))
        return BITLINEAR_ERR_INVALID_ARG;
    if (x_dtype == BITLINEAR_I8 && (!aligned16(X) || ldx % 16 || (reinterpret_cast<uintptr_t>(beta_in) & 3u)))
        return BITLINEAR_ERR_INVALID_ARG;
    if (x_dtype == BITLINEAR_I8_TILED && (!aligned16(X) || (reinterpret_cast<uintptr_t>(beta_in) & 3u)))
        return BITLINEAR_ERR_INVALID_ARG;

    // with the quantiser's outputs requested the product reads them (as I8 input)
    const int64_t need = bitlinear_forward_workspace_bytes(M, N, K, layout, q_out ? BITLINEAR_I8 : x_dtype);
    // (check_only: every check but the workspace's, which the caller owns)
    if (!check_only && need > 0 && (!ws || ws_bytes < need)) return BITLINEAR_ERR_WORKSPACE;
    if (need > 0 && ws && !aligned16(ws)) return BITLINEAR_ERR_INVALID_ARG;

    const int64_t pb = bitlinear_packed_bytes(N, K, layout);
    const int64_t xt = bl::tiled_bytes(M, K, layout);
    const Span sp = span_of(P, 1, pb, pb, 1),
               sx = x_dtype == BITLINEAR_I8_TILED ? span_of(X, 1, xt, xt, 1) : span_of(X, M, ldx, K, dtype_size(x_dtype)),
               sy = span_of(Y, M, ldy, N, dtype_size(y_dtype)), sg = span_of(gamma, 1, 1, 1, 4);
    if (overlap(sy, sp) || overlap(sy, sx) || overlap(sy, sg)) return BITLINEAR_ERR_INVALID_ARG;
    if (beta_in && overlap(sy, span_of(beta_in, 1, M, M, 4))) return BITLINEAR_ERR_INVALID_ARG;
    if (need > 0 && ws) {
        const Span sw = span_of(ws, 1, need, need, 1);
        if (overlap(sw, sp) || overlap(sw, sx) || overlap(sw, sy) || overlap(sw, sg))
            return BITLINEAR_ERR_INVALID_ARG;
    }
    if (q_out) {
        const Span sq = span_of(Xq_out, M, ldxq, ldxq, 1), sb = span_of(beta_out, 1, M, M, 4);
        const Span others[] = {sp, sx, sy, sg};
        for (const Span &o : others)
            if (overlap(sq, o) || overlap(sb, o)) return BITLINEAR_ERR_INVALID_ARG;
        if (overlap(sq, sb)) return BITLINEAR_ERR_INVALID_ARG;
        if (need > 0 && ws) {
            const Span sw = span_of(ws, 1, need, need, 1);
            if (overlap(sw, sq) || overlap(sw, sb)) return BITLINEAR_ERR_INVALID_ARG;
        }
    }

    const int64_t ldq_user = x_dtype == BITLINEAR_I8 ? ldx : (q_out ? ldxq : 0);
    const bool user_rows = x_dtype == BITLINEAR_I8 || q_out;
    if (algo == BITLINEAR_ALGO_GEMM_MFMA && user_rows && !gemm_offsets_fit(M, K, ldq_user))
        return BITLINEAR_ERR_UNSUPPORTED;
    if (algo == BITLINEAR_ALGO_AUTO) {
        algo = auto_algo(M, N, layout, q_out ? BITLINEAR_I8 : x_dtype);
        if (algo == BITLINEAR_ALGO_GEMM_MFMA && user_rows && !gemm_offsets_fit(M, K, ldq_user))
            algo = BITLINEAR_ALGO_GEMV_MFMA; // 64-bit row addressing
    }
    if (algo == BITLINEAR_ALGO_GEMV_ADDSUB && (M > 16 || layout != BITLINEAR_LAYOUT_I2))
        return BITLINEAR_ERR_UNSUPPORTED;
    if (x_dtype == BITLINEAR_I8_TILED && algo != BITLINEAR_ALGO_GEMV_MFMA) return BITLINEAR_ERR_UNSUPPORTED;
    if (check_only) return BITLINEAR_OK;

    (void)hipGetLastError();
    hipStream_t st = as_stream(stream);
    bl::GemvArgs a;
    a.P = P;
    a.layout = layout;
    a.gamma = gamma;
    a.M = M;
    a.N = N;
    a.K = K;
    a.Y = Y;
    a.y_dtype = y_dtype;
    a.ldy = ldy;
    a.tiled = false;
    if (q_out) {
        // the quantiser writes the caller's buffers; the product reads them
        const hipError_t e = bl::launch_quant_act(X, x_dtype, M, K, ldx, Xq_out, ldxq, beta_out, st);
        if (e != hipSuccess) return BITLINEAR_ERR_LAUNCH;
        X = Xq_out;
        x_dtype = BITLINEAR_I8;
        ldx = ldxq;
        beta_in = beta_out;
    }
    const bool x_int8_now = x_dtype == BITLINEAR_I8 || x_dtype == BITLINEAR_I8_TILED;
    if (!x_int8_now && algo == BITLINEAR_ALGO_GEMV_MFMA && bl::gemv_fq_ok(layout, M, N, K, x_dtype, X, ldx)) {
        // 1-4 tokens: the GEMV quantises the activations itself (one launch)
        a.Xq = nullptr;
        a.ldq = 0;
        a.beta = nullptr;
        return status_of(bl::launch_gemv_fq(a, X, x_dtype, ldx, st));
    }
    if (x_int8_now) {
        a.Xq = static_cast<const int8_t *>(X);
        a.ldq = ldx;
        a.beta = beta_in;
        a.tiled = x_dtype == BITLINEAR_I8_TILED;
    } else {
        int8_t *xq = static_cast<int8_t *>(ws);
        float *beta = reinterpret_cast<float *>(static_cast<char *>(ws) + staged_xq_bytes(M, K, layout));
        // The matrix-core GEMV reads tiled activations when a token group has
        // more than a few live rows (with few rows the clamped row-major reads
        // touch few cache lines).
        const bool tiled = algo == BITLINEAR_ALGO_GEMV_MFMA && M > 4 && K <= kTiledMaxK;
        hipError_t e;
        if (tiled) {
            e = bl::launch_quant_act_tiled(X, x_dtype, M, K, ldx, layout, xq, beta, st);
            a.ldq = 0;
        } else {
            a.ldq = staged_ldq(K);
            e = bl::launch_quant_act(X, x_dtype, M, K, ldx, xq, a.ldq, beta, st);
        }
        if (e != hipSuccess) return BITLINEAR_ERR_LAUNCH;
        a.Xq = xq;
        a.beta = beta;
        a.tiled = tiled;
    }
    hipError_t e;
    switch (algo) {
    case BITLINEAR_ALGO_GEMV_ADDSUB: e = bl::launch_gemv_addsub(a, st); break;
    case BITLINEAR_ALGO_GEMV_MFMA: e = bl::launch_gemv_mfma(a, st); break;
    default: e = bl::launch_gemm_mfma(a, st);
        break;
    }
    return status_of(e);
}

int bitlinear_forward_algo(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                           const void *X, int x_dtype, int64_t ldx, const float *beta_in, void *Y, int y_dtype,
                           int64_t ldy, void *ws, int64_t ws_bytes, int algo, void *stream)
{
    return forward_impl(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, ws, ws_bytes, nullptr,
                        0, nullptr, algo, stream);
}

int bitlinear_forward_ex(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                         const void *X, int x_dtype, int64_t ldx, const float *beta_in, void *Y, int y_dtype,
                         int64_t ldy, int8_t *Xq_out, int64_t ldxq, float *beta_out, void *ws, int64_t ws_bytes,
                         int algo, void *stream)
{
    return forward_impl(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, ws, ws_bytes, Xq_out,
                        ldxq, beta_out, algo, stream);
}

// ---- grouped forward --------------------------------------------------------
namespace {

// Whether a job runs inside the grouped launch (else as its own forward).
// The grouped kernel reads a job's packed weights through one buffer range
// with 32-bit byte offsets (and 2^31 as its out-of-range offset), so the
// job's packed bytes must stay below 2^31.
bool group_eligible(const bitlinear_job_t &j, int layout)
{
    const int64_t kblk = layout == BITLINEAR_LAYOUT_I2 ? 64 : (layout == BITLINEAR_LAYOUT_B3 ? 80 : 128);
    const int64_t nsteps = ((j.K + kblk - 1) / kblk + 3) / 4;
    return j.M <= 16 && nsteps <= bl::group_max_nsteps(layout) && j.N <= (int64_t(1) << 30) &&
           bitlinear_packed_bytes(j.N, j.K, layout) <= INT32_MAX;
}

// The distinct inputs of the grouped jobs: jobs with the same X, M, K and ldx
// share one quantisation.  in_of[j]: the input of job j (-1: not grouped).
struct GroupInputs {
    int n = 0;
    int first_job[BITLINEAR_MAX_GROUP];
    int in_of[BITLINEAR_MAX_GROUP];
};

GroupInputs group_inputs(const bitlinear_job_t *jobs, int njobs, int layout)
{
    GroupInputs g;
    for (int j = 0; j < njobs; ++j) {
        g.in_of[j] = -1;
        if (!group_eligible(jobs[j], layout)) continue;
        for (int u = 0; u < g.n; ++u) {
            const bitlinear_job_t &o = jobs[g.first_job[u]];
            if (o.X == jobs[j].X && o.M == jobs[j].M && o.K == jobs[j].K && o.ldx == jobs[j].ldx) g.in_of[j] = u;
        }
        if (g.in_of[j] < 0) {
            g.first_job[g.n] = j;
            g.in_of[j] = g.n++;
        }
    }
    return g;
}

// Whether the grouped launch quantises the activations itself: every grouped
// job has 1 to 4 tokens of 16-byte aligned rows whose bytes a 32-bit buffer
// range covers.
bool group_fused(const bitlinear_job_t *jobs, int njobs, int x_dtype, const GroupInputs &g)
{
    if (g.n == 0) return false;
    const int64_t es = x_dtype == BITLINEAR_F32 ? 4 : 2;
    for (int j = 0; j < njobs; ++j) {
        if (g.in_of[j] < 0) continue;
        const bitlinear_job_t &J = jobs[j];
        if (J.M > 4 || !aligned16(J.X) || (J.ldx * es) % 16 || ((J.M - 1) * J.ldx + J.K) * es + 15 > INT32_MAX)
            return false;
    }
    return true;
}

int64_t group_input_bytes(const bitlinear_job_t &j, int layout)
{
    return round_up(bl::tiled_bytes(j.M, j.K, layout), 256) + round_up(4 * j.M, 256);
}

int64_t grouped_ws_bytes(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype, const GroupInputs &g)
{
    int64_t total = 0, single = 0;
    if (!group_fused(jobs, njobs, x_dtype, g))
        for (int u = 0; u < g.n; ++u) total += group_input_bytes(jobs[g.first_job[u]], layout);
    for (int j = 0; j < njobs; ++j)
        if (g.in_of[j] < 0) {
            const bitlinear_job_t &J = jobs[j];
            const int64_t b = bitlinear_forward_workspace_bytes(J.M, J.N, J.K, layout, x_dtype);
            single = b > single ? b : single;
        }
    return total + round_up(single, 256);
}

// Argument checks of one job (the same as bitlinear_forward's for F32 / BF16
// input), plus: its output overlaps no buffer of any job.
int check_job(const bitlinear_job_t *jobs, int njobs, int j, int layout, int x_dtype, int y_dtype)
{
    const bitlinear_job_t &J = jobs[j];
    if (!J.P || !J.gamma || !J.X || !J.Y) return BITLINEAR_ERR_INVALID_ARG;
    if (J.M < 1 || J.M > BITLINEAR_MAX_M || J.N < 1 || J.N > (int64_t(1) << 31) || J.K < 1 || J.K > BITLINEAR_MAX_K)
        return BITLINEAR_ERR_INVALID_ARG;
    if (J.ldx < J.K || !stride_ok(J.M, J.ldx) || J.ldy < J.N || !stride_ok(J.M, J.ldy))
        return BITLINEAR_ERR_INVALID_ARG;
    if (!aligned16(J.P) || (reinterpret_cast<uintptr_t>(J.gamma) & 3u) ||
        (reinterpret_cast<uintptr_t>(J.X) % dtype_size(x_dtype)) ||
        (reinterpret_cast<uintptr_t>(J.Y) % dtype_size(y_dtype)))
        return BITLINEAR_ERR_INVALID_ARG;
    const Span sy = span_of(J.Y, J.M, J.ldy, J.N, dtype_size(y_dtype));
    for (int o = 0; o < njobs; ++o) {
        const bitlinear_job_t &O = jobs[o];
        if (!O.P || !O.gamma || !O.X || O.M < 1 || O.N < 1 || O.K < 1 || O.ldx < O.K) return BITLINEAR_ERR_INVALID_ARG;
        const int64_t pb = bitlinear_packed_bytes(O.N, O.K, layout);
        if (pb < 0) return BITLINEAR_ERR_INVALID_ARG;
        if (overlap(sy, span_of(O.P, 1, pb, pb, 1)) || overlap(sy, span_of(O.gamma, 1, 1, 1, 4)) ||
            overlap(sy, span_of(O.X, O.M, O.ldx, O.K, dtype_size(x_dtype))))
            return BITLINEAR_ERR_INVALID_ARG;
        if (o != j && O.Y && O.M >= 1 && O.N >= 1 && O.ldy >= O.N &&
            overlap(sy, span_of(O.Y, O.M, O.ldy, O.N, dtype_size(y_dtype))))
            return BITLINEAR_ERR_INVALID_ARG;
    }
    return BITLINEAR_OK;
}

bool group_args_ok(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype, int y_dtype)
{
    return jobs && njobs >= 1 && njobs <= BITLINEAR_MAX_GROUP && valid_layout(layout) &&
           (x_dtype == BITLINEAR_F32 || x_dtype == BITLINEAR_BF16) &&
           (y_dtype == BITLINEAR_F32 || y_dtype == BITLINEAR_BF16 || y_dtype == BITLINEAR_I32);
}

// The device-side description of the grouped jobs and their inputs, carved
// out of the workspace.
void group_build(const bitlinear_job_t *jobs, int njobs, int layout, int y_dtype, const GroupInputs &g, void *ws,
                 bl::GroupQuantArgs &qa, bl::GroupGemvArgs &ga)
{
    // (ws is NULL when the grouped launch quantises inside: no input areas)
    char *p = static_cast<char *>(ws);
    qa.ninputs = g.n;
    qa.layout = layout;
    for (int u = 0; u < g.n; ++u) {
        const bitlinear_job_t &J = jobs[g.first_job[u]];
        bl::GroupInput &in = qa.in[u];
        in.X = J.X;
        in.ldx = J.ldx;
        in.M = static_cast<int>(J.M);
        in.K = static_cast<int>(J.K);
        in.nsteps = static_cast<int>(bl::tiled_nsteps(J.K, layout));
        in.Xt = p ? reinterpret_cast<int8_t *>(p) : nullptr;
        in.beta = p ? reinterpret_cast<float *>(p + round_up(bl::tiled_bytes(J.M, J.K, layout), 256)) : nullptr;
        if (p) p += group_input_bytes(J, layout);
    }
    ga.njobs = 0;
    ga.y_dtype = y_dtype;
    for (int j = 0; j < njobs; ++j) {
        if (g.in_of[j] < 0) continue;
        const bitlinear_job_t &J = jobs[j];
        bl::GroupJob &d = ga.job[ga.njobs++];
        const int64_t kblk = layout == BITLINEAR_LAYOUT_I2 ? 64 : (layout == BITLINEAR_LAYOUT_B3 ? 80 : 128);
        d.P = J.P;
        d.gamma = J.gamma;
        d.Xt = qa.in[g.in_of[j]].Xt;
        d.beta = qa.in[g.in_of[j]].beta;
        d.X = J.X;
        d.ldx = J.ldx;
        d.K = static_cast<int>(J.K);
        d.Y = J.Y;
        d.ldy = J.ldy;
        d.M = static_cast<int>(J.M);
        d.N = static_cast<int>(J.N);
        d.KB = static_cast<int>((J.K + kblk - 1) / kblk);
        d.nsteps = (d.KB + 3) / 4;
        d.wg0 = d.nwg = 0;
    }
}

} // namespace

int64_t bitlinear_forward_grouped_workspace_bytes(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype)
{
    if (!group_args_ok(jobs, njobs, layout, x_dtype, BITLINEAR_F32)) return -1;
    for (int j = 0; j < njobs; ++j)
        if (jobs[j].M < 1 || jobs[j].M > BITLINEAR_MAX_M || jobs[j].N < 1 || jobs[j].K < 1 ||
            jobs[j].K > BITLINEAR_MAX_K)
            return -1;
    return grouped_ws_bytes(jobs, njobs, layout, x_dtype, group_inputs(jobs, njobs, layout));
}

namespace {
// The grouped product's algorithm for these (valid) jobs: 1 = the vector-ALU
// products, 0 = the matrix cores, -1 = the algorithm cannot take them.  The
// vector-ALU products take i2 jobs of one token each; the grouped launch
// quantises their inputs itself, and under BITLINEAR_ALGO_GEMV_ADDSUB the
// jobs it leaves out (rows too long) run on the single-layer add/sub GEMV.
// AUTO takes them for every group of one-token i2 jobs: measured on ten
// layer sets of the 3B and 70B models at one token, they were 0.7-5 % faster
// than the matrix cores in eight (3B q/k/v/o/gate/up 10.08 against 10.61 us,
// the 70B q/k/v/o/gate/up 32.1 against 32.7 us) and level (within 1.5 %) in
// the two that mix the 3B down projection (three k-steps per wave) with
// layers of one (the whole 3B set: 11.38 against 11.34 us).
int group_algo(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype, const GroupInputs &g, int algo)
{
    if (algo == BITLINEAR_ALGO_GEMV_MFMA) return 0;
    if (algo != BITLINEAR_ALGO_AUTO && algo != BITLINEAR_ALGO_GEMV_ADDSUB) return -1;
    const bool forced = algo == BITLINEAR_ALGO_GEMV_ADDSUB;
    bool ok = layout == BITLINEAR_LAYOUT_I2 && (g.n == 0 || group_fused(jobs, njobs, x_dtype, g));
    for (int j = 0; j < njobs && ok; ++j) {
        if (!forced && g.in_of[j] < 0) continue; // AUTO: plain forwards choose for themselves
        if (jobs[j].M != 1) ok = false;
    }
    if (forced) return ok ? 1 : -1;
    return ok && g.n > 0 ? 1 : 0;
}
} // namespace

const char *bitlinear_grouped_kernel_algo(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype, int algo)
{
    thread_local char name[96];
    if (bitlinear_forward_grouped_workspace_bytes(jobs, njobs, layout, x_dtype) < 0) return nullptr;
    const GroupInputs g = group_inputs(jobs, njobs, layout);
    if (g.n == 0) return nullptr;
    const int a = group_algo(jobs, njobs, layout, x_dtype, g, algo);
    if (a < 0) return nullptr;
    bl::group_gemv_kernel_name(layout, group_fused(jobs, njobs, x_dtype, g) ? x_dtype : BITLINEAR_I8, a == 1, name,
                               sizeof name);
    return name;
}

const char *bitlinear_grouped_kernel(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype)
{
    return bitlinear_grouped_kernel_algo(jobs, njobs, layout, x_dtype, BITLINEAR_ALGO_AUTO);
}

int bitlinear_forward_grouped(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype, int y_dtype,
                              void *ws, int64_t ws_bytes, void *stream)
{
    return bitlinear_forward_grouped_algo(jobs, njobs, layout, x_dtype, y_dtype, BITLINEAR_ALGO_AUTO, ws, ws_bytes,
                                          stream);
}

int bitlinear_forward_grouped_algo(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype, int y_dtype,
                                   int algo, void *ws, int64_t ws_bytes, void *stream)
{
    if (!group_args_ok(jobs, njobs, layout, x_dtype, y_dtype)) return BITLINEAR_ERR_INVALID_ARG;
    if (algo < BITLINEAR_ALGO_AUTO || algo > BITLINEAR_ALGO_GEMM_MFMA) return BITLINEAR_ERR_INVALID_ARG;
    for (int j = 0; j < njobs; ++j) {
        const int st = check_job(jobs, njobs, j, layout, x_dtype, y_dtype);
        if (st != BITLINEAR_OK) return st;
    }
    const GroupInputs g = group_inputs(jobs, njobs, layout);
    const int galgo = group_algo(jobs, njobs, layout, x_dtype, g, algo);
    if (galgo < 0) return BITLINEAR_ERR_UNSUPPORTED;
    const int64_t need = grouped_ws_bytes(jobs, njobs, layout, x_dtype, g);
    if (need > 0 && (!ws || ws_bytes < need)) return BITLINEAR_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return BITLINEAR_ERR_INVALID_ARG;
    if (need > 0) {
        const Span sw = span_of(ws, 1, need, need, 1);
        for (int j = 0; j < njobs; ++j) {
            const bitlinear_job_t &J = jobs[j];
            const int64_t pb = bitlinear_packed_bytes(J.N, J.K, layout);
            if (overlap(sw, span_of(J.P, 1, pb, pb, 1)) || overlap(sw, span_of(J.gamma, 1, 1, 1, 4)) ||
                overlap(sw, span_of(J.X, J.M, J.ldx, J.K, dtype_size(x_dtype))) ||
                overlap(sw, span_of(J.Y, J.M, J.ldy, J.N, dtype_size(y_dtype))))
                return BITLINEAR_ERR_INVALID_ARG;
        }
    }
    (void)hipGetLastError();
    hipStream_t st = as_stream(stream);
    int64_t group_bytes = 0;
    if (g.n > 0) {
        bl::GroupQuantArgs qa;
        bl::GroupGemvArgs ga;
        const bool fused = group_fused(jobs, njobs, x_dtype, g);
        group_build(jobs, njobs, layout, y_dtype, g, fused ? nullptr : ws, qa, ga);
        if (!fused) {
            for (int u = 0; u < g.n; ++u) group_bytes += group_input_bytes(jobs[g.first_job[u]], layout);
            if (bl::launch_group_quant(qa, x_dtype, st) != hipSuccess) return BITLINEAR_ERR_LAUNCH;
        }
        const int gemv_x = fused ? x_dtype : BITLINEAR_I8;
        // one product launch, or several when the jobs need more workgroups
        // than one launch maps (each job needs one per GROUP_STAGE_TILES tiles)
        bl::GroupGemvArgs part;
        part.y_dtype = ga.y_dtype;
        part.njobs = 0;
        int need_wgs = 0;
        for (int j = 0; j <= ga.njobs; ++j) {
            const int nwg = j < ga.njobs ? ((ga.job[j].N + 15) / 16 + bl::GROUP_STAGE_TILES - 1) / bl::GROUP_STAGE_TILES : 0;
            if (part.njobs > 0 && (j == ga.njobs || need_wgs + nwg > bl::GROUP_MAX_WGS / 2 - 16)) {
                const bl::GroupPlan plan = bl::group_plan(part, layout);
                if (bl::launch_group_gemv(part, plan, layout, gemv_x, st, galgo == 1) != hipSuccess)
                    return BITLINEAR_ERR_LAUNCH;
                part.njobs = 0;
                need_wgs = 0;
            }
            if (j < ga.njobs) {
                part.job[part.njobs++] = ga.job[j];
                need_wgs += nwg;
            }
        }
    }
    // the jobs the grouped launch does not take, one forward each (their
    // workspace follows the grouped inputs'; they run one after another)
    void *rest = static_cast<char *>(ws) + group_bytes;
    for (int j = 0; j < njobs; ++j) {
        if (g.in_of[j] >= 0) continue;
        const bitlinear_job_t &J = jobs[j];
        const int64_t nb = bitlinear_forward_workspace_bytes(J.M, J.N, J.K, layout, x_dtype);
        const int s = forward_impl(J.P, layout, J.gamma, J.M, J.N, J.K, J.X, x_dtype, J.ldx, nullptr, J.Y, y_dtype,
                                   J.ldy, nb > 0 ? rest : nullptr, nb, nullptr, 0, nullptr,
                                   algo == BITLINEAR_ALGO_GEMV_ADDSUB ? BITLINEAR_ALGO_GEMV_ADDSUB
                                                                      : BITLINEAR_ALGO_AUTO,
                                   stream);
        if (s != BITLINEAR_OK) return s;
    }
    return BITLINEAR_OK;
}

// ---- allocation-free forward ------------------------------------------------
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];

// The device address of 'scratch' on the current device, looked up once per
// device (each GPU holds its own copy of the array at its own address).
void *scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
    return p;
}

} // namespace

int bitlinear_forward_noalloc(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                              const void *X, int x_dtype, int64_t ldx, const float *beta_in, void *Y, int y_dtype,
                              int64_t ldy, void *stream)
{
    const int64_t need = bitlinear_forward_workspace_bytes(M, N, K, layout, x_dtype);
    if (need < 0) return BITLINEAR_ERR_INVALID_ARG;
    // every argument check first (on the host; nothing is enqueued)
    const int st = forward_impl(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, nullptr, 0,
                                nullptr, 0, nullptr, BITLINEAR_ALGO_AUTO, stream, true);
    if (st != BITLINEAR_OK) return st;
    if (need > int64_t(BITLINEAR_NOALLOC_SCRATCH_BYTES)) return BITLINEAR_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        ws = scratch_ptr();
        if (!ws) return BITLINEAR_ERR_DEVICE;
    }
    return forward_impl(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, ws, need, nullptr, 0,
                        nullptr, BITLINEAR_ALGO_AUTO, stream);
}

int64_t bitlinear_forward_chain_parts(int64_t M, int64_t N, int64_t K, int layout)
{
    if (M < 1 || M > 16 || N < 1 || N > (int64_t(1) << 31) || K < 1 || K > kTiledMaxK || !valid_layout(layout))
        return -1;
    return bl::gemv_mfma_parts(layout, M, N, K);
}

int bitlinear_forward_chain(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                            const void *X, int x_dtype, int64_t ldx, const float *pmax_in, int64_t nparts_in,
                            void *Y, int y_dtype, int64_t ldy, float *pmax_out, int64_t pmax_cols, void *ws,
                            int64_t ws_bytes, void *stream)
{
    if (x_dtype != BITLINEAR_F32 && x_dtype != BITLINEAR_BF16) return BITLINEAR_ERR_INVALID_ARG;
    // every check of the plain forward (workspace alignment and overlaps included)
    const int st0 = forward_impl(P, layout, gamma, M, N, K, X, x_dtype, ldx, nullptr, Y, y_dtype, ldy, ws, ws_bytes,
                                 nullptr, 0, nullptr, BITLINEAR_ALGO_GEMV_MFMA, stream, true);
    if (st0 != BITLINEAR_OK) return st0;
    if (M > 16 || K > kTiledMaxK) return BITLINEAR_ERR_UNSUPPORTED;
    const int64_t need = bitlinear_forward_workspace_bytes(M, N, K, layout, x_dtype);
    if (!ws || ws_bytes < need) return BITLINEAR_ERR_WORKSPACE;
    if ((pmax_in != nullptr) != (nparts_in > 0) || nparts_in < 0 || (reinterpret_cast<uintptr_t>(pmax_in) & 3u))
        return BITLINEAR_ERR_INVALID_ARG;
    const int64_t parts = bl::gemv_mfma_parts(layout, M, N, K);
    const Span sy = span_of(Y, M, ldy, N, dtype_size(y_dtype)), sw = span_of(ws, 1, need, need, 1);
    if (pmax_in) {
        const Span si = span_of(pmax_in, 1, nparts_in * 16, nparts_in * 16, 4);
        if (overlap(si, sy) || overlap(si, sw)) return BITLINEAR_ERR_INVALID_ARG;
    }
    if (pmax_out) {
        if (y_dtype == BITLINEAR_I32 || pmax_cols < 1 || pmax_cols > N || (reinterpret_cast<uintptr_t>(pmax_out) & 3u))
            return BITLINEAR_ERR_INVALID_ARG;
        const int64_t pb = bitlinear_packed_bytes(N, K, layout);
        const Span so = span_of(pmax_out, 1, parts * 16, parts * 16, 4);
        const Span others[] = {sy, sw, span_of(P, 1, pb, pb, 1), span_of(X, M, ldx, K, dtype_size(x_dtype)),
                               span_of(gamma, 1, 1, 1, 4)};
        for (const Span &o : others)
            if (overlap(so, o)) return BITLINEAR_ERR_INVALID_ARG;
        if (pmax_in && overlap(so, span_of(pmax_in, 1, nparts_in * 16, nparts_in * 16, 4)))
            return BITLINEAR_ERR_INVALID_ARG;
    } else if (pmax_cols != 0) {
        return BITLINEAR_ERR_INVALID_ARG;
    }
    (void)hipGetLastError();
    hipStream_t st = as_stream(stream);
    int8_t *xq = static_cast<int8_t *>(ws);
    float *beta = reinterpret_cast<float *>(static_cast<char *>(ws) + staged_xq_bytes(M, K, layout));
    hipError_t e = bl::launch_quant_act_tiled(X, x_dtype, M, K, ldx, layout, xq, beta, st, pmax_in, nparts_in);
    if (e != hipSuccess) return BITLINEAR_ERR_LAUNCH;
    bl::GemvArgs a;
    a.P = P;
    a.layout = layout;
    a.gamma = gamma;
    a.M = M;
    a.N = N;
    a.K = K;
    a.Xq = xq;
    a.ldq = 0;
    a.tiled = true;
    a.beta = beta;
    a.Y = Y;
    a.y_dtype = y_dtype;
    a.ldy = ldy;
    a.pmax = pmax_out;
    a.pmax_cols = pmax_out ? pmax_cols : 0;
    return status_of(bl::launch_gemv_mfma(a, st));
}

// i2 rewrite of b3 / b1 weights, then the small-batch dX's partial tiles
static int64_t bwd_dx_rewrite_bytes(int64_t N, int64_t K, int layout)
{
    return layout == BITLINEAR_LAYOUT_I2 ? 0 : round_up(bitlinear_packed_bytes(N, K, BITLINEAR_LAYOUT_I2), 256);
}

int64_t bitlinear_backward_dx_workspace_bytes(int64_t M, int64_t N, int64_t K, int layout)
{
    if (M < 1 || M > BITLINEAR_MAX_M || bitlinear_packed_bytes(N, K, layout) < 0 || N > kMaxElems / K) return -1;
    return bwd_dx_rewrite_bytes(N, K, layout) + bl::bwd_dx_partial_bytes(M, N, K);
}

int bitlinear_backward_dx(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                          const float *dY, int64_t lddy, float *dX, int64_t lddx, void *ws, int64_t ws_bytes,
                          void *stream)
{
    if (!P || !gamma || !dY || !dX || !valid_layout(layout)) return BITLINEAR_ERR_INVALID_ARG;
    if (M < 1 || M > BITLINEAR_MAX_M || N < 1 || K < 1 || K > BITLINEAR_MAX_K || N > kMaxElems / K ||
        lddy < N || lddx < K || !stride_ok(M, lddy) || !stride_ok(M, lddx))
        return BITLINEAR_ERR_INVALID_ARG;
    const int64_t need = bitlinear_backward_dx_workspace_bytes(M, N, K, layout);
    if (need > 0 && (!ws || ws_bytes < need)) return BITLINEAR_ERR_WORKSPACE;
    if (!aligned16(P) || (need > 0 && !aligned16(ws)) || (reinterpret_cast<uintptr_t>(dY) & 3u) ||
        (reinterpret_cast<uintptr_t>(dX) & 3u) || (reinterpret_cast<uintptr_t>(gamma) & 3u))
        return BITLINEAR_ERR_INVALID_ARG;
    const int64_t pb = bitlinear_packed_bytes(N, K, layout);
    const Span sx = span_of(dX, M, lddx, K, 4), sy = span_of(dY, M, lddy, N, 4), sp = span_of(P, 1, pb, pb, 1),
               sg = span_of(gamma, 1, 1, 1, 4);
    if (overlap(sx, sy) || overlap(sx, sp) || overlap(sx, sg)) return BITLINEAR_ERR_INVALID_ARG;
    if (need > 0) {
        const Span sw = span_of(ws, 1, need, need, 1);
        if (overlap(sw, sx) || overlap(sw, sy) || overlap(sw, sp) || overlap(sw, sg)) return BITLINEAR_ERR_INVALID_ARG;
    }
    (void)hipGetLastError();
    hipStream_t st = as_stream(stream);
    const uint8_t *p2 = P;
    if (layout != BITLINEAR_LAYOUT_I2) {
        uint8_t *w2 = static_cast<uint8_t *>(ws);
        const hipError_t e = layout == BITLINEAR_LAYOUT_B3 ? bl::launch_b3_to_i2(P, N, K, w2, st)
                                                           : bl::launch_b1_to_i2(P, N, K, w2, st);
        if (e != hipSuccess) return BITLINEAR_ERR_LAUNCH;
        p2 = w2;
    }
    float *part = need > 0 ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + bwd_dx_rewrite_bytes(N, K, layout))
                           : nullptr;
    return status_of(bl::launch_bwd_dx(p2, gamma, M, N, K, dY, lddy, dX, lddx, part, st));
}

const char *bitlinear_backward_kernel(int64_t M, int64_t N, int64_t K, int which)
{
    if (M < 1 || M > BITLINEAR_MAX_M || N < 1 || K < 1 || K > BITLINEAR_MAX_K || N > kMaxElems / K ||
        (which != 0 && which != 1))
        return nullptr;
    return bl::bwd_kernel_name(which == 0, M, K);
}

int bitlinear_backward_dw(const int8_t *Xq, int64_t ldq, const float *beta, int64_t M, int64_t N, int64_t K,
                          const float *dY, int64_t lddy, float *dW, int64_t lddw, void *stream)
{
    if (!Xq || !beta || !dY || !dW) return BITLINEAR_ERR_INVALID_ARG;
    if (M < 1 || M > BITLINEAR_MAX_M || N < 1 || K < 1 || K > BITLINEAR_MAX_K || N > kMaxElems / K || ldq < K ||
        lddy < N || lddw < K || !stride_ok(M, ldq) || !stride_ok(M, lddy) || !stride_ok(N, lddw))
        return BITLINEAR_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(dY) & 3u) || (reinterpret_cast<uintptr_t>(dW) & 3u) ||
        (reinterpret_cast<uintptr_t>(beta) & 3u))
        return BITLINEAR_ERR_INVALID_ARG;
    const Span sw = span_of(dW, N, lddw, K, 4), sq = span_of(Xq, M, ldq, K, 1), sb = span_of(beta, 1, M, M, 4),
               sy = span_of(dY, M, lddy, N, 4);
    if (overlap(sw, sq) || overlap(sw, sb) || overlap(sw, sy)) return BITLINEAR_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return status_of(bl::launch_bwd_dw(Xq, ldq, beta, M, N, K, dY, lddy, dW, lddw, as_stream(stream)));
}

int bitlinear_forward(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                      const void *X, int x_dtype, int64_t ldx, const float *beta_in, void *Y, int y_dtype,
                      int64_t ldy, void *ws, int64_t ws_bytes, void *stream)
{
    return bitlinear_forward_algo(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, ws,
                                  ws_bytes, BITLINEAR_ALGO_AUTO, stream);
}

} // extern "C"
