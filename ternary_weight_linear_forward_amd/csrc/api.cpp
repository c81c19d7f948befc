// api.cpp -- the C ABI of libbitlinear (declared in include/bitlinear.h).
// Validates every argument on the host, then enqueues the kernels.  Nothing is
// launched when validation fails.  No allocation, no synchronisation, no
// mutable global state.
#include "bitlinear.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40; // keeps per-exponent sums of |W| below 2^64
// Largest M the add/subtract GEMV takes when the kernel is chosen
// automatically.  Measured on MI355X the matrix-core GEMV is faster at every M
// (the vector ALU reaches 4 int8 MACs per lane-cycle, the matrix core takes the
// MACs off it), so automatic dispatch never picks add/subtract; it stays
// available as BITLINEAR_ALGO_GEMV_ADDSUB.
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
// input), then, with more than 16 tokens and weights the GEMM rewrites as i2
// (gemm_rewrites), room for that rewrite.
int64_t staging_bytes(int64_t M, int64_t K, int layout, int x_dtype)
{
    if (x_dtype == BITLINEAR_I8 || x_dtype == BITLINEAR_I8_TILED) return 0;
    return staged_xq_bytes(M, K, layout) + round_up(4 * M, 256);
}
// The GEMM reads i2 weights or decodes b3 itself; b1 weights, and b3 weights
// of shapes where the decode would repeat over many token blocks, are
// rewritten as i2 first.
bool gemm_rewrites(int64_t M, int64_t N, int layout)
{
    return layout == BITLINEAR_LAYOUT_B1 || (layout == BITLINEAR_LAYOUT_B3 && !bl::gemm_b3_native(M, N));
}
int64_t transcode_bytes(int64_t M, int64_t N, int64_t K, int layout)
{
    return M > 16 && gemm_rewrites(M, N, layout) ? round_up(bitlinear_packed_bytes(N, K, BITLINEAR_LAYOUT_I2), 256)
                                                 : 0;
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
    return staging_bytes(M, K, layout, x_dtype) + transcode_bytes(M, N, K, layout);
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
        (algo == BITLINEAR_ALGO_GEMM_MFMA && layout == BITLINEAR_LAYOUT_B1 && M <= 16) ||
        (x_dtype == BITLINEAR_I8_TILED && algo != BITLINEAR_ALGO_GEMV_MFMA))
        return nullptr;
    if (algo == BITLINEAR_ALGO_GEMV_ADDSUB) {
        bl::gemv_addsub_kernel_name(M, name, sizeof name);
    } else if (algo == BITLINEAR_ALGO_GEMM_MFMA) {
        bl::gemm_kernel_name(gemm_rewrites(M, N, layout) ? BITLINEAR_LAYOUT_I2 : layout, M, N, name, sizeof name);
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

int bitlinear_forward_algo(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                           const void *X, int x_dtype, int64_t ldx, const float *beta_in, void *Y, int y_dtype,
                           int64_t ldy, void *ws, int64_t ws_bytes, int algo, void *stream)
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
    if (!aligned16(P) || (reinterpret_cast<uintptr_t>(gamma) & 3u) ||
        (reinterpret_cast<uintptr_t>(X) % dtype_size(x_dtype)) ||
        (reinterpret_cast<uintptr_t>(Y) % dtype_size(y_dtype)))
        return BITLINEAR_ERR_INVALID_ARG;
    if (x_dtype == BITLINEAR_I8 && (!aligned16(X) || ldx % 16 || (reinterpret_cast<uintptr_t>(beta_in) & 3u)))
        return BITLINEAR_ERR_INVALID_ARG;
    if (x_dtype == BITLINEAR_I8_TILED && (!aligned16(X) || (reinterpret_cast<uintptr_t>(beta_in) & 3u)))
        return BITLINEAR_ERR_INVALID_ARG;

    const int64_t need = bitlinear_forward_workspace_bytes(M, N, K, layout, x_dtype);
    if (need > 0 && (!ws || ws_bytes < need)) return BITLINEAR_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return BITLINEAR_ERR_INVALID_ARG;

    const int64_t pb = bitlinear_packed_bytes(N, K, layout);
    const int64_t xt = bl::tiled_bytes(M, K, layout);
    const Span sp = span_of(P, 1, pb, pb, 1),
               sx = x_dtype == BITLINEAR_I8_TILED ? span_of(X, 1, xt, xt, 1) : span_of(X, M, ldx, K, dtype_size(x_dtype)),
               sy = span_of(Y, M, ldy, N, dtype_size(y_dtype)), sg = span_of(gamma, 1, 1, 1, 4);
    if (overlap(sy, sp) || overlap(sy, sx) || overlap(sy, sg)) return BITLINEAR_ERR_INVALID_ARG;
    if (beta_in && overlap(sy, span_of(beta_in, 1, M, M, 4))) return BITLINEAR_ERR_INVALID_ARG;
    if (need > 0) {
        const Span sw = span_of(ws, 1, need, need, 1);
        if (overlap(sw, sp) || overlap(sw, sx) || overlap(sw, sy) || overlap(sw, sg))
            return BITLINEAR_ERR_INVALID_ARG;
    }

    if (algo == BITLINEAR_ALGO_AUTO) algo = auto_algo(M, N, layout, x_dtype);
    if (algo == BITLINEAR_ALGO_GEMV_ADDSUB && (M > 16 || layout != BITLINEAR_LAYOUT_I2))
        return BITLINEAR_ERR_UNSUPPORTED;
    if (algo == BITLINEAR_ALGO_GEMM_MFMA && layout == BITLINEAR_LAYOUT_B1 && M <= 16) return BITLINEAR_ERR_UNSUPPORTED;
    if (x_dtype == BITLINEAR_I8_TILED && algo != BITLINEAR_ALGO_GEMV_MFMA) return BITLINEAR_ERR_UNSUPPORTED;

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
    if (!x_int8 && algo == BITLINEAR_ALGO_GEMV_MFMA && bl::gemv_fq_ok(layout, M, N, K, x_dtype, X, ldx)) {
        // 1-4 tokens: the GEMV quantises the activations itself (one launch)
        a.Xq = nullptr;
        a.ldq = 0;
        a.beta = nullptr;
        return status_of(bl::launch_gemv_fq(a, X, x_dtype, ldx, st));
    }
    if (x_int8) {
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
    default:
        if (gemm_rewrites(M, N, layout)) {
            // rewrite the weights as i2 into the workspace first
            uint8_t *p2 = static_cast<uint8_t *>(ws) + staging_bytes(M, K, layout, x_dtype);
            e = layout == BITLINEAR_LAYOUT_B3 ? bl::launch_b3_to_i2(P, N, K, p2, st) : bl::launch_b1_to_i2(P, N, K, p2, st);
            if (e != hipSuccess) return BITLINEAR_ERR_LAUNCH;
            a.P = p2;
            a.layout = BITLINEAR_LAYOUT_I2;
        }
        e = bl::launch_gemm_mfma(a, st);
        break;
    }
    return status_of(e);
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
