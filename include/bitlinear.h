/*
 * bitlinear.h -- C ABI of libbitlinear, the BitLinear forward pass of
 * BitNet b1.58 on AMD Instinct MI355X (gfx950).
 *
 * Method (what the sources say):
 *   - "The Era of 1-bit LLMs: All Large Language Models are in 1.58 Bits",
 *     Abstract: every weight of a BitNet b1.58 model is ternary, {-1, 0, +1}.
 *   - LIT-380 record (dmarx anthology), Key takeaways, bullet 1: BitLinear is
 *     the drop-in replacement of nn.Linear; weights go to {-1, 0, +1} through
 *     an absmean quantisation function; activations are 8-bit integers.
 *   - LIT-380, Key takeaways, bullet 4: the matrix product becomes integer
 *     additions and subtractions, with no multiplications.
 *   - HackerPapers digest, thread "GPUs Go Brrr": 1.58 bits are 2 bits in
 *     practice; thread "How to pack ternary numbers in 8-bit bytes": five
 *     ternary digits fit one byte.
 * The pages give no formulas; this library fixes the plainest reading:
 *   gamma   = mean |W| over the whole tensor, exact, rounded once to binary32;
 *   T       = clamp(rint(W / gamma), -1, +1), IEEE division, ties to even;
 *   beta_m  = max_k |x_mk| (per token);
 *   q_mk    = clamp(rint(x_mk * (127 / beta_m)), -127, 127), ties to even,
 *             in binary32 at the power-of-two scale of the row where beta_m
 *             lies in [1, 2) (one rounded division 127 / b per token, one
 *             rounded product per element), so a row and its 2^k multiple
 *             give the same q, tiny rows included;
 *   acc_mn  = sum_k q_mk * T_nk, exact in int32;
 *   y_mn    = float(acc_mn) * ((gamma * beta_m) / 127), binary32.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major.  W and T are [N x K] (out x in, like
 *     nn.Linear.weight), X and Xq are [M x K], Y is [M x N].  "ld*" arguments
 *     are row strides in elements, at most 2^40, with (rows - 1) * ld at most
 *     2^44 (larger strides are rejected as invalid arguments).
 *   - All array pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; it keeps no mutable global state.
 *   - 'stream' is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns before the work finishes.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     returned as a status; nothing is launched in that case.  A failed launch
 *     returns BITLINEAR_ERR_LAUNCH.  The library never prints.
 *   - Non-finite floating-point inputs are outside the contract.
 *   - K <= BITLINEAR_MAX_K keeps |acc| < 2^24, so float(acc) is exact.
 *   - Pointers read with 128-bit loads (P, Xq, ws) must be 16-byte aligned.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_MAX_K 131072
#define BITLINEAR_MAX_M 65536

typedef enum {
    BITLINEAR_OK = 0,
    BITLINEAR_ERR_INVALID_ARG = 1, /* null pointer, bad size, stride, enum or alignment */
    BITLINEAR_ERR_UNSUPPORTED = 2, /* valid request this library does not implement     */
    BITLINEAR_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required        */
    BITLINEAR_ERR_LAUNCH = 4,      /* a kernel launch failed                            */
    BITLINEAR_ERR_DEVICE = 5,      /* no usable gfx950 device on the current HIP device  */
    BITLINEAR_ERR_SCRATCH = 6      /* bitlinear_forward_noalloc: needs more than its scratch */
} bitlinear_status_t;

typedef enum {
    BITLINEAR_F32 = 0,
    BITLINEAR_BF16 = 1,
    BITLINEAR_I8 = 2,      /* int8, row-major                                       */
    BITLINEAR_I32 = 3,
    BITLINEAR_I8_TILED = 4 /* int8 in the tiled activation layout (see below)      */
} bitlinear_dtype_t;

typedef enum {
    BITLINEAR_LAYOUT_I2 = 0, /* 2 bits per weight                     */
    BITLINEAR_LAYOUT_B3 = 1, /* base 3, 5 weights per byte            */
    BITLINEAR_LAYOUT_B1 = 2  /* 1 bit per weight, binary weights only */
} bitlinear_layout_t;

typedef enum {
    BITLINEAR_ALGO_AUTO = 0,        /* pick by M and layout                                 */
    BITLINEAR_ALGO_GEMV_ADDSUB = 1, /* vector-ALU add/subtract GEMV, M <= 16                */
    BITLINEAR_ALGO_GEMV_MFMA = 2,   /* 16-token int8 matrix-core tiles, any M (token groups) */
    BITLINEAR_ALGO_GEMM_MFMA = 3    /* LDS-tiled int8 matrix-core GEMM: i2 and b3 any M, b1 M > 16 */
} bitlinear_algo_t;

/* Static description of a status code (never NULL). */
const char *bitlinear_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int bitlinear_version(void);

/*
 * Packed layouts (this library's convention; the pages fix none).
 * I2 and B3 store code c = T + 1 in {0, 1, 2} and pad with T = 0 (rows up to a
 * multiple of 16, columns up to a whole k-block).  Rows are grouped in tiles
 * of 16.  Inside a tile, 16-byte chunks are ordered by k-block, then by row:
 * the chunk of row n and k-block kb starts at byte
 *     ((n / 16) * KB + kb) * 256 + (n % 16) * 16.
 *   I2: a k-block is 64 weights, KB = ceil(K / 64).  Little-endian 32-bit word
 *       d (0..3) of a chunk holds weights kb*64 + 16d + 4s + j (s, j in 0..3)
 *       at bits 8j+2s .. 8j+2s+1, so (word >> 2s) & 0x03030303 gives the
 *       codes of 4 consecutive weights, one per byte.
 *   B3: a k-block is 80 weights, KB = ceil(K / 80).  Byte i (0..15) of a chunk
 *       holds weights kb*80 + 16t + i (t = 0..4): with v = sum_t c_t * 3^(4-t)
 *       (t = 0 most significant), the byte is ceil(256 * v / 243), v / 243 as
 *       an 8-bit fraction rounded up (v = floor(243 * byte / 256)), so that
 *       digit t is floor(byte * 3^(t+1) / 256) - 3 * floor(byte * 3^t / 256).
 *       Base-3 digit t of the 16 bytes covers 16 consecutive weights; 13 of
 *       the 256 byte values never occur.  Padding (T = 0) is the byte 128.
 *   B1: binary weights T in {-1, +1} only.  A k-block is 128 weights,
 *       KB = ceil(K / 128).  Word d (0..3) of a chunk holds weights
 *       kb*128 + 32d + 4s + j (s in 0..7, j in 0..3) at bit 8j+s: 1 for +1,
 *       0 for -1.  Padding bits are 0 (a weight of -1 that the product meets
 *       with zero activations).
 * Returns the byte size of P, or -1 if N, K or layout is invalid.
 */
int64_t bitlinear_packed_bytes(int64_t N, int64_t K, int layout);

/* Workspace bytes bitlinear_quantize_weights needs (-1 if N or K is invalid). */
int64_t bitlinear_quantize_weights_workspace_bytes(int64_t N, int64_t K);

/*
 * Workspace bytes bitlinear_forward needs for these sizes (-1 if invalid).
 * Covers the staged int8 activations and beta of the fused quantiser (x_dtype
 * F32 or BF16); 0 for pre-quantised input.  Weights are read in their own
 * layout and never rewritten.
 */
int64_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K, int layout, int x_dtype);

/*
 * The product algorithm bitlinear_forward (algo AUTO) runs for these sizes:
 * BITLINEAR_ALGO_GEMV_MFMA for pre-tiled input, for M <= 16, and for larger
 * M when the GEMM would launch too few workgroup tiles to fill the GPU;
 * BITLINEAR_ALGO_GEMM_MFMA otherwise (it decodes b3 and b1 weights itself).
 * Returns -1 for invalid
 * sizes, layout or dtype.  Host-only; enqueues nothing.
 */
int bitlinear_auto_algo(int64_t M, int64_t N, int64_t K, int layout, int x_dtype);

/*
 * Name of the product kernel a forward with these arguments launches (algo
 * AUTO resolved as above), as profilers print it without the argument list,
 * e.g. "bl::k_gemv_persist<0, 1, 8, true>"; NULL for invalid or unsupported
 * arguments.  For 1 to 4 tokens of F32 / BF16 input it names the GEMV that
 * quantises the activations itself ("bl::k_gemv_fq<...>" or
 * "bl::k_gemv_persist_fq<...>"), which a forward runs when X and its rows
 * are 16-byte aligned (otherwise: the quantiser, then the int8 GEMV).  The
 * string lives in thread-local storage until the calling thread's next call.
 * Host-only; enqueues nothing.
 */
const char *bitlinear_product_kernel(int64_t M, int64_t N, int64_t K, int layout, int x_dtype, int algo);

/*
 * Absmean weight ternarisation (LIT-380 Key takeaways bullet 1).
 *   W      fp32 [N x K], row stride ldw >= K (device, read-only).
 *   T      int8 [N x K], row stride K (device, written): values in {-1, 0, +1}.
 *   gamma  1 fp32 (device, written): the exact mean of |W| rounded once to
 *          binary32, ties to even.  The sum is exact and order-independent.
 *   ws     >= bitlinear_quantize_weights_workspace_bytes(N, K) bytes, 16-byte
 *          aligned; contents on entry are ignored.
 * Requires N * K < 2^40.  gamma == 0 (all-zero W) gives T = 0.
 */
int bitlinear_quantize_weights(const float *W, int64_t N, int64_t K, int64_t ldw, int8_t *T,
                               float *gamma, void *ws, int64_t ws_bytes, void *stream);

/*
 * Binary weights of the original BitNet, the predecessor the 1.58-bit method
 * extends with a zero state (LIT-380 Key takeaways bullet 2; HackerPapers
 * digest).  Arguments, workspace and gamma as bitlinear_quantize_weights;
 * T[n][k] = +1 where W[n][k] >= 0 (also -0), else -1.  Pack T with
 * BITLINEAR_LAYOUT_B1 (or I2 / B3, which hold any ternary values).
 */
int bitlinear_binarize_weights(const float *W, int64_t N, int64_t K, int64_t ldw, int8_t *T,
                               float *gamma, void *ws, int64_t ws_bytes, void *stream);

/*
 * Packing of the ternary weights: 1.58 bits of information per weight, stored
 * as 2 bits in practice (HackerPapers digest, thread "GPUs Go Brrr") or five
 * ternary digits to a byte (thread "How to pack ternary numbers in 8-bit
 * bytes"); the layouts are this library's convention (see above).
 * Pack ternary weights T int8 [N x K] (row stride ldt >= K, values in
 * {-1, 0, +1}) into P (bitlinear_packed_bytes(N, K, layout) bytes, 16-byte
 * aligned).  Every byte of P is written, padding included.  Values of T
 * outside {-1, 0, +1} are outside the contract, and so is T = 0 for
 * BITLINEAR_LAYOUT_B1 (it is packed as -1).
 */
int bitlinear_pack(const int8_t *T, int64_t N, int64_t K, int64_t ldt, int layout, uint8_t *P,
                   void *stream);

/*
 * Load-time rewrite of packed weights as i2 (a format change of the same
 * ternary values; the 2-bit form is the one the HackerPapers digest's thread
 * "GPUs Go Brrr" stores).  No forward rewrites weights: the products read b3
 * and b1 bytes themselves, and a caller that keeps a b3 / b1 layer mainly for
 * many-token products, where the base-3 digit decode costs more than the i2
 * unpack, can call this once when it loads the layer and pass the i2 copy
 * (layout I2) to those forwards instead.
 *   P     packed [N x K] in layout B3 or B1 (device, read-only, 16-byte aligned).
 *   P2    bitlinear_packed_bytes(N, K, I2) bytes (device, written, 16-byte
 *         aligned, not overlapping P): every byte, padding included, equals
 *         what bitlinear_pack writes for the same T with layout I2.
 * Returns INVALID_ARG for a null or misaligned pointer, layout I2 or an
 * unknown layout, N < 1, K out of [1, BITLINEAR_MAX_K], N * K >= 2^40, or
 * overlapping buffers; LAUNCH if the launch fails.  Enqueued on stream.
 */
int bitlinear_transcode_i2(const uint8_t *P, int layout, int64_t N, int64_t K, uint8_t *P2, void *stream);

/*
 * Per-token absmax int8 activation quantisation (LIT-380 Key takeaways
 * bullet 1: 8-bit activations).
 *   X      [M x K], x_dtype F32 or BF16, row stride ldx >= K.
 *   Xq     int8 [M x K], row stride ldq >= K, 16-byte aligned, ldq % 16 == 0.
 *          Bytes K .. ldq-1 of every row are written with 0.
 *   beta   fp32 [M]: beta_m = max_k |x_mk|; a zero row gives beta = 0, q = 0.
 */
int bitlinear_quantize_act(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t *Xq,
                           int64_t ldq, float *beta, void *stream);

/*
 * Tiled activation layout (this library's convention): the int8 activations
 * as the operands of the matrix-core product, 1 KiB per operand.  With
 * S = 256 weights per k-step for I2 (320 for B3, 512 for B1), F = 4 operands
 * per k-step for I2 (5 for B3, 8 for B1), nsteps = ceil(K / S) and
 * G = ceil(M / 16) token groups,
 * q[m][k] with m = 16*tg + i, k = s*S + g*(S/4) + 16*d + e (g in 0..3,
 * d in 0..F-1, e in 0..15) is stored at byte
 *     (((tg * nsteps + s) * F + d) * 64 + g * 16 + i) * 16 + e
 * and every byte outside [0, M) x [0, K) is 0.  Size: G * nsteps * F * 1024.
 * Returns that size, or -1 if an argument is invalid.
 */
int64_t bitlinear_act_tiled_bytes(int64_t M, int64_t K, int layout);

/*
 * Per-token absmax int8 quantisation (as bitlinear_quantize_act) written in
 * the tiled activation layout for 'layout'.
 *   Xt     bitlinear_act_tiled_bytes(M, K, layout) bytes, 16-byte aligned;
 *          every byte is written (padding with 0).
 *   beta   fp32 [M].
 * Quantising once and passing Xt to several forwards (x_dtype I8_TILED) lets
 * BitLinears that share an input (q, k and v, or gate and up) skip the
 * quantiser.
 */
int bitlinear_quantize_act_tiled(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int layout,
                                 int8_t *Xt, int64_t xt_bytes, float *beta, void *stream);

/*
 * BitLinear forward, the drop-in replacement of nn.Linear (LIT-380 record, Key
 * takeaways, bullet 1: ternary weights from the absmean function, 8-bit
 * activations), whose product is integer additions and subtractions only
 * (bullet 4), computed exactly in int32 and rescaled by gamma * beta_m / 127:
 * Y = rescale(quant(X) (x) T^T), T given packed in P.
 *   P        packed weights of T [N x K] in 'layout' (16-byte aligned).
 *   gamma    1 fp32 (device): the weight scale returned by quantize_weights.
 *   X        x_dtype F32 or BF16: quantised per token inside the call.  For
 *            1 to 4 tokens on GEMV shapes, with X and ldx * element size
 *            16-byte aligned, the GEMV quantises the rows itself (one
 *            launch, ws untouched); otherwise the quantiser runs first and
 *            its int8 output is staged in ws.  x_dtype I8: X is already quantised (16-byte aligned,
 *            ldx % 16 == 0, M rows of ldx bytes readable) and beta_in (fp32
 *            [M], device) gives beta.  x_dtype I8_TILED: X is
 *            bitlinear_act_tiled_bytes(M, K, layout) bytes in the tiled
 *            activation layout of the same 'layout' (ldx is ignored) and
 *            beta_in gives beta; only the matrix-core GEMV takes it.
 *   beta_in  required iff x_dtype is I8 or I8_TILED, else must be NULL.
 *   Y        [M x N], y_dtype F32, BF16 (round to nearest even), or I32 (the
 *            exact accumulators acc, no rescale); row stride ldy >= N.
 *   ws       >= bitlinear_forward_workspace_bytes(M, N, K, layout, x_dtype)
 *            bytes, 16-byte aligned (may be NULL when that size is 0).
 * The accumulators are exact; Y in F32 is bit-identical to the binary32
 * formula above.  Calls that share a workspace must be ordered on one stream.
 */
int bitlinear_forward(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                      const void *X, int x_dtype, int64_t ldx, const float *beta_in, void *Y, int y_dtype,
                      int64_t ldy, void *ws, int64_t ws_bytes, void *stream);

/* Same as bitlinear_forward with an explicit kernel choice (bitlinear_algo_t);
 * returns BITLINEAR_ERR_UNSUPPORTED if that kernel cannot take these sizes
 * (among them: BITLINEAR_ALGO_GEMM_MFMA on int8 rows whose stride makes the
 * rows of one 256-token tile span 2^31 bytes or more; AUTO takes the GEMV
 * there). */
int bitlinear_forward_algo(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N,
                           int64_t K, const void *X, int x_dtype, int64_t ldx, const float *beta_in,
                           void *Y, int y_dtype, int64_t ldy, void *ws, int64_t ws_bytes, int algo,
                           void *stream);

/*
 * bitlinear_forward_algo that also returns the quantiser's outputs, for a
 * backward pass that needs them (bitlinear_backward_dw takes Xq and beta).
 *   Xq_out   int8 [M x K] (device, written), row stride ldxq >= K with
 *            ldxq % 16 == 0, 16-byte aligned; bytes K .. ldxq-1 of each row
 *            are written with 0.  NULL: not requested.
 *   beta_out fp32 [M] (device, written): beta_m.  NULL iff Xq_out is NULL.
 * Both must be NULL when x_dtype is I8 or I8_TILED (the caller already holds
 * them).  When requested, the quantiser writes them and the product reads
 * them as int8 input: the workspace is then the one of x_dtype I8
 * (bitlinear_forward_workspace_bytes(M, N, K, layout, BITLINEAR_I8)), and Y
 * is bit-identical to bitlinear_forward's.  Neither may overlap another
 * buffer of the call.
 */
int bitlinear_forward_ex(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                         const void *X, int x_dtype, int64_t ldx, const float *beta_in, void *Y, int y_dtype,
                         int64_t ldy, int8_t *Xq_out, int64_t ldxq, float *beta_out, void *ws, int64_t ws_bytes,
                         int algo, void *stream);

/*
 * bitlinear_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid allocation).  Arguments and results are those of
 * bitlinear_forward (algo AUTO); the workspace that call would take
 * (bitlinear_forward_workspace_bytes(M, N, K, layout, x_dtype) bytes: the
 * staged int8 activations and beta) is a static device array of BITLINEAR_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends.  The
 * call allocates nothing and frees nothing; it looks the array's address up
 * once per device, on its first call there (make that first call outside
 * graph capture).  Every call on one GPU uses the same array: calls that
 * overlap in time on one GPU (different streams, or host threads, without
 * ordering) race and give undefined results; calls ordered on one stream are
 * safe.  No byte of the array needs to start at any value.
 * Returns BITLINEAR_ERR_SCRATCH, before anything is enqueued, when the
 * workspace would exceed the array.
 */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES (64u << 20)
int bitlinear_forward_noalloc(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                              const void *X, int x_dtype, int64_t ldx, const float *beta_in, void *Y, int y_dtype,
                              int64_t ldy, void *stream);

/*
 * One link of a chain of BitLinears whose per-token activation maxima come
 * from the producer: the per-token absmax of the 8-bit activation quantiser
 * (LIT-380 record, Key takeaways, bullet 1) taken in the epilogue of the
 * product that writes the activations, the fusion across layers the
 * HackerPapers digest's thread "Scalable MatMul-Free Language Modeling"
 * discusses.  The forward of bitlinear_forward (the tiled quantiser, then the
 * matrix-core GEMV) for M <= 16 tokens of fp32 / bf16 X, with two optional
 * additions:
 *   pmax_in, nparts_in  nparts_in x 16 floats (device, read-only) written by
 *        the previous link's pmax_out over exactly the K columns X holds; beta_m
 *        is then their maximum over the parts (bit-identical to the absmax of
 *        the row) and the quantiser makes one pass over X instead of two.
 *        NULL and 0 for none.
 *   pmax_out, pmax_cols  bitlinear_forward_chain_parts(M, N, K, layout) x 16
 *        floats (device, written): entry p * 16 + m is the maximum of |Y[m][n]|
 *        as stored (fp32 or bf16) over the columns n < pmax_cols that
 *        workgroup p of the product wrote (0 for tokens m >= M), written with
 *        plain stores, no atomics.  pmax_cols (1 <= pmax_cols <= N) is the next
 *        link's K (it reads Y[:, :pmax_cols]).  NULL and 0 for none; y_dtype
 *        must be F32 or BF16 with pmax_out.
 * The other arguments, the workspace (bitlinear_forward_workspace_bytes) and
 * the results are those of bitlinear_forward; outputs are bit-identical to it.
 * Returns UNSUPPORTED for M > 16 or K > 65536, INVALID_ARG for the argument
 * errors of bitlinear_forward, a misaligned or overlapping pmax buffer,
 * pmax_cols out of range, or pmax_in and nparts_in not given together.
 */
int bitlinear_forward_chain(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                            const void *X, int x_dtype, int64_t ldx, const float *pmax_in, int64_t nparts_in,
                            void *Y, int y_dtype, int64_t ldy, float *pmax_out, int64_t pmax_cols, void *ws,
                            int64_t ws_bytes, void *stream);

/* Parts (workgroups) of bitlinear_forward_chain's product for these sizes: its
 * pmax_out holds that many x 16 floats.  -1 if M > 16, K > 65536 or invalid. */
int64_t bitlinear_forward_chain_parts(int64_t M, int64_t N, int64_t K, int layout);

/*
 * Grouped forward: several BitLinears in one call, the way a decode step runs
 * the layers of a model (q, k, v and o; gate, up and down).  Each BitLinear's
 * weights are only a few MB, so alone its product cannot fill the chip before
 * its launch ends, while on stock GPUs the packed-weight stream is the whole
 * cost (LIT-380 record, closing section "Standing in the anthology").  Here
 * every job of at most 16 tokens becomes part of one quantiser launch (every
 * distinct input) and one product launch (every layer); other jobs run as
 * bitlinear_forward would run them, after it, on the same stream.
 *
 * Job j computes exactly what bitlinear_forward computes for
 *   P, gamma    packed weights of T [N x K] in the call's 'layout' and their
 *               scale (as bitlinear_forward);
 *   X, ldx      activations [M x K] of the call's x_dtype (F32 or BF16), row
 *               stride ldx >= K;
 *   Y, ldy      output [M x N] of the call's y_dtype, row stride ldy >= N;
 * with the same results bit for bit.  Jobs with the same X, M, K and ldx
 * (e.g. q, k and v) share one quantisation.  No Y may overlap any other
 * buffer of any job.  At most BITLINEAR_MAX_GROUP jobs.
 */
#define BITLINEAR_MAX_GROUP 32

typedef struct {
    const uint8_t *P;
    const float *gamma;
    const void *X;
    void *Y;
    int64_t M, N, K;
    int64_t ldx, ldy;
} bitlinear_job_t;

/* Workspace bytes of bitlinear_forward_grouped for these jobs (host-side,
 * reads jobs only), or -1 for invalid arguments. */
int64_t bitlinear_forward_grouped_workspace_bytes(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype);

/*
 *   jobs     host array of njobs (1 .. BITLINEAR_MAX_GROUP) descriptions; the
 *            call reads it before it returns (the device pointers in it are
 *            used by the enqueued work).
 *   ws       >= bitlinear_forward_grouped_workspace_bytes(...) bytes,
 *            16-byte aligned, overlapping no job buffer.
 * Every job is validated before anything is enqueued (the checks of
 * bitlinear_forward); the first failure is returned.
 */
int bitlinear_forward_grouped(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype, int y_dtype,
                              void *ws, int64_t ws_bytes, void *stream);

/* Name of the product kernel of the grouped launch for these jobs (as
 * profilers print it, e.g. "bl::k_group_gemv<0, 1>" (the quantiser inside,
 * bf16 input), "bl::k_group_gemv<0, 2>" (quantised by k_group_quant_tiled
 * first) or "bl::k_group_gemv_addsub<1>" (the vector-ALU products, see
 * bitlinear_forward_grouped_algo)), or NULL when no job is grouped or the
 * arguments are invalid.  Thread-local storage; host-only. */
const char *bitlinear_grouped_kernel(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype);

/*
 * bitlinear_forward_grouped with the product algorithm chosen by the caller.
 * The decode product is a sum of activations with weights in {-1, 0, +1}:
 * integer additions and subtractions only (LIT-380 record, Key takeaways,
 * the fourth point).  algo:
 *   BITLINEAR_ALGO_AUTO          what bitlinear_forward_grouped runs: the
 *                                vector-ALU products when every grouped job
 *                                is i2 with one token and inputs the launch
 *                                quantises itself (measured as fast or
 *                                faster there), else the matrix cores; jobs
 *                                left out of the grouped launch run as
 *                                bitlinear_forward;
 *   BITLINEAR_ALGO_GEMV_MFMA     the int8 matrix-core products;
 *   BITLINEAR_ALGO_GEMV_ADDSUB   the products on the vector ALU
 *                                ("bl::k_group_gemv_addsub<x_dtype>"): packed
 *                                dot products of the 2-bit codes (T + 1, so
 *                                no multiplier sees a weight other than 0,
 *                                1, 2 or 3 times a power of two) with the
 *                                activations, minus their sum; only for i2
 *                                jobs of one token each, the grouped ones
 *                                with inputs the launch quantises itself
 *                                (16-byte aligned rows), else
 *                                BITLINEAR_ERR_UNSUPPORTED; jobs the grouped
 *                                launch leaves out (rows too long) run as
 *                                bitlinear_forward_algo with this algo;
 *   BITLINEAR_ALGO_GEMM_MFMA     BITLINEAR_ERR_UNSUPPORTED.
 * Results are bit-identical across algorithms.  Other arguments, workspace
 * and errors as bitlinear_forward_grouped; nothing is enqueued on an error.
 */
int bitlinear_forward_grouped_algo(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype, int y_dtype,
                                   int algo, void *ws, int64_t ws_bytes, void *stream);

/* bitlinear_grouped_kernel for bitlinear_forward_grouped_algo with this algo
 * (NULL also where that call returns BITLINEAR_ERR_UNSUPPORTED). */
const char *bitlinear_grouped_kernel_algo(const bitlinear_job_t *jobs, int njobs, int layout, int x_dtype,
                                          int algo);

/*
 * Backward pass under the straight-through estimator (the pages quote the
 * BitNet paper: training lets the gradient bypass the non-differentiable
 * quantisation functions; HackerPapers digest, comment on the
 * straight-through estimator).  Reading: rounding and clipping have
 * derivative 1 and gamma, beta_m are constants, so the layer acts like
 * y = Xhat @ What^T with What = gamma * T and Xhat[m][k] = q[m][k] * r_m,
 * r_m = beta_m / 127 rounded to binary32.  Gradients are fp32 [row-major],
 * accumulated in fp32 (order unspecified; the error is within
 * (n + 2) * 2^-24 of the sum of the absolute terms, n the contraction length).
 */

/* Workspace bytes bitlinear_backward_dx needs for M tokens: room for the i2
 * rewrite of b3 / b1 weights, and, for small batches whose weight rows are
 * split over workgroups, the splits' fp32 partial sums (at most 16 x M x K
 * floats); 0 when neither applies, -1 if invalid. */
int64_t bitlinear_backward_dx_workspace_bytes(int64_t M, int64_t N, int64_t K, int layout);

/*
 * Gradient with respect to the layer input: dX = gamma * (dY @ T).
 *   P, layout, gamma  the forward's packed weights [N x K] and scale.
 *   dY    fp32 [M x N], row stride lddy >= N (device, read-only).
 *   dX    fp32 [M x K], row stride lddx >= K (device, written).
 *   ws    >= bitlinear_backward_dx_workspace_bytes(M, N, K, layout) bytes,
 *         16-byte aligned (may be NULL when that is 0); contents on entry
 *         are ignored.
 * Small batches split the weight rows over workgroups; the splits' partial
 * sums are added in a fixed order by a second kernel, so results are
 * deterministic.
 */
int bitlinear_backward_dx(const uint8_t *P, int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                          const float *dY, int64_t lddy, float *dX, int64_t lddx, void *ws, int64_t ws_bytes,
                          void *stream);

/*
 * Gradient with respect to the latent fp32 weights W (the estimator passes
 * d/dWhat straight to W): dW = dY^T @ Xhat.
 *   Xq, ldq, beta  the forward's int8 activations [M x K] (row stride
 *         ldq >= K) and per-token beta [M], as bitlinear_quantize_act
 *         writes them.
 *   dY    fp32 [M x N], row stride lddy >= N.
 *   dW    fp32 [N x K], row stride lddw >= K (written, not accumulated).
 */
int bitlinear_backward_dw(const int8_t *Xq, int64_t ldq, const float *beta, int64_t M, int64_t N, int64_t K,
                          const float *dY, int64_t lddy, float *dW, int64_t lddw, void *stream);

/*
 * Name of the main kernel a backward call with these sizes launches (which =
 * 0: bitlinear_backward_dx, 1: bitlinear_backward_dw), e.g. "bl::k_bwd_dx"
 * or, for small batches, "bl::k_bwd_dx_few" ("bl::k_bwd_dx_vec<1>" for one
 * token; either is followed by "bl::k_bwd_dx_sum" when it splits the weight
 * rows) and "bl::k_bwd_dw_few" ("bl::k_bwd_dw_vec" for one token); NULL for
 * sizes or a 'which' the calls reject.  A static string; host-only,
 * enqueues nothing.
 */
const char *bitlinear_backward_kernel(int64_t M, int64_t N, int64_t K, int which);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
