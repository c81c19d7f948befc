// launch.h -- host-side launchers of the libbitlinear kernels (internal).
// Each launcher enqueues its kernels on 'stream' and returns hipGetLastError().
// Arguments are validated by api.cpp before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

hipError_t launch_quantize_weights(const float *W, int64_t N, int64_t K, int64_t ldw, int8_t *T, float *gamma,
                                   void *ws, hipStream_t stream);

hipError_t launch_pack(const int8_t *T, int64_t N, int64_t K, int64_t ldt, int layout, uint8_t *P,
                       hipStream_t stream);

// Rewrite b3-packed weights P3 [N x K] in the i2 layout (P2, i2 packed size).
hipError_t launch_b3_to_i2(const uint8_t *P3, int64_t N, int64_t K, uint8_t *P2, hipStream_t stream);
// Rewrite b1-packed (binary) weights P1 [N x K] in the i2 layout; positions
// past K become T = 0.
hipError_t launch_b1_to_i2(const uint8_t *P1, int64_t N, int64_t K, uint8_t *P2, hipStream_t stream);
// Binary weights: gamma = mean|W| as for the ternary path, T = +1 where
// w >= 0, else -1.
hipError_t launch_binarize_weights(const float *W, int64_t N, int64_t K, int64_t ldw, int8_t *T, float *gamma,
                                   void *ws, hipStream_t stream);

hipError_t launch_quant_act(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t *Xq,
                            int64_t ldq, float *beta, hipStream_t stream);

// Tiled activation layout: see bitlinear_act_tiled_bytes in bitlinear.h.
inline int64_t tiled_step_k(int layout) { return layout == 0 ? 256 : (layout == 1 ? 320 : 512); }
inline int64_t tiled_nmf(int layout) { return layout == 0 ? 4 : (layout == 1 ? 5 : 8); }
inline int64_t tiled_nsteps(int64_t K, int layout) { return (K + tiled_step_k(layout) - 1) / tiled_step_k(layout); }
inline int64_t tiled_bytes(int64_t M, int64_t K, int layout)
{
    return (M + 15) / 16 * tiled_nsteps(K, layout) * tiled_nmf(layout) * 1024;
}

// pmax (optional, M <= 16): nparts x 16 producer-side maxima of |x| per token
// over exactly the K columns; beta is their maximum (no pass over the values).
hipError_t launch_quant_act_tiled(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int layout,
                                  int8_t *Xt, float *beta, hipStream_t stream, const float *pmax = nullptr,
                                  int64_t nparts = 0);

// ---- grouped forward (several BitLinears of at most 16 tokens) ------------
constexpr int GROUP_MAX_INPUTS = 32;
constexpr int GROUP_MAX_JOBS = 32;

// One distinct input of the group: X [M x K] (row stride ldx), quantised per
// token into the tiled layout Xt (token group 0; only the M real rows are
// written) and beta [M].  The grouped quantiser's grid is (largest M, inputs):
// workgroup (m, u) quantises row m of input u (none when m >= M).
struct GroupInput {
    const void *X;
    int8_t *Xt;
    float *beta;
    int64_t ldx;
    int M, K, nsteps;
};
struct GroupQuantArgs {
    int ninputs, layout;
    GroupInput in[GROUP_MAX_INPUTS];
};
// Quantise every input of the group (one launch).
hipError_t launch_group_quant(const GroupQuantArgs &args, int x_dtype, hipStream_t stream);

// One BitLinear of the group: packed weights P of [N x K] (KB k-blocks,
// nsteps k-steps), its tiled int8 activations and beta, output Y (row stride
// ldy).  Workgroups wg0 .. wg0 + nwg - 1 of the grouped GEMV's grid serve
// it; jobidx (four 8-bit job indices per word) maps a workgroup to its job.
struct GroupJob {
    const uint8_t *P;
    const float *gamma;
    const int8_t *Xt;  // quantised activations (tiled; separate quantiser)
    const float *beta; // their beta
    const void *X;     // or the fp32 / bf16 rows, quantised inside (1-4 tokens)
    int64_t ldx;
    void *Y;
    int64_t ldy;
    int M, N, K, KB, nsteps, wg0, nwg;
};
constexpr int GROUP_MAX_WGS = 512; // workgroups of one grouped launch
struct GroupGemvArgs {
    int njobs, y_dtype;
    uint32_t jobidx[GROUP_MAX_WGS / 4];
    GroupJob job[GROUP_MAX_JOBS];
};
// Largest k-step count a grouped job may have, its row tiles per workgroup,
// and the plan of a launch (workgroups per job are filled in by the plan).
int group_max_nsteps(int layout);
constexpr int GROUP_STAGE_TILES = 24;
struct GroupPlan {
    int waves; // per workgroup
    int spw;   // k-steps per wave (template)
    int wgs;   // workgroups in all (at most GROUP_MAX_WGS; 0: too many)
};
GroupPlan group_plan(GroupGemvArgs &args, int layout);
// x_dtype DT_I8: the jobs read Xt / beta (k_group_quant_tiled ran first);
// DT_F32 / DT_BF16: every job has 1 to 4 tokens of 16-byte aligned rows X,
// quantised inside.
// addsub: the products on the vector ALU (k_group_gemv_addsub), for i2 jobs of
// one token each (group_addsub_ok).
hipError_t launch_group_gemv(const GroupGemvArgs &args, const GroupPlan &plan, int layout, int x_dtype,
                             hipStream_t stream, bool addsub = false);
bool group_addsub_ok(const GroupGemvArgs &args, int layout);
void group_gemv_kernel_name(int layout, int x_dtype, bool addsub, char *buf, size_t n);

// Product + rescale on int8 activations Xq [M x K] (row stride ldq, 16-byte
// aligned rows) with per-token beta.
struct GemvArgs {
    const uint8_t *P;
    int layout;
    const float *gamma;
    int64_t M, N, K;
    const int8_t *Xq;
    int64_t ldq;
    bool tiled; // Xq holds the tiled activation layout (ldq unused)
    const float *beta;
    void *Y;
    int y_dtype;
    int64_t ldy;
    // optional (k_gemv_mfma / k_gemv_persist, one token group): per-workgroup
    // maxima of |Y| per token over the columns below pmax_cols, written to
    // pmax[workgroup * 16 + token]
    float *pmax = nullptr;
    int64_t pmax_cols = 0;
};

hipError_t launch_gemv_addsub(const GemvArgs &a, hipStream_t stream);
// Workgroups along the row tiles of the matrix-core GEMV for one token group
// (the number of partial maxima it writes with GemvArgs::pmax).
int64_t gemv_mfma_parts(int layout, int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_mfma(const GemvArgs &a, hipStream_t stream);
// The matrix-core GEMV with the activation quantiser inside (k_gemv_fq): the
// whole forward in one launch for 1 to 4 tokens of fp32 / bf16 input X (rows
// of ldx values); a.Xq, a.ldq and a.beta are unused.  gemv_fq_shape: the
// shape qualifies; gemv_fq_ok: the shape and X's alignment and extent do.
bool gemv_fq_shape(int layout, int64_t M, int64_t N, int64_t K, int x_dtype);
bool gemv_fq_ok(int layout, int64_t M, int64_t N, int64_t K, int x_dtype, const void *X, int64_t ldx);
hipError_t launch_gemv_fq(const GemvArgs &a, const void *X, int x_dtype, int64_t ldx, hipStream_t stream);
hipError_t launch_gemm_mfma(const GemvArgs &a, hipStream_t stream); // i2 or b3 weights
// Size of an M x N product in 64 x 128 output tiles: below about 128 of them
// the matrix-core GEMV is faster than the GEMM (measured on the 70B layers).
int64_t gemm_tiles(int64_t M, int64_t N);
// Whether the GEMM decodes b3 weights itself for this shape.  Every M-block of
// a workgroup tile decodes its weight tiles again (about 30 VALU instructions
// per 20 weights), so with more than two M-blocks one rewrite of the weights
// as i2 (a single pass) and the i2 GEMM are faster (measured on the 70B
// layers: gate at 64 tokens 45 us native against 60 us, q and down at 176
// tokens the other way round).

// Straight-through-estimator gradients (backward.hip): dX from i2-packed
// weights, dW from the forward's int8 activations and beta.
// Name of the kernel bitlinear_backward_dx (dx) or _dw (!dx) launches for M
// tokens and K columns.
const char *bwd_kernel_name(bool dx, int64_t M, int64_t K);
// Splits of the weight rows the small-batch dX kernel uses, and the bytes of
// their partial tiles (0 when it does not split).
int64_t bwd_dx_splits(int64_t M, int64_t N, int64_t K);
int64_t bwd_dx_partial_bytes(int64_t M, int64_t N, int64_t K);
// part: bwd_dx_partial_bytes(M, N, K) bytes, 16-byte aligned (unused if 0).
hipError_t launch_bwd_dx(const uint8_t *P2, const float *gamma, int64_t M, int64_t N, int64_t K, const float *dY,
                         int64_t lddy, float *dX, int64_t lddx, float *part, hipStream_t stream);
hipError_t launch_bwd_dw(const int8_t *Xq, int64_t ldq, const float *beta, int64_t M, int64_t N, int64_t K,
                         const float *dY, int64_t lddy, float *dW, int64_t lddw, hipStream_t stream);

// Names (as profilers print them, without the argument list) of the kernel a
// product launch runs for a shape.
void gemv_kernel_name(int layout, int64_t M, int64_t N, int64_t K, bool tiled, char *buf, size_t n);
void gemv_addsub_kernel_name(int64_t M, char *buf, size_t n);
void gemv_fq_kernel_name(int layout, int64_t M, int64_t N, int64_t K, int x_dtype, char *buf, size_t n);
void gemm_kernel_name(int layout, int64_t M, int64_t N, char *buf, size_t n);

} // namespace bl
