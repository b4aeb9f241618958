/*
 * moegq -- gathered affine-quantized MoE expert matmul for AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a device pointer owned by the caller unless
 * stated otherwise; the library never allocates, frees or retains memory.  Every entry
 * point except moegq_selfcheck and moegq_validate_indices is asynchronous on
 * `stream` (a hipStream_t passed as void*; NULL = the default stream): it only
 * validates its arguments on the host and enqueues kernels; it never
 * synchronizes and never reads device memory back.  Outputs are valid once the
 * stream reaches that point.
 *
 * Errors: the return value is MOEGQ_OK (0) or a negative moegq_status.  On any
 * argument error nothing is launched and outputs are untouched.  Empty inputs
 * (zero pairs / rows / tokens) return MOEGQ_OK with no launch.
 *
 * Index preconditions that would need a device->host read to check are the
 * caller's: 0 <= expert index < E, 0 <= row index < rows of x, and a truthful
 * `sorted_indices` hint.  moegq_validate_indices checks them (synchronizing).
 *
 * Formats (the pages' packed affine layout):
 *   packed weights  uint32 [E, N, K*bits/32]; code k of a row sits at bit
 *                   offset k*bits of the row's little-endian word stream
 *                   (LSB first);
 *   scales, biases  bf16   [E, N, K/group_size]; w = q*scale + bias;
 *   activations     bf16, row-major.
 * Sources: nuvec-core tests/quantized.rs ("round_trip_error_is_about_half_a_step",
 * "composed"); MLX issue 4509 (benchmark script, gq()).
 */
#ifndef MOEGQ_H
#define MOEGQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOEGQ_OK = 0,
  MOEGQ_ERR_NULL_ARG = -1,     /* a required pointer is NULL                       */
  MOEGQ_ERR_BITS = -2,         /* bit width outside the supported set              */
  MOEGQ_ERR_GROUP_SIZE = -3,   /* group size outside {32, 64, 128}                 */
  MOEGQ_ERR_SHAPE = -4,        /* K % group_size, packed width, inner size, counts */
  MOEGQ_ERR_DTYPE = -5,        /* integer activations, non-u32 packed words,
                                  float indices                                    */
  MOEGQ_ERR_UNSUPPORTED = -6,  /* valid for the format but not built here (bit
                                  widths other than 4 and 8 outside gather_qmm,
                                  64-bit indices, and the entry points whose
                                  comment says so)                                 */
  MOEGQ_ERR_WORKSPACE = -7,    /* workspace NULL or smaller than required          */
  MOEGQ_ERR_LAUNCH = -8,       /* a kernel launch failed (hipGetLastError)         */
  MOEGQ_ERR_SELFCHECK = -9,    /* fused combine differs from the unfused tail      */
  MOEGQ_ERR_INDEX = -10,       /* moegq_validate_indices found a bad index         */
  MOEGQ_ERR_ALIGN = -11        /* activations, packed weights, outputs and
                                  workspaces must be 16-byte aligned               */
} moegq_status;

/* dtype codes for the checked operands */
typedef enum {
  MOEGQ_BF16 = 0, MOEGQ_F16 = 1, MOEGQ_F32 = 2, MOEGQ_F64 = 3,
  MOEGQ_I32 = 4, MOEGQ_U32 = 5, MOEGQ_I64 = 6
} moegq_dtype;

/* switch_glu modes */
enum { MOEGQ_MODE_AUTO = 0, MOEGQ_MODE_DECODE = 1, MOEGQ_MODE_SORTED = 2 };
/* row-tile modes of the sorted route */
enum { MOEGQ_TILES_SCHEDULED = 0, MOEGQ_TILES_NAIVE = 1 };
/* operations whose workspace can be queried */
enum { MOEGQ_OP_GATHER_QMM = 0, MOEGQ_OP_SWITCH_GLU_DECODE = 1, MOEGQ_OP_SWITCH_GLU_SORTED = 2,
       MOEGQ_OP_COMBINE_UNFUSED = 3, MOEGQ_OP_SELFCHECK = 4, MOEGQ_OP_SORT_PAIRS = 5,
       MOEGQ_OP_MOE_DECODE = 6, MOEGQ_OP_GATHER_MM = 7 };

const char* moegq_status_string(int status);
const char* moegq_version(void);

/* Bytes of workspace an operation needs.  Arguments not used by `op` are
 * ignored: GATHER_QMM(P, E, N=M rows per batch, bm ignored),
 * SWITCH_GLU_DECODE(P pairs, E, N = I, bm), SWITCH_GLU_SORTED(P, E, N = I, bm; bm 0 = auto),
 * COMBINE_UNFUSED(P = T*top_k, E ignored, N = H), SELFCHECK(all ignored),
 * SORT_PAIRS(P, E), MOE_DECODE(P = T*top_k, E, N = I).  Returns 0 for an unknown op. */
size_t moegq_workspace_bytes(int op, int64_t P, int64_t E, int64_t N, int bm);

/*
 * gather_qmm: out[p] = x[lhs(p)] . dequant(w[rhs[p]])^T  for p in [0, P).
 *   MLX issue 4509, gq(): gather_qmm(x, w, scales, biases, rhs_indices,
 *   transpose, group_size, bits, sorted_indices); nuvec "gather_qmm_selects_batches"
 *   adds lhs_indices (each output batch = quantized_matmul of the selected x
 *   batch and weight batch).
 * x        [X, M, K] activations, x_dtype BF16, F16 or F32 (F64 and integers ->
 *          MOEGQ_ERR_DTYPE).
 * transpose=1: w [E, N, K*bits/32] uint32 (w_dtype must be MOEGQ_U32),
 *          scales, biases [E, N, K/group_size] bf16 (groups along K).
 * transpose=0: w [E, K, N*bits/32], scales, biases [E, K, N/group_size] bf16
 *          (groups along N; nuvec "quantized_matmul_equals_the_dequantized_product"
 *          runs this layout with K as the weight rows): out = x . dequant(W).
 * lhs_indices [P] (idx_dtype I32 or U32) or NULL -> lhs(p) = p / lhs_div
 *          (lhs_div >= 1; P1's x[M,1,1,K] with idx[M,top_k] is lhs_div = top_k).
 * rhs_indices [P] expert per pair (same idx_dtype), required.
 * sorted_indices  hint that rhs is non-decreasing; with M == 1 it selects the
 *          expert-grouped MFMA route (needs workspace).
 * out      [P, M, N] in the promoted type (nuvec "reference": activation type
 *          promoted with the bf16 scale type): bf16 for BF16 activations,
 *          float32 for F16 and F32 ones.
 * bits     1, 2, 3, 4, 5, 6 or 8 (nuvec "round_trip_error_is_about_half_a_step":
 *          the format's widths; code k of a row at bits [k*bits, (k+1)*bits) of
 *          its little-endian word stream); group_size 32, 64 or 128.
 * Routes: bf16 activations with transpose=1 and 4 or 8 bits use the
 *          matrix-vector, few-row MFMA and tile kernels; transpose=0, F16/F32
 *          activations or the other widths use the vector-unit kernels, whose
 *          K split keeps fp32 partial sums in the workspace (one matrix must be
 *          below 2 GiB, else UNSUPPORTED).
 * workspace/workspace_bytes: moegq_gather_qmm_workspace_bytes(...) bytes (0 when
 *          the route needs none; then NULL is accepted).  Not shared between
 *          calls that overlap on one stream or on several streams.
 */
int moegq_gather_qmm(const void* x, int x_dtype, int64_t X, int64_t M, int64_t K,
                     const void* w, int w_dtype, const void* scales, const void* biases,
                     int64_t E, int64_t N,
                     const void* lhs_indices, int64_t lhs_div, const void* rhs_indices,
                     int idx_dtype, int64_t P, int sorted_indices, int transpose,
                     int group_size, int bits, void* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes that moegq_gather_qmm needs for these arguments (every
 * route; sorted_indices as passed to the call).  0 for arguments the call
 * rejects. */
size_t moegq_gather_qmm_workspace_bytes(int64_t P, int64_t E, int64_t M, int64_t N, int64_t K, int x_dtype,
                                        int transpose, int bits, int sorted_indices);

/* mx modes of gather_qmm */
enum { MOEGQ_MXFP4 = 1, MOEGQ_MXFP8 = 2 };

/*
 * gather_qmm_mx: gather_qmm for the microscaling modes.  MLX PR 4787's
 * benchmark script runs quantized_matmul with mode "mxfp8" (and lists
 * "mxfp4"), whose quantize() returns no biases.  Encoding (OCP Microscaling):
 * elements E2M1 (MOEGQ_MXFP4, 8 per uint32 word) or E4M3 (MOEGQ_MXFP8, 4 per
 * word), packed LSB-first like the affine codes; one E8M0 scale byte
 * (2^(e-127), 255 = NaN) per 32 consecutive elements along the packed axis.
 * transpose=1: w [E, N, K*bits/32] uint32, scales [E, N, K/32] uint8.
 * transpose=0: w [E, K, N*bits/32], scales [E, K, N/32] uint8.
 * The packed axis must be a multiple of 32 (else MOEGQ_ERR_SHAPE); mode
 * other than the two -> MOEGQ_ERR_BITS.  Other arguments, the result type
 * (bf16 for BF16 activations, float32 for F16/F32) and the workspace rules
 * are those of moegq_gather_qmm; workspace bytes from
 * moegq_gather_qmm_mx_workspace_bytes.
 */
int moegq_gather_qmm_mx(const void* x, int x_dtype, int64_t X, int64_t M, int64_t K, const void* w,
                        const void* scales, int64_t E, int64_t N, const void* lhs_indices, int64_t lhs_div,
                        const void* rhs_indices, int idx_dtype, int64_t P, int transpose, int mode, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);
size_t moegq_gather_qmm_mx_workspace_bytes(int64_t P, int64_t M, int64_t N, int64_t K, int transpose, int mode);

/*
 * gather_qmm_glu: h[p] = bf16( silu(g) * u ) with g = x[lhs(p)] . dequant(wg[rhs[p]])^T
 * and u = x[lhs(p)] . dequant(wu[rhs[p]])^T, g and u rounded to bf16 first:
 * the gate/up half of SwitchGLU over gathered experts (MLX issue 4509, moe():
 * up and gate are gather_qmm outputs, then g * sigmoid(g) * u).  Arguments as
 * moegq_gather_qmm with two weight triples (both [E, N, K*bits/32] u32 and
 * [E, N, K/group_size] bf16); out [P, M, N] bf16; transpose is implied.
 */
int moegq_gather_qmm_glu(const void* x, int x_dtype, int64_t X, int64_t M, int64_t K,
                         const void* wg, const void* sg, const void* bg,
                         const void* wu, const void* su, const void* bu,
                         int64_t E, int64_t N, const void* lhs_indices, int64_t lhs_div,
                         const void* rhs_indices, int idx_dtype, int64_t P, int sorted_indices,
                         int group_size, int bits, void* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * affine_qmm: out = x . dequant(w)^T, x [M, K] bf16, w [N, K*bits/32] u32,
 * scales/biases [N, K/group_size] bf16, out [M, N] bf16.
 *   nuvec "quantized_matmul_equals_the_dequantized_product"; MLX PR 4787
 *   (few-row affine quantized_matmul, 3-16 rows).
 * residual: NULL, or [M, N] bf16 added after rounding:
 *   out = bf16(residual + bf16(x . W^T)) (the decoder chain's residual add,
 *   MLX PR 4787 benchmark script).  out may alias residual.
 * x_dtype must be BF16 and transpose 1 (else MOEGQ_ERR_UNSUPPORTED): the other
 *   activation types and the layout without the transpose are served by
 *   moegq_gather_qmm with one weight batch (E = 1, rhs all zero), which takes
 *   a workspace for its K split.
 */
int moegq_affine_qmm(const void* x, int x_dtype, int64_t M, int64_t K,
                     const void* w, int w_dtype, const void* scales, const void* biases,
                     int64_t N, int transpose, int group_size, int bits,
                     const void* residual, void* out, void* stream);
/*
 * affine_qmm_ws / affine_qmm_glu_ws: the same products with a workspace that
 * lets 5..16-row products with K a multiple of 128 split K over workgroups
 * (so that products with few output columns still fill the machine; 1..4
 * rows run the matrix-vector kernel, which takes no workspace):
 * moegq_affine_qmm_workspace_bytes(M, N, K, glu) bytes, 16-byte aligned,
 * ZERO-FILLED before its first use; every call leaves it in that state (its
 * per-column-group counters return to zero, the fp32 partials are scratch).
 * A NULL or smaller workspace runs the same kernel without the split.  The
 * split's partial sums are added in split order, so results do not depend on
 * timing; they can differ from the unsplit call's in the last bits of fp32
 * (a different summation order), within the format's tolerance.  The layout
 * (counters, then partials) depends on N, K and glu, not on M: one workspace
 * serves every call with the same N, K and glu; a call of another shape may
 * leave nonzero words where this shape keeps its counters, so each product
 * shape takes a workspace of its own.  Calls that overlap (several streams)
 * must not share one workspace.
 */
int moegq_affine_qmm_ws(const void* x, int x_dtype, int64_t M, int64_t K,
                        const void* w, int w_dtype, const void* scales, const void* biases,
                        int64_t N, int transpose, int group_size, int bits,
                        const void* residual, void* out, void* workspace, size_t workspace_bytes,
                        void* stream);
size_t moegq_affine_qmm_workspace_bytes(int64_t M, int64_t N, int64_t K, int glu);

/*
 * affine_qmm_glu: out = bf16( silu(x . Wg^T) * (x . Wu^T) ), the dense SwiGLU
 * front half (MLX issue 4509: "up, gate, silu(gate)*up"; MLX PR 4787 script:
 * g * sigmoid(g) * u).  Wg, Wu [N, K*bits/32], scales/biases [N, K/gs].
 */
int moegq_affine_qmm_glu(const void* x, int64_t M, int64_t K,
                         const void* wg, const void* sg, const void* bg,
                         const void* wu, const void* su, const void* bu,
                         int64_t N, int group_size, int bits, void* out, void* stream);
int moegq_affine_qmm_glu_ws(const void* x, int64_t M, int64_t K,
                            const void* wg, const void* sg, const void* bg,
                            const void* wu, const void* su, const void* bu,
                            int64_t N, int group_size, int bits, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * switch_glu: the routed-expert chain of a MoE layer (MLX issue 4509, moe():
 * up, gate, silu(gate)*up, down over gathered experts; MTPLX PR 558 Change:
 * the sorted chain sorts the (token, slot) pairs by expert, runs the experts on
 * the sorted rows and returns the sorted output with its inverse permutation).
 * x [T, H] bf16; idx [T, top_k] int32 expert ids (0 <= id < E);
 * gate/up: w [E, I, H*bits/32] u32, s/b [E, I, H/gs] bf16;
 * down:    w [E, H, I*bits/32] u32, s/b [E, H, I/gs] bf16.
 * mode DECODE: y [T*top_k, H] in token order (pair p = t*top_k + k); inv, if
 *   not NULL, receives the identity permutation.
 * mode SORTED: y [T*top_k, H] in expert-sorted order; inv [T*top_k] receives
 *   the inverse permutation (pair -> sorted row), required.
 * mode AUTO: resolves to DECODE or SORTED as moegq_switch_glu_mode() says;
 *   inv is then required, so the caller's combine works for either layout.
 * tile_mode: SCHEDULED (expert-aware tiles, MLX PR 4567) or NAIVE (fixed row
 *   tiles, one K pass per expert present); bm: row-tile height (16/32/64/128),
 *   0 = auto.
 * workspace: moegq_workspace_bytes(MOEGQ_OP_SWITCH_GLU_{DECODE,SORTED}, T*top_k, E, I, bm).
 */
int moegq_switch_glu(const void* x, int64_t T, int64_t H, int64_t I, int64_t E,
                     const int32_t* idx, int64_t top_k,
                     const void* wg, const void* sg, const void* bg,
                     const void* wu, const void* su, const void* bu,
                     const void* wd, const void* sd, const void* bd,
                     int group_size, int bits, int mode, int tile_mode, int bm,
                     void* y, int32_t* inv, void* workspace, size_t workspace_bytes,
                     void* stream);

/* The mode AUTO resolves to for T*top_k pairs over E experts (DECODE or SORTED). */
int moegq_switch_glu_mode(int64_t T, int64_t top_k, int64_t E);

/*
 * moe_prefill: one whole MoE layer on the expert-sorted route (MTPLX PR 558
 * Summary and Change: sorted gather, gated shared expert, one-pass combine;
 * MLX PR 4567 Proposed changes: per-expert offsets and row tiles of one
 * expert each; MLX issue 4509 moe(): gate, up, silu(gate) * up, down):
 *   out[t] = bf16( bf16( sum_k bf16(y[t,k] * score[t,k]) ) + shared[t] ),
 *   shared[t] = bf16( sigmoid(z[t]) * s[t] ), z[t] = bf16(x[t] . dequant(w_gate)^T),
 *   s[t] = SwiGLU of the shared expert (gate/up [I, H], down [H, I]), y as in
 *   moegq_switch_glu.
 * The shared expert rides in the routed launches as one more expert whose
 * rows are the T tokens.  Float parity with the composition moegq_switch_glu
 * (SORTED) + moegq_affine_qmm_glu / moegq_affine_qmm / moegq_sigmoid_gate +
 * moegq_moe_combine (the combine is bit-identical given the same y, s, z).
 * x [T, H] bf16; idx [T, top_k] int32; scores [T, top_k] bf16; routed weights
 * as moegq_switch_glu; shared matrices with the routed matrices' shapes minus
 * the expert axis (the shared intermediate size must equal I), gate row
 * [1, H*bits/32] words + [1, H/gs] scales/biases.  shg_w == NULL: no shared
 * expert (every shared pointer ignored).  H and I must be multiples of 128
 * and of 8 * group_size (else MOEGQ_ERR_UNSUPPORTED).
 * out [T, H] bf16.  workspace: moegq_moe_prefill_workspace_bytes(...) bytes;
 * it includes room for the unfused tail, which the layer runs (sigmoid gate,
 * unsort, score, sum, add: same bits) instead of the one-pass combine after a
 * failed moegq_selfcheck on the current device.
 */
int moegq_moe_prefill(const void* x, int64_t T, int64_t H, int64_t I, int64_t E,
                      const int32_t* idx, int64_t top_k, const void* scores,
                      const void* wg, const void* sg, const void* bg,
                      const void* wu, const void* su, const void* bu,
                      const void* wd, const void* sd, const void* bd,
                      const void* shg_w, const void* shg_s, const void* shg_b,
                      const void* shu_w, const void* shu_s, const void* shu_b,
                      const void* shd_w, const void* shd_s, const void* shd_b,
                      const void* gate_w, const void* gate_s, const void* gate_b,
                      int group_size, int bits, void* out, void* workspace,
                      size_t workspace_bytes, void* stream);
size_t moegq_moe_prefill_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t H, int64_t I,
                                         int has_shared);

/*
 * moe_prefill_layout: where moegq_moe_prefill keeps its sort results and its
 * two tile tables inside the caller's workspace, for inspection after a call
 * (MLX PR 4567 Proposed changes: each tile is (row start, expert, valid
 * rows); the whole-layer route writes one table of up-to-128-row tiles and
 * one of up-to-32-row tiles).  Writes, for the same (T, top_k, E, H, I,
 * has_shared) as the call:
 *   offsets[9]: byte offsets from the workspace start of inv [P] int32,
 *     lhs [P + extra] int32 (extra = T with a shared expert, else 0),
 *     sorted_rhs [P], counts [E], expert offsets [E + 1], the 128-row table
 *     [caps[0], 3], the 32-row table [caps[1], 3], the two tile counts
 *     [2] int32, and the unfused tail's scratch [P + 2 T, H] bf16 (written
 *     only after a failed self-check);
 *   caps[2]: capacity (entries) of the two tables;
 *   params[4]: the big tile height (128), the small tile height (32), the
 *     workgroup slots and the first pass's column blocks (ceil(I / 128))
 *     that decide, on the current device, whether any expert gets 128-row
 *     tiles (every expert takes 32-row tiles when the 128-row tiles times the
 *     column blocks come to at most slots / 8).
 * Host-only (no launch, no device access); all pointers are host memory owned
 * by the caller.  Errors: MOEGQ_ERR_SHAPE, MOEGQ_ERR_UNSUPPORTED (E > 1024),
 * MOEGQ_ERR_NULL_ARG.
 */
int moegq_moe_prefill_layout(int64_t T, int64_t top_k, int64_t E, int64_t H, int64_t I, int has_shared,
                             int64_t* offsets, int64_t* caps, int32_t* params);

/*
 * moe_decode: the routed half of a MoE decode layer in two kernels.  Kernel 1
 * is the gathered gate/up with silu(gate)*up (MLX issue 4509, moe()); kernel 2
 * is the gathered down projection fused with the combine tail (MTPLX PR 558:
 * unsort, x score, sum over top_k, + shared expert), so y never round-trips
 * through HBM:
 *   out[t] = bf16( bf16( sum_k bf16(y[t,k] * score[t,k]) ) + shared[t] ),
 *   y[t,k] = bf16( h[t,k] . dequant(Wd[idx[t,k]])^T ),
 *   h[t,k] = bf16( silu(bf16(g)) * bf16(u) ),  g/u = x[t] . dequant(Wg/Wu[idx[t,k]])^T.
 * Bit-identical to moegq_switch_glu (DECODE) followed by moegq_moe_combine.
 * x [T, H] bf16; idx [T, top_k] int32; scores [T, top_k] bf16; shared [T, H]
 * bf16 or NULL; weights as moegq_switch_glu; out [T, H] bf16; y [T*top_k, H]
 * bf16 or NULL (receives the expert outputs when given).
 * workspace: moegq_workspace_bytes(MOEGQ_OP_MOE_DECODE, T*top_k, E, I, 0)
 * bytes (for top_k > 8 the two steps run unfused and y must be given).
 */
int moegq_moe_decode(const void* x, int64_t T, int64_t H, int64_t I, int64_t E,
                     const int32_t* idx, int64_t top_k, const void* scores, const void* shared,
                     const void* wg, const void* sg, const void* bg,
                     const void* wu, const void* su, const void* bu,
                     const void* wd, const void* sd, const void* bd,
                     int group_size, int bits, void* out, void* y,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_decode_static: moegq_moe_decode for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, kernels and results, without the
 * workspace; the gate/up intermediate [T * top_k, I] bf16 lives in a static
 * device array of the library, one per GPU, of moegq_static_scratch_bytes()
 * bytes (8 MiB: T * top_k * I <= 4 Mi, e.g. 256 tokens at top-8 and inter
 * 2048), held until the process ends.  Larger sizes return
 * MOEGQ_ERR_WORKSPACE with nothing launched; no memory is allocated or freed.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (several streams or host threads) race and must be serialized by the
 * caller.  The array keeps the last call's contents; nothing in it needs to
 * start at zero (each call writes the intermediate before reading it).
 */
int moegq_moe_decode_static(const void* x, int64_t T, int64_t H, int64_t I, int64_t E,
                            const int32_t* idx, int64_t top_k, const void* scores, const void* shared,
                            const void* wg, const void* sg, const void* bg,
                            const void* wu, const void* su, const void* bu,
                            const void* wd, const void* sd, const void* bd,
                            int group_size, int bits, void* out, void* y, void* stream);
size_t moegq_static_scratch_bytes(void);

/*
 * moe_combine (fused, one pass): MTPLX PR 558 Summary/Motivation -- unsort,
 * multiply by the routing scores, sum over top_k and add the gated shared
 * expert in one pass, with the rounding of the unfused tail:
 *   out[t] = bf16( bf16( sum_k bf16(y[inv[t*top_k+k]] * score[t,k]) ) + shared[t] )
 * Each bf16 op is evaluated in fp32 and rounded to nearest even; the sum over
 * k starts at slot 0 and adds slots in order in fp32.
 * y [T*top_k, H] bf16; inv [T*top_k] int32 or NULL (= identity, token order);
 * scores [T, top_k] bf16; shared [T, H] bf16 or NULL; out [T, H] bf16.
 * Bit-identical to moegq_moe_combine_unfused on the same inputs.
 * After a failed moegq_selfcheck on the current device it launches nothing
 * and returns MOEGQ_ERR_SELFCHECK (the caller runs moegq_moe_combine_unfused).
 */
int moegq_moe_combine(const void* y, const int32_t* inv, const void* scores, const void* shared,
                      int64_t T, int64_t top_k, int64_t H, void* out, void* stream);

/*
 * moe_combine_gated: moegq_moe_combine with the shared expert's sigmoid gate
 * applied in the same pass: shared[t] is the ungated shared expert output and
 * z [T] bf16 its gate logit; the added term is bf16(sigmoid(z[t]) * shared[t]),
 * the arithmetic of moegq_sigmoid_gate (MTPLX PR 558 Summary: the combine
 * takes the gated shared expert).  Bit-identical to moegq_sigmoid_gate
 * followed by moegq_moe_combine.  After a failed moegq_selfcheck on the
 * current device it launches nothing and returns MOEGQ_ERR_SELFCHECK.
 */
int moegq_moe_combine_gated(const void* y, const int32_t* inv, const void* scores, const void* shared,
                            const void* z, int64_t T, int64_t top_k, int64_t H, void* out, void* stream);

/*
 * moe_combine_unfused: the same arithmetic as four kernels that each write a
 * bf16 tensor (unsort -> [T, top_k, H], x score -> [T, top_k, H], sum -> [T, H],
 * + shared -> out), as the stock tail does (MTPLX PR 558 Motivation).
 * scratch: moegq_workspace_bytes(MOEGQ_OP_COMBINE_UNFUSED, T*top_k, 0, H, 0) bytes.
 */
int moegq_moe_combine_unfused(const void* y, const int32_t* inv, const void* scores,
                              const void* shared, int64_t T, int64_t top_k, int64_t H,
                              void* out, void* scratch, size_t scratch_bytes, void* stream);

/*
 * sort_pairs: stable sort of the flattened (token, slot) pairs by expert
 * (MTPLX PR 558 Change, "_gather_sort"; MLX PR 4567: offsets precomputed from
 * rhs_indices).  idx [T, top_k] (I32/U32).  Outputs (all int32, device):
 * order [P] (sorted row -> pair p = t*top_k + k; ties keep pair order),
 * lhs [P] = order / top_k, sorted_rhs [P], inv [P] (pair -> sorted row),
 * counts [E], offsets [E+1] (exclusive prefix of counts).  Any output except
 * inv, counts and offsets may be NULL.  E <= 1024.
 * workspace: moegq_workspace_bytes(MOEGQ_OP_SORT_PAIRS, P, E, 0, 0) bytes (per-block
 * expert counts of the multi-workgroup sort).
 */
int moegq_sort_pairs(const void* idx, int idx_dtype, int64_t T, int64_t top_k, int64_t E,
                     int32_t* order, int32_t* lhs, int32_t* sorted_rhs, int32_t* inv,
                     int32_t* counts, int32_t* offsets, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * schedule_tiles: row tiles over expert-sorted rows from offsets [E+1].
 * SCHEDULED (MLX PR 4567 Proposed changes, schedule_row_tile): for e ascending
 *   and j < ceil(c_e/bm): tile = (offsets[e] + j*bm, e, min(bm, c_e - j*bm)).
 * NAIVE: tile t = (t*bm, -1, min(bm, P - t*bm)).
 * tiles [cap, 3] int32 (row_start, expert, valid_rows); *n_tiles (device int32)
 * receives the tile count.  cap must be >= the upper bound
 * ceil(P/bm) + min(E, P) (P = offsets[E] is not known on the host: pass P_max).
 */
int moegq_schedule_tiles(const int32_t* offsets, int64_t E, int64_t P_max, int bm, int tile_mode,
                         int32_t* tiles, int64_t cap, int32_t* n_tiles, void* stream);

/* rms_norm: out = bf16( x / sqrt(mean(x^2) + eps) * w ), x [M, K], w [K]
 * (MLX PR 4787 benchmark script, mx.fast.rms_norm). */
int moegq_rms_norm(const void* x, const void* w, int64_t M, int64_t K, float eps, void* out,
                   void* stream);

/*
 * gather_mm: out[j] = bf16( x[lhs[j]] . w[rhs[j]]^T ) with unquantized bf16
 * expert matrices (MLX PR 4567, "[Metal] Gather mm improvement": the
 * expert-aware row-tile schedule is built for this operation).  x [X, M, K]
 * bf16; w [E, N, K] bf16 (a linear layer's weights; the product takes their
 * transpose); lhs_indices [P] int32 or NULL (then the x batch of pair j is
 * j / lhs_div); rhs_indices [P] int32 expert ids; out [P, M, N] bf16 in pair
 * order.  sorted_indices = 1 promises rhs ascending: with M = 1, P >= 64 and
 * K a multiple of 128 the pairs run as per-expert 64-row tiles on the matrix
 * cores (one K pass per tile).  M = 1 otherwise: one pass per pair over its
 * expert's rows.  M > 1: per-pair tiles on the matrix cores (K a multiple of
 * 128, else MOEGQ_ERR_UNSUPPORTED).  K must be a multiple of 8; N * K and
 * X * M * K below 2^31.  workspace: moegq_workspace_bytes(MOEGQ_OP_GATHER_MM,
 * P, E, M, 0) bytes.
 */
int moegq_gather_mm(const void* x, int64_t X, int64_t M, int64_t K, const void* w, int64_t E, int64_t N,
                    const int32_t* lhs_indices, int64_t lhs_div, const int32_t* rhs_indices, int64_t P,
                    int sorted_indices, void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * route: the MoE block's routing from its router logits, which produces the
 * idx and scores the expert path takes (MTPLX PR 558 Change: the one-kernel
 * block keeps the unfused block's routing ahead of the sorted experts and the
 * combine).  logits [T, E] fp32 row-major (finite).  idx [T, top_k] int32:
 * the top_k experts by logit, ties to the lower id, stored in ascending expert
 * id.  scores [T, top_k] bf16: each chosen expert's softmax probability over
 * all E logits, evaluated in float64 with the largest logit subtracted, not
 * renormalised, rounded to fp32 and then to bf16.  1 <= E <= 1024 and
 * 1 <= top_k <= min(E, 64) (else MOEGQ_ERR_SHAPE); T = 0 launches nothing.
 */
int moegq_route(const void* logits, int64_t T, int64_t E, int64_t top_k, int32_t* idx, void* scores,
                void* stream);

/* sigmoid_gate: out = bf16( sigmoid(z[t]) * s[t, :] ), z [T] (stride z_stride) bf16,
 * s [T, H] bf16: the shared expert's sigmoid gate (MTPLX PR 558 Summary). */
int moegq_sigmoid_gate(const void* s, const void* z, int64_t z_stride, int64_t T, int64_t H,
                       void* out, void* stream);

/* kv_feed: out = bf16( q + bf16(k[:, 0] + v[:, 0]) ), q [M, Nq], k [M, Nk], v [M, Nv]
 * (MLX PR 4787 benchmark script: o is applied to q + (k[:, :1] + v[:, :1])). */
int moegq_kv_feed(const void* q, const void* k, const void* v, int64_t M, int64_t Nq,
                  int64_t Nk, int64_t Nv, void* out, void* stream);
/* kv_feed with row strides (element counts): q row m at q + m*ldq (ldq >= Nq),
 * k[m, 0] at k + m*ldk, v[m, 0] at v + m*ldv; out [M, Nq] bf16.  With one
 * stacked product qkv [M, Nq + Nk + Nv]: q = qkv, k = qkv + Nq, v = qkv + Nq + Nk,
 * every stride Nq + Nk + Nv. */
int moegq_kv_feed_ld(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                     int64_t M, int64_t Nq, void* out, void* stream);

/*
 * selfcheck: runs the fused and the unfused combine on seeded data of 128
 * rows, top-8, hidden 2048 (MTPLX PR 558: the bitwise self-check lane at that
 * geometry) and compares them bit for bit.  Synchronizes.  Returns MOEGQ_OK or
 * MOEGQ_ERR_SELFCHECK.  workspace: moegq_workspace_bytes(MOEGQ_OP_SELFCHECK,...).
 * Setting the environment variable MOEGQ_FORCE_SELFCHECK_FAIL=1 makes it
 * report a failure (for testing the fallback).  The result is kept per
 * device: after a failure moegq_moe_prefill runs the unfused tail and
 * moegq_moe_combine / moegq_moe_combine_gated return MOEGQ_ERR_SELFCHECK
 * (MTPLX PR 558 Change and Tests: a failed check turns the one-kernel route
 * off for the process); a later passing check turns it back on.
 */
int moegq_selfcheck(void* workspace, size_t workspace_bytes, void* stream);
/* selfcheck_state: the current device's last self-check result: 0 not run,
 * 1 passed, 2 failed.  Host-only. */
int moegq_selfcheck_state(void);

/*
 * Measured ceilings (diagnostics, not part of the MoE path): the two plain
 * kernels that the path's results are stated against besides the published
 * peaks.
 * probe_stream_read: reads every byte of buf [bytes] (bytes a multiple of 16,
 *   buf 16-byte aligned) once with 128-bit loads, blocks workgroups of 256
 *   threads striding over the buffer; sink: 4 bytes of device memory that the
 *   kernel only writes when the data XOR to a sentinel (keeps the loads live).
 * probe_mfma_bf16: blocks workgroups of 4 waves; each wave runs iters rounds
 *   of 8 independent v_mfma_f32_16x16x32_bf16 on registers, i.e.
 *   blocks * 4 * iters * 8 * 16384 flops; out: 4 bytes of device memory,
 *   written only on a sentinel value.
 * Both asynchronous on `stream`; errors MOEGQ_ERR_SHAPE, _NULL_ARG, _ALIGN.
 */
int moegq_probe_stream_read(const void* buf, int64_t bytes, void* sink, int blocks, void* stream);
int moegq_probe_mfma_bf16(int iters, int blocks, void* out, void* stream);

/* validate_indices: synchronizing debug check that every idx[i] (i < n,
 * int32) lies in [0, E); if `sorted` also that idx is non-decreasing.
 * workspace: 4 bytes of device memory.  Returns MOEGQ_OK or MOEGQ_ERR_INDEX. */
int moegq_validate_indices(const int32_t* idx, int64_t n, int64_t E, int sorted,
                           int32_t* workspace, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOEGQ_H */
