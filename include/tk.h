/*
 * tk.h -- C ABI of the MoE routing hot path for AMD Instinct MI355X (gfx950).
 *
 * Four stream-ordered steps of a DeepSeek-V3-style MoE layer's token routing:
 *
 *   tk_route         top-k expert gating and scoring        (logits -> idx, w)
 *   tk_map           token-to-expert mapping                (idx -> counts,
 *                                                            offsets, pos)
 *   tk_map_aligned   the same with every expert segment     (idx -> counts,
 *                    padded for a grouped GEMM                 offsets, pos)
 *   tk_expand_quant  expand into expert-contiguous rows,    (x -> rows [+ FP8
 *                    optionally fused 1x128 FP8 E4M3 quant    scales])
 *   tk_reduce        weighted combine back to tokens        (rows, w -> out)
 *   tk_reduce_dense  the same, faster when (nearly) every
 *                    slot has a row
 *
 * quantisation at other granularities (power-of-two scales, 128x128 tiles,
 * per channel, FP4),
 *
 *   tk_quant         bf16 matrix -> FP8 / FP4 codes + scales
 *
 * per-expert load statistics and the load-balance loss,
 *
 *   tk_balance_loss  f, P and sum_e f_e P_e of one batch    (logits, idx ->
 *                                                             f, P, loss)
 *
 * the next step after an expert's first grouped GEMM,
 *
 *   tk_swiglu_quant  SwiGLU + 1x128 FP8 quantisation        (rows -> codes,
 *                    (+ routing weight)                        scales)
 *   tk_swiglu_quant_t  the same plus the transposed layout  (rows -> codes,
 *                    (1x128 blocks along tokens)               scales, both
 *                                                              layouts)
 *   tk_silu_bf16     the SwiGLU gate factor g * sigmoid(g)  (bf16 -> fp32)
 *
 * plus tk_expert_standin, a dequantise-and-scale harness kernel that stands in
 * for the expert computation in end-to-end tests.
 *
 * The operations are the ones the pages list for TileKernels' moe/ module --
 * top-k gating and expert scoring, the token-to-expert mapping, the fused
 * expand and reduce, and the tensor-parallel mask ("刚刚！DeepSeek开源高性能GPU算子库
 * TileKernels", item moe/; "剛剛，DeepSeek開始頻繁更新：Tile Kernels、DeepEP V2",
 * feature list) -- with per-token FP8 quantisation from the quant/ module
 * (same pages) fused into the expand, at the DeepSeek-V3 shape with FP8
 * dispatch and BF16 combine ("剛剛，DeepSeek開始頻繁更新…", section 性能表現).
 * The top-k order and tie rule follow the gating listing on "DeepSeek 的 GPU
 * 内核帝国：从 TileLang DSL 到 Engram 条件记忆…", section 第三层：TileKernels,
 * subsection "MoE TopK 门控".
 *
 * Conventions for every call:
 *  - Pointers are device pointers owned by the caller (a HIP allocation, e.g.
 *    a torch tensor's storage).  The library allocates nothing, keeps no state
 *    between calls and never synchronises the host: every call enqueues
 *    kernels on `stream` and returns.  Calls are thread-safe.
 *  - Tensors are dense and row-major.  Pointers of vector-accessed tensors
 *    (noted per argument) must be 16-byte aligned.
 *  - Host-side argument checks run before anything is launched; a failed
 *    check returns TK_ERR_ARG (or TK_ERR_UNSUPPORTED for valid arguments the
 *    kernels do not implement) and launches nothing.  A HIP launch error
 *    returns TK_ERR_DEVICE.  tk_last_error() then describes the failure.
 *    The library never aborts or exits.
 *  - T == 0 (no tokens) is a valid no-op for every call that takes T, except
 *    tk_balance_loss, whose statistics are not defined without tokens.
 *  - Device data that breaks a call's contract (an expert id out of range, a
 *    row index beyond the capacity) never causes an out-of-bounds access:
 *    the affected route or row is skipped as documented per call.
 */
#ifndef TK_H
#define TK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tk_status;
#define TK_OK 0
#define TK_ERR_ARG (-1)          /* invalid arguments; nothing launched */
#define TK_ERR_UNSUPPORTED (-2)  /* valid but not implemented; nothing launched */
#define TK_ERR_DEVICE (-3)       /* HIP launch / runtime error */

/* Limits of this implementation. */
#define TK_MAX_EXPERTS 1024
#define TK_MAX_TOPK 32

/* Text of the last failure on the calling thread; owned by the library, valid
 * until the next tk_* call on that thread.  "" when the last call succeeded. */
const char* tk_last_error(void);

/* ------------------------------------------------------------------ route */
#define TK_SCORE_SOFTMAX 0
#define TK_SCORE_SIGMOID 1

typedef struct tk_route_opts {
    int32_t score;        /* TK_SCORE_SOFTMAX or TK_SCORE_SIGMOID */
    int32_t n_groups;     /* expert groups of E/n_groups consecutive experts;
                             1 = no group limiting */
    int32_t topk_groups;  /* groups kept per token (n_groups > 1) */
    int32_t group_topn;   /* a group's score is the sum of its group_topn
                             largest selection keys (n_groups > 1) */
    int32_t renormalize;  /* 1: weights of the k chosen experts are normalised
                             to sum to route_scale; 0: raw scores * scale */
    float route_scale;    /* final multiplier of the weights */
} tk_route_opts;

/*
 * tk_route -- top-k expert gating and scoring, one token per wavefront (two
 * per wavefront for T >= 12288 with 128 < E <= 256; the results are the same).
 *
 * Per token t (row t of logits):
 *  1. selection key per expert e (fp32):
 *       softmax: key = logit (softmax is increasing in the logit, so its top-k
 *                is the top-k of the logits);
 *       sigmoid: s = 1/(1+E(-x)) with a fixed fp32 evaluation of E(y) = e^y
 *                (Cody-Waite reduction by ln 2 in two parts, degree-7 Taylor
 *                polynomial in Horner form with fused multiply-adds, IEEE
 *                division), key = s + bias[e] (bias optional, selection only);
 *  2. if n_groups > 1: group score = fp32 sum (largest first) of the group's
 *     group_topn largest keys; the topk_groups best groups (ties -> lower
 *     group) stay eligible, the other groups' experts do not;
 *  3. k rounds of argmax over the eligible experts: largest key first, ties
 *     to the lower expert index (-0 == +0), each winner removed; round j
 *     writes slot j (the listing's rounds of max + min-index argmax);
 *  4. weights (fp32):
 *       sigmoid: w_j = s_j / (s_0 + ... + s_{k-1}) * route_scale (unbiased
 *                scores, sum in slot order), or s_j * route_scale;
 *       softmax: w_j = e^(x_j - x_0) / sum_i e^(x_i - x_0) * route_scale over
 *                the k chosen experts, or the softmax over all E experts
 *                times route_scale when renormalize == 0.
 *
 * logits   device, fp32 (T, E), 4-byte aligned; 16-byte aligned when E > 128
 *          and E % 4 == 0 (four experts per lane, read as one vector load).
 *          Finite values: for a token with a NaN or infinite logit the
 *          experts and weights are unspecified (a NaN may win or lose any
 *          comparison, and an expert may repeat), but every index written is
 *          in [0, E), so the map, expand and combine stay within their buffers
 * bias     device, fp32 (E) or NULL; sigmoid only; aligned as logits
 * T        tokens, >= 0
 * E        experts, 1..TK_MAX_EXPERTS
 * k        experts per token, 1..min(E, TK_MAX_TOPK)
 * opts     host pointer; n_groups must divide E, topk_groups in 1..n_groups,
 *          group_topn in 1..E/n_groups, topk_groups*E/n_groups >= k.  Group
 *          limiting additionally needs E/n_groups to be a multiple of the
 *          experts held per lane (ceil(E/64) rounded up to a power of two) and
 *          the lanes per group a power of two, else TK_ERR_UNSUPPORTED.
 * topk_idx device, int32 (T, k) out: chosen experts, descending key order
 * topk_w   device, fp32 (T, k) out: weights, slot-aligned with topk_idx
 */
tk_status tk_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                   const tk_route_opts* opts, int32_t* topk_idx, float* topk_w,
                   hipStream_t stream);

/* -------------------------------------------------------------------- map */
/* Bytes of device workspace tk_map needs for T tokens, k slots and
 * n_local = local_end - local_begin experts (0 for T == 0). */
size_t tk_map_workspace_bytes(int32_t T, int32_t k, int32_t n_local);

/*
 * tk_map -- token-to-expert mapping with a local-expert mask: the
 * token-to-expert mapping and tensor-parallel mask operations of
 * TileKernels' moe/ module ("刚刚！DeepSeek开源高性能GPU算子库TileKernels",
 * item moe/), the mask read as the experts one expert-parallel rank owns.
 *
 * Route (t, j) is local when local_begin <= topk_idx[t,j] < local_end (the
 * experts one expert-parallel rank owns; [0, E) keeps every route).  An
 * expert id repeated within one token's row is routed only at its first
 * occurrence; ids outside [0, E) are never local.
 *   counts[e]   = number of local routes to expert local_begin + e
 *   offsets     = exclusive prefix sum of counts, offsets[n_local] = R
 *   pos[t,j]    = offsets[e] + number of tokens t' < t routed to e: rows are
 *                 expert-contiguous and, within an expert, in token order
 *                 (stable); -1 for a route that is not local
 *   row_src[r]  = token of expanded row r, for r < R (optional)
 * Not-local routes keep their weights (nothing is renormalised), so partial
 * combines of different ranks add up to the full combine.  Bit-exact and
 * deterministic: no result depends on the order of atomics.
 *
 * topk_idx  device, int32 (T, k)
 * T, k      T >= 0, 1 <= k <= TK_MAX_TOPK
 * E         total experts, 1..TK_MAX_EXPERTS; 0 <= local_begin < local_end <= E
 * counts    device, int32 (n_local) out
 * offsets   device, int32 (n_local + 1) out
 * pos       device, int32 (T, k) out
 * row_src   device, int32 (T * k) out, or NULL; entries r >= R are untouched
 * workspace device, >= tk_map_workspace_bytes(T, k, n_local) bytes, 16-byte
 *           aligned; scratch, contents on entry ignored
 */
tk_status tk_map(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                 int32_t local_begin, int32_t local_end, int32_t* counts, int32_t* offsets,
                 int32_t* pos, int32_t* row_src, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * tk_map_aligned -- tk_map with every expert's segment padded for an
 * M-blocked grouped GEMM (the expert-contiguous layout a grouped GEMM such as
 * DeepGEMM's m-grouped kernel reads, "DeepSeek 的 GPU 内核帝国…", section
 * 第二层：DeepGEMM, kernel list; the new GEMM layout of DeepEP V2 in
 * "剛剛，DeepSeek開始頻繁更新：Tile Kernels、DeepEP V2", EPv2 features):
 *   offsets[0] = 0, offsets[e+1] = offsets[e] + roundup(counts[e], align)
 *   pos[t,j]   = offsets[e] + number of tokens t' < t routed to e (or -1)
 *   row_src[r] = source token of row r, -1 for a padding row, r < offsets[n_local]
 * so every segment starts at a multiple of align.  align = 1 is tk_map.  The
 * padded row count offsets[n_local] is at most T*k + n_local*(align-1), which
 * is the capacity callers allocate for row_src and the expanded rows; that
 * bound must fit in int32.  Padding rows are never written by
 * tk_expand_quant nor read by tk_reduce.
 *
 * align  >= 1; the other arguments as for tk_map
 */
tk_status tk_map_aligned(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                         int32_t local_begin, int32_t local_end, int32_t align, int32_t* counts,
                         int32_t* offsets, int32_t* pos, int32_t* row_src, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * tk_map_noalloc -- tk_map for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments minus the workspace, the same checks,
 * results and errors.  The count matrix lives in a device array of
 * TK_MAP_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; the call allocates nothing.  Sizes whose workspace
 * (tk_map_workspace_bytes) exceeds that array return TK_ERR_ARG.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * concurrent streams, or from several host threads) race and must be
 * serialised by the caller.  The stream must belong to the current device
 * (else TK_ERR_ARG); the first call on a device looks the array's address up
 * there.
 */
#define TK_MAP_NOALLOC_SCRATCH_BYTES (1 << 20)
tk_status tk_map_noalloc(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                         int32_t local_begin, int32_t local_end, int32_t* counts,
                         int32_t* offsets, int32_t* pos, int32_t* row_src, hipStream_t stream);

/* ----------------------------------------------------------------- expand */
#define TK_EXPAND_BF16 0            /* rows are bitwise copies of the token */
#define TK_EXPAND_FP8_E4M3_1X128 1  /* rows are 1x128-block FP8 E4M3 codes */

/*
 * tk_expand_quant -- gather tokens into expert-contiguous rows: the fused
 * expand of TileKernels' moe/ module with the per-token FP8 quantisation of
 * its quant/ module fused in ("刚刚！DeepSeek开源高性能GPU算子库TileKernels",
 * items moe/ and quant/), the FP8 dispatch of the DeepSeek-V3 test shape
 * ("剛剛，DeepSeek開始頻繁更新：Tile Kernels、DeepEP V2", section 性能表現).
 *
 * For every route with 0 <= pos[t,j] < rows_capacity, row pos[t,j] of `out`
 * receives token t (routes outside that range are skipped).  Each token is
 * read from HBM once and written to all its rows.
 * TK_EXPAND_FP8_E4M3_1X128: per token and block b of 128 columns,
 *   amax = max(max |x|, 1e-4), scale = RN32(amax / 448),
 *   q = E4M3(RN32(x / scale)) -- OCP E4M3FN, round to nearest even, sign kept;
 *   scales[row, b] = scale for every row of the token.
 * The FP8 mode assumes finite x: a block holding a NaN or an infinity gets
 * unspecified codes and scale (the bf16 mode copies any bits).  Where the
 * rows go never depends on the values.
 *
 * x_bf16        device, bf16 (T, H), 16-byte aligned
 * T, H, k       T >= 0; H > 0 with H % 8 == 0 (bf16) or H % 128 == 0 (FP8)
 * pos           device, int32 (T, k) (as written by tk_map)
 * mode          TK_EXPAND_BF16 or TK_EXPAND_FP8_E4M3_1X128
 * out           device, (rows_capacity, H) of bf16 or E4M3 bytes, 16-byte aligned
 * scales        device, fp32 (rows_capacity, H/128), FP8 mode only (else NULL)
 * rows_capacity rows available in out (and scales), >= 0
 */
tk_status tk_expand_quant(const void* x_bf16, int32_t T, int32_t H, int32_t k,
                          const int32_t* pos, int32_t mode, void* out, float* scales,
                          int64_t rows_capacity, hipStream_t stream);

/* ----------------------------------------------------------------- reduce */
/*
 * tk_reduce -- weighted combine of expert outputs back to tokens: the fused
 * reduce of TileKernels' moe/ module ("刚刚！DeepSeek开源高性能GPU算子库
 * TileKernels", item moe/), the BF16 combine of the DeepSeek-V3 test shape
 * ("剛剛，DeepSeek開始頻繁更新：Tile Kernels、DeepEP V2", section 性能表現).
 *
 *   out[t, c] = bf16_RNE( fp32 fma chain over j = 0..k-1, in slot order, of
 *               topk_w[t,j] * y[pos[t,j], c] ), starting from +0,
 * skipping routes with pos < 0 or pos >= rows.  A token without such a route
 * gets a row of +0.
 *
 * y_bf16  device, bf16 (rows, H), 16-byte aligned
 * rows    rows in y, >= 0
 * pos     device, int32 (T, k)
 * topk_w  device, fp32 (T, k)
 * T, k, H T >= 0; 1 <= k <= TK_MAX_TOPK; H > 0, H % 8 == 0
 * out     device, bf16 (T, H) out, 16-byte aligned
 */
tk_status tk_reduce(const void* y_bf16, int64_t rows, const int32_t* pos, const float* topk_w,
                    int32_t T, int32_t k, int32_t H, void* out_bf16, hipStream_t stream);

/*
 * tk_reduce_dense -- tk_reduce for dense routings: the same arguments,
 * checks, errors and bit-identical results.  A workgroup combines up to 16
 * consecutive tokens, holds the results in registers and stores their rows
 * as one burst after all of its reads; the workgroups run in rounds of one
 * per compute unit with the tokens spread evenly over them, and for large
 * rows (a round of at least 480 MiB) each round is a launch of its own on
 * `stream`.  This pays off when (nearly) every
 * slot has a row -- no local-expert mask, as in a single-GPU layer -- and
 * loses to tk_reduce when most slots are masked (one GPU's share of an
 * expert-parallel layer).  It takes tk_reduce's kernel itself for small T
 * (fewer than one workgroup of tokens per compute unit), short rows
 * (H <= 1536), runtime k (k not in {1, 2, 4, 6, 8}) and H > 114688.
 */
tk_status tk_reduce_dense(const void* y_bf16, int64_t rows, const int32_t* pos,
                          const float* topk_w, int32_t T, int32_t k, int32_t H, void* out_bf16,
                          hipStream_t stream);

/*
 * tk_swiglu_quant_t -- the transposing form of the same fusion (SwiGLU + FP8
 * quantisation + matrix transpose in one pass, "刚刚！DeepSeek开源高性能GPU算子库
 * TileKernels", item quant/): from one read of h it writes both
 *   out, scales      exactly as tk_swiglu_quant (1x128 blocks along each row)
 *   out_t, scales_t  the transpose a^T (I, rows) quantised with 1x128 blocks
 *                    along its rows -- 128 consecutive rows of one column of a:
 *                    scales_t[c, b] = RN32(max(max |a[128b..128b+127, c]|,
 *                    1e-4) / 448), out_t[c, r] = E4M3(RN32(a[r, c] /
 *                    scales_t[c, r/128]))
 * for all `rows` rows (a host count; no device-side row count).
 *
 * h_bf16        device, bf16 (rows, 2*I), 16-byte aligned
 * rows          a multiple of 128, >= 0
 * I             a positive multiple of 128
 * row_src, pos, topk_w, T, k   as for tk_swiglu_quant (all NULL: unweighted)
 * out           device, E4M3 (rows, I); scales: fp32 (rows, I/128)
 * out_t         device, E4M3 (I, rows); scales_t: fp32 (I, rows/128)
 *               (out and out_t 16-byte aligned)
 */
tk_status tk_swiglu_quant_t(const void* h_bf16, int64_t rows, int32_t I, const int32_t* row_src,
                            const int32_t* pos, const float* topk_w, int32_t T, int32_t k,
                            void* out, float* scales, void* out_t, float* scales_t,
                            hipStream_t stream);

/*
 * tk_silu_bf16 -- the gate factor of the fusion on its own: out[i] =
 * RN32(g[i] * sigmoid(g[i])) with the pinned fp32 sigmoid, for bf16 g.  It
 * runs the SwiGLU kernels' sigmoid lookup (the table the build tabulates
 * from the pinned steps), so a caller can check that table on every bf16
 * value or use the factor alone.
 *
 * g_bf16   device, bf16 (n), 2-byte aligned
 * out      device, fp32 (n), 4-byte aligned
 * n        >= 0 (0: nothing is launched)
 */
tk_status tk_silu_bf16(const void* g_bf16, int64_t n, float* out, hipStream_t stream);

/* --------------------------------------------- quantisation granularities */
#define TK_QUANT_FP8_1X128 0        /* per-token 1x128 blocks, scale = amax/448 */
#define TK_QUANT_FP8_1X128_POW2 1   /* 1x128 blocks, power-of-two scales */
#define TK_QUANT_FP8_128X128 2      /* one scale per 128x128 tile */
#define TK_QUANT_FP8_PER_CHANNEL 3  /* one scale per column */
#define TK_QUANT_FP4_1X32 4         /* E2M1, 1x32 blocks, power-of-two scales */

/* Bytes of device workspace tk_quant needs (non-zero only for per-channel). */
size_t tk_quant_workspace_bytes(int64_t rows, int32_t cols, int32_t mode);

/*
 * tk_quant -- quantise a bf16 matrix x (rows, cols) at one of the
 * granularities of TileKernels' quant/ module ("刚刚！DeepSeek开源高性能GPU算子库
 * TileKernels", item quant/: per-token, per-block and per-channel FP8;
 * "剛剛，DeepSeek開始頻繁更新：Tile Kernels、DeepEP V2", feature list: FP8 and FP4
 * conversion).  amax is the block's largest |x| (bf16 -> fp32 exact), clamped
 * to >= 1e-4.  FP8 codes are OCP E4M3FN of RN32(x / scale), nearest even,
 * sign kept, saturating at 448.
 *   TK_QUANT_FP8_1X128       blocks of 128 columns of one row; scale =
 *                            RN32(amax/448) -- tk_expand_quant's codec.
 *                            out (rows, cols), scales (rows, cols/128)
 *   TK_QUANT_FP8_1X128_POW2  the same blocks; scale = the smallest power of
 *                            two with 448*scale >= amax (UE8M0-representable)
 *   TK_QUANT_FP8_128X128     tiles of 128 rows x 128 columns (the last tile
 *                            row may be shorter); scale = RN32(amax/448).
 *                            out (rows, cols), scales (ceil(rows/128), cols/128)
 *   TK_QUANT_FP8_PER_CHANNEL one block per column, over all rows; scale =
 *                            RN32(amax/448).  out (rows, cols), scales (cols);
 *                            needs tk_quant_workspace_bytes of workspace
 *   TK_QUANT_FP4_1X32        FP4 E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 *                            nearest, ties to the even code, sign kept,
 *                            saturating at 6) of x / scale over blocks of 32
 *                            columns; scale = 2^(floor(log2 amax) - 2) (the
 *                            OCP MX shared-exponent rule for E2M1).  Two
 *                            codes per byte, column 2i in the low nibble:
 *                            out (rows, cols/2); scales (rows, cols/32), fp32
 *                            powers of two.
 * cols must be a positive multiple of 128 (FP8 block and tile modes), 8
 * (per-channel) or 32 (FP4).  Inputs are finite.
 *
 * x_bf16, out, scales  device, 16-byte aligned
 * workspace            device, 16-byte aligned, per-channel only (else NULL)
 */
tk_status tk_quant(const void* x_bf16, int64_t rows, int32_t cols, int32_t mode, void* out,
                   float* scales, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------ load balance */
/* Bytes of device workspace tk_balance_loss needs for T tokens and E experts. */
size_t tk_balance_workspace_bytes(int32_t T, int32_t E);

/*
 * tk_balance_loss -- per-expert load statistics and the load-balance loss of
 * one batch: the load-balancing loss computation of TileKernels' moe/
 * module ("刚刚！DeepSeek开源高性能GPU算子库TileKernels", item moe/), in the form
 * DeepSeek-V3 trains with:
 *   count_e = number of (t, j) with topk_idx[t,j] = e (ids outside [0,E) ignored)
 *   f[e]    = E / (k*T) * count_e             (1 everywhere for an even load)
 *   P[e]    = (1/T) sum_t p_{t,e}, with p_{t,.} the token's scores over all E
 *             experts normalised to sum 1: sigmoid scores (the pinned sigmoid
 *             of tk_route, no bias) divided by their sum, or the softmax
 *   loss[0] = sum_e f[e] * P[e]               (the caller applies its weight)
 * fp32 sums in a fixed order (deterministic); the loss is accumulated in fp64.
 *
 * logits     device, fp32 (T, E), the router logits tk_route ranked
 * topk_idx   device, int32 (T, k), the experts tk_route chose
 * T, E, k    T >= 1; 1 <= E <= TK_MAX_EXPERTS; 1 <= k <= TK_MAX_TOPK
 * score      TK_SCORE_SIGMOID or TK_SCORE_SOFTMAX
 * f, P       device, fp32 (E) out;  loss: device, fp32 (1) out
 * workspace  device, >= tk_balance_workspace_bytes(T, E) bytes, 4-byte aligned;
 *            scratch, contents on entry ignored
 */
tk_status tk_balance_loss(const float* logits, const int32_t* topk_idx, int32_t T, int32_t E,
                          int32_t k, int32_t score, float* f, float* P, float* loss,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------- SwiGLU + FP8 quant */
/*
 * tk_swiglu_quant -- SwiGLU activation fused with per-token 1x128 FP8 E4M3
 * quantisation of expert rows, optionally applying each row's routing weight:
 * the SwiGLU and FP8 quantisation fusion of TileKernels' quant/ module
 * ("刚刚！DeepSeek开源高性能GPU算子库TileKernels", item quant/; "剛剛，DeepSeek
 * 開始頻繁更新：Tile Kernels、DeepEP V2", feature list) and the weighted
 * SwiGLU-to-FP8 helper of the DeepGEMM kernel list ("DeepSeek 的 GPU 内核帝国…",
 * section 第二层：DeepGEMM).
 *
 * Per row r < n (n = *n_rows clamped to [0, rows_capacity], or rows_capacity
 * when n_rows is NULL) and column c < I, in fp32 with one IEEE rounding per
 * step:
 *   g = h[r, c], u = h[r, I + c];  s = 1/(1 + E(-g)) (the pinned sigmoid of
 *   tk_route);  a = RN(RN(g*s)*u);  weighted: a = RN(a * w_r)
 * then per 128-column block: amax = max(max |a|, 1e-4), scale = RN(amax/448),
 * out[r, c] = E4M3(RN(a / scale)) (OCP E4M3FN, nearest even, sign kept),
 * scales[r, c/128] = scale.  Rows r >= n are not written.
 * A NaN or infinite h, or an activation that overflows fp32 (|g*u| beyond
 * ~3.4e38), gives its block unspecified codes and scale.
 * Weighted when row_src, pos and topk_w are all given (all NULL: unweighted):
 * w_r = topk_w[t, j] for t = row_src[r] and the slot j with pos[t, j] == r
 * (as written by tk_map), 0 if there is none.
 *
 * h_bf16        device, bf16 (rows_capacity, 2*I): gate columns then up
 *               columns; 16-byte aligned
 * rows_capacity rows of h, out and scales, >= 0
 * n_rows        device, one int32 (e.g. offsets + n_local from tk_map), or NULL
 * I             output columns, a positive multiple of 128
 * row_src, pos, topk_w, T, k
 *               device int32 (rows_capacity), int32 (T, k), fp32 (T, k): the
 *               map and the routing weights; or all NULL
 * out           device, E4M3 bytes (rows_capacity, I), 16-byte aligned
 * scales        device, fp32 (rows_capacity, I/128)
 */
tk_status tk_swiglu_quant(const void* h_bf16, int64_t rows_capacity, const int32_t* n_rows,
                          int32_t I, const int32_t* row_src, const int32_t* pos,
                          const float* topk_w, int32_t T, int32_t k, void* out, float* scales,
                          hipStream_t stream);

/* -------------------------------------------------------- test harness */
/*
 * tk_expert_standin -- stand-in for the expert computation in end-to-end
 * tests of one expert-parallel rank: dequantise each FP8 row and scale it,
 *   y[r, c] = bf16_RNE( RN32( RN32(dec(xq[r, c]) * scales[r, c/128]) * mult ) )
 * for r < *n_rows (read on the device, e.g. offsets + n_local from tk_map,
 * clamped to rows_capacity).  Not part of the routing path.
 *
 * xq      device, E4M3 (rows_capacity, H), 16-byte aligned
 * scales  device, fp32 (rows_capacity, H/128)
 * n_rows  device, one int32
 * H       H > 0, H % 128 == 0
 * y_bf16  device, bf16 (rows_capacity, H) out, 16-byte aligned
 */
tk_status tk_expert_standin(const uint8_t* xq, const float* scales, const int32_t* n_rows,
                            int64_t rows_capacity, int32_t H, float mult, void* y_bf16,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TK_H */
