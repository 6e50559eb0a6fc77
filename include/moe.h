/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts layer of a prefill
 * step: router + top-k gating, dispatch (permute) by expert, per-expert SwiGLU
 * FFN as a grouped GEMM, and the weighted combine back to token order.
 *
 * Where the operation is defined:
 *  - "ASAP: A DiSaggregated and Asynchronous Inference System for MoE
 *    Prefill", section 3.4.2: the MoE kernel is a grouped matrix
 *    multiplication (GMM) whose left operand is the hidden states and whose
 *    right operand is the expert weights of the layer.
 *  - same page, Table 1 (K experts per token out of E_total, hidden size H) and
 *    Table 2 with section 3.2 (the dispatch carries expert IDs, token counts
 *    per expert and the hidden states; the combine returns the expert results
 *    per token and choice).
 *  - "Memory-Compute Disaggregation ... AFD Architecture Analysis", section 3:
 *    the FFN side receives hidden states plus batch metadata, performs gated
 *    routing and expert computation, and returns the layer output.
 *  - same page, section 5 (MegaMoE operator fusion): routing/movement and the
 *    expert GEMM are separable stages; this library exposes each stage and
 *    the composed layer.
 * The pages do not write the formulas; the exact arithmetic (scores, group
 * limit, renormalisation, SwiGLU, fp8 block scales) is stated at each entry
 * point below.
 *
 * Conventions (all entry points):
 *  - Every array argument is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or keeps memory; scratch space is the
 *    caller's workspace `ws` of at least moe_workspace_bytes() bytes, 256-byte
 *    aligned.
 *  - Every call is asynchronous on `stream` (a hipStream_t, NULL = the null
 *    stream).  Nothing is read back to the host and no call synchronises.
 *    Buffers must stay alive until the stream has executed the work.
 *  - Arguments are checked on the host before anything is enqueued; an error
 *    enqueues nothing.  A HIP launch error returns MOE_ERR_HIP; a device fault
 *    shows up at the caller's next synchronisation.  moe_last_error() gives
 *    the message of the last failure on the calling thread.
 *  - Inputs are never written.  Outputs are written in full (padding included).
 *  - T == 0 is valid: the call returns MOE_OK and enqueues nothing.
 *  - Matrices are [out][in] row-major (the reduction index is contiguous):
 *    w_router [E][H]; w_gate, w_up [E][I][H]; w_down [E][H][I]; the shared
 *    expert sh_gate, sh_up [I_shared][H], sh_down [H][I_shared].
 *  - Pointers are 16-byte aligned; H and I are multiples of 8 (bf16/fp32) or
 *    of 128 (fp8).
 *  - The library is stateless: concurrent calls on different streams need
 *    different workspaces and outputs.
 */
#ifndef EXPERT_LAYER_AMD_MOE_H
#define EXPERT_LAYER_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* a size, pointer or option is out of range */
    MOE_ERR_UNSUPPORTED = 2, /* a valid combination this library does not implement */
    MOE_ERR_WORKSPACE = 3,   /* ws is NULL, misaligned or smaller than required */
    MOE_ERR_HIP = 4          /* the HIP runtime reported an error at enqueue */
} moe_status;

typedef enum moe_dtype {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    MOE_FP8_E4M3 = 2, /* OCP e4m3: bias 7, max 448, S.1111.111 = NaN, no inf */
    MOE_FP4_E2M1 = 3  /* expert weights only: OCP MX FP4 (E2M1) codes, two a byte
                         (the even element in the low nibble), one E8M0 scale
                         byte per 32 consecutive elements of a row */
} moe_dtype;

typedef enum moe_score_fn { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;
typedef enum moe_group_score { MOE_GROUP_TOP2_SUM = 0, MOE_GROUP_MAX = 1 } moe_group_score;

typedef enum moe_layout {
    MOE_LAYOUT_ROWMAJOR = 0, /* [out][in] row-major, the reduction index contiguous */
    MOE_LAYOUT_TILED = 1,    /* weights: the bf16 or e4m3 layout moe_tile_weights writes; x_perm: bf16 tiled rows */
    MOE_LAYOUT_INDEXED = 2   /* x_layout only: no x_perm; the FFN reads x through row_src */
} moe_layout;

typedef enum moe_stage {
    MOE_STAGE_ROUTE = 0,
    MOE_STAGE_PERMUTE = 1,
    MOE_STAGE_FFN = 2,
    MOE_STAGE_LAYER = 3
} moe_stage;

/* Problem statement of one MoE layer call.
 *   T            tokens in the batch (rows of x)
 *   H            hidden size
 *   E            routed experts (ASAP's E_total; not its EP degree)
 *   k            experts chosen per token (ASAP's K), 1 <= k <= min(E, 32)
 *   I            intermediate size of a routed expert
 *   n_groups     expert groups for group-limited routing (1 = none); E % n_groups == 0
 *   topk_groups  groups kept per token (1 <= topk_groups <= n_groups)
 *   score_fn     MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID
 *   group_score  MOE_GROUP_TOP2_SUM or MOE_GROUP_MAX
 *   renormalize  1: the k weights are divided by their sum
 *   routed_scale factor applied to the k weights after renormalisation
 *   has_shared   1: a shared expert (weight 1) is added to every token
 *   I_shared     intermediate size of the shared expert
 *   act_dtype    x dtype (MOE_F32, MOE_BF16, or MOE_FP8_E4M3 for the grouped FFN)
 *   w_dtype      expert weight dtype: equal to act_dtype; or MOE_FP8_E4M3
 *                or MOE_FP4_E2M1 (MXFP4) with act_dtype MOE_BF16
 *                ("low-precision experts": moe_layer quantises x per token
 *                with moe_quantize_fp8's rule and runs the experts on e4m3
 *                rows; moe_grouped_ffn refuses this pair -- call it on the
 *                quantised rows with act_dtype = MOE_FP8_E4M3); or
 *                MOE_FP4_E2M1 with act_dtype MOE_FP8_E4M3 (grouped FFN).
 *                e4m3 and MXFP4 weights need H, I (and I_shared) to be
 *                multiples of 128 up to 16384.
 *   y_dtype      dtype of the per-row expert outputs (y_rows, y_shared):
 *                MOE_F32 or MOE_BF16
 *   out_dtype    dtype of the layer output: MOE_F32 or MOE_BF16
 *   m_tile       row padding of each expert segment produced by moe_permute
 *                (1 = no padding; 0 = library default, 1)
 *   x_layout     layout of x_perm between moe_permute and moe_grouped_ffn:
 *                MOE_LAYOUT_ROWMAJOR: [moe_max_rows][H] in act_dtype;
 *                MOE_LAYOUT_TILED (bf16, m_tile a multiple of 16): the rows
 *                in 1 KiB blocks of 16 rows x 32 columns, block (rb, ks) at
 *                byte (rb * KS + ks) * 1024 with KS = ceil(H / 32), the 16-byte
 *                chunk c (columns 8c .. 8c+7) of block row r at byte
 *                (r * 4 + (c ^ s(r))) * 16, s(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1),
 *                zero padded; R16 = roundup(moe_max_rows, 16) rows, followed,
 *                when has_shared, by the same layout of x's T rows (padded to
 *                16) that the shared expert reads;
 *                MOE_LAYOUT_INDEXED (bf16 or e4m3, x under 2 GiB): x_perm is
 *                not materialised -- moe_permute writes the maps only and
 *                moe_grouped_ffn reads dispatched row r from x itself (e4m3:
 *                and its scale from x_scale [T][H/128]), at token
 *                row_src[r] / k;
 *                moe_x_perm_bytes gives the size (0 when indexed).
 * E <= 1024. */
typedef struct moe_cfg {
    int32_t T, H, E, k, I;
    int32_t n_groups, topk_groups;
    int32_t score_fn, group_score, renormalize;
    float routed_scale;
    int32_t has_shared, I_shared;
    int32_t act_dtype, w_dtype, y_dtype, out_dtype;
    int32_t m_tile;
    int32_t x_layout;
} moe_cfg;

/* Expert weights.  For fp8 weights the s_* arrays hold one fp32 scale per
 * 128 x 128 block: s_gate, s_up [E][I/128][H/128]; s_down [E][H/128][I/128]
 * (dequantised weight = e4m3 value * block scale); NULL otherwise.  For
 * MXFP4 weights (w_dtype MOE_FP4_E2M1, the OCP Microscaling format that
 * gfx950's scaled MFMA reads; the 4-bit expert weights of the DWDP page,
 * appendix A4) the matrices are packed codes w_gate, w_up [E][I][H/2],
 * w_down [E][H][I/2] and the s_* pointers are uint8_t E8M0 scales, one per
 * 32 consecutive elements of a row: s_gate, s_up [E][I][H/32], s_down
 * [E][H][I/32] (dequantised weight = E2M1 value * 2^(scale - 127)).  sh_* are
 * the shared expert's matrices (NULL when has_shared == 0), sh_s_* their
 * scales (low-precision experts only: fp8 [I_shared/128][H/128] for gate
 * and up, [H/128][I_shared/128] for down; MXFP4 [I_shared][H/32] and
 * [H][I_shared/32]).
 * layout MOE_LAYOUT_ROWMAJOR: the matrices as above.  layout MOE_LAYOUT_TILED
 * (bf16 or e4m3 weights): w_gate and sh_gate point to the gate+up matrices and
 * w_down and sh_down to the down matrices that moe_tile_weights writes,
 * rearranged into the order in which the GEMMs load MFMA operands (an internal
 * layout: write it with moe_tile_weights only); w_up and sh_up are unused
 * (NULL); e4m3 block scales keep their row-major arrays.
 * bf16 needs H, I, I_shared <= 65536 and one expert's gate+up matrices
 * (padded: 2 * roundup(I, 128) x roundup(H, 32) bf16) under 2 GiB. */
typedef struct moe_weights {
    const void *w_gate, *w_up, *w_down;
    const float *s_gate, *s_up, *s_down;
    const void *sh_gate, *sh_up, *sh_down;
    int32_t layout;
    const float *sh_s_gate, *sh_s_up, *sh_s_down;
    /* Pointer-table weights: the layer-oblivious grouped GEMM of ASAP
     * (section 3.4.2, "Bubble-Free Kernel Dispatching", Figure 9b: pointer
     * access to the expert weights of every layer, an on-device address array,
     * the layer id a device-side argument) and the per-buffer weight list of
     * DWDP (section 4.2: experts held in separate local and prefetched buffers,
     * read in place).  NULL: the matrices are the contiguous arrays above.
     * Non-NULL: `table` is a device array [n_layers][E + has_shared][6] of
     * device pointers {gate, up, down, s_gate, s_up, s_down} to ONE expert's
     * matrices (the layouts above without the leading [E]; entry E of a layer
     * is the shared expert; scale entries NULL for bf16 weights; with
     * layout MOE_LAYOUT_TILED, gate points to the expert's tiled gate+up
     * matrix, down to its tiled down matrix, up is unused); `layer` is a device
     * int32 that the grouped FFN's kernels read when they run, so a call (or a
     * captured graph) can be enqueued before the layer is known.  A *layer
     * outside [0, n_layers) makes the FFN kernels skip all work (y_rows,
     * y_shared and, in moe_layer, out are then undefined).  The other pointer
     * fields are ignored.  Matrices 16-byte aligned, scales 4-byte.  Supported on
     * the bf16 and fp8 paths (not fp32).  moe_weight_table fills a table from
     * contiguous per-layer weights. */
    const void *const *table;
    const int32_t *layer;
    int32_t n_layers;
} moe_weights;

/* Checks a configuration on the host (no HIP call).  MOE_OK if every entry
 * point accepts it. */
moe_status moe_validate(const moe_cfg *cfg);

/* Host helper of pointer-table weights (no HIP call, nothing dereferenced):
 * writes to the HOST array table[n_layers * (E + has_shared) * 6] the
 * addresses of each expert's matrices in the contiguous weights layers[l]
 * (table == NULL in each; layout row-major or tiled, as cfg's dtypes allow),
 * in the order moe_weights.table reads.  The caller copies the array to the
 * device.  MOE_ERR_UNSUPPORTED for fp32 weights. */
moe_status moe_weight_table(const moe_cfg *cfg, const moe_weights *layers, int32_t n_layers,
                            const void **table);

/* Upper bound of the dispatched rows: T*k + E*(m_tile - 1).  Sizes row_src,
 * x_perm and y_rows.  Returns -1 for an invalid cfg. */
int64_t moe_max_rows(const moe_cfg *cfg);

/* Workspace bytes the given stage needs (0 if none); (size_t)-1 for an
 * invalid cfg or stage. */
size_t moe_workspace_bytes(const moe_cfg *cfg, int32_t stage);

/* Workspace bytes of moe_grouped_ffn for n_rows_cap rows (the FFN stage of
 * moe_workspace_bytes is this with n_rows_cap = moe_max_rows(cfg)).
 * (size_t)-1 for an invalid cfg or a negative / too large n_rows_cap. */
size_t moe_ffn_workspace_bytes(const moe_cfg *cfg, int64_t n_rows_cap);

/* Bytes of x_perm for cfg->x_layout (moe_max_rows * H * sizeof(act_dtype)
 * when row-major); (size_t)-1 for an invalid cfg. */
size_t moe_x_perm_bytes(const moe_cfg *cfg);

/* Bytes of the tiled copy of the expert weights (routed and shared) that
 * moe_tile_weights writes; (size_t)-1 for an invalid cfg or weights without a
 * tiled layout (fp32, MXFP4). */
size_t moe_tiled_weights_bytes(const moe_cfg *cfg);

/* Rewrites row-major bf16 or e4m3 expert weights into the tiled layout the
 * grouped GEMMs stream with contiguous loads, each wave's weight fragments of
 * a K stage one contiguous block (weights are static: done once, at load
 * time).  Rows and columns past a matrix are zero; the routed experts follow
 * each other, then the shared expert's two matrices.
 * bf16: a matrix of R rows and K columns becomes 4 KiB blocks of 64 rows x 32
 * columns, block (r / 64, k / 32) at byte ((r / 64) * ceil(K / 32) + k / 32) *
 * 4096; inside, the 16-byte chunk j * 64 + l (j < 4, l < 64) holds row
 * 32 (j / 2) + l % 32, columns 16 (j % 2) + 8 (l / 32) .. + 7.  Gate and up
 * merge into one matrix of 2 * roundup(I, 128) rows: rows 64 q + c hold gate
 * row 32 q + c (c < 32) and up row 32 q + c - 32 (c >= 32).  Down keeps its H
 * rows.  Per expert the gate+up matrix spans 2 * roundup(I, 128) / 64 *
 * ceil(H / 32) blocks and the down matrix ceil(H / 64) * ceil(I / 32).
 * e4m3: 4 KiB blocks of 32 rows x 128 columns, block (r / 32, k / 128) at byte
 * ((r / 32) * (K / 128) + k / 128) * 4096; inside, byte 1024 i + 16 l + b
 * (i < 4, l < 64, b < 16) holds row 16 (i / 2) + l % 16, column 32 (l / 16) +
 * 16 (i % 2) + b.  Gate and up merge into 2 I rows: rows 32 q + c hold gate row
 * 16 q + c (c < 16) and up row 16 q + c - 16 (c >= 16).  The byte counts are
 * the row-major ones; the fp32 block scales are not rewritten: `tiled` points
 * s_* and sh_s_* at src's arrays, which must stay alive.
 * src: row-major weights (w_gate, w_up, w_down, and sh_* when has_shared);
 * dst: device buffer of moe_tiled_weights_bytes(cfg) bytes, 256-byte aligned;
 * tiled: filled with the pointers into dst and layout MOE_LAYOUT_TILED.
 * MOE_ERR_UNSUPPORTED for fp32 or MXFP4 weights. */
moe_status moe_tile_weights(const moe_cfg *cfg, const moe_weights *src, void *dst, size_t dst_bytes,
                            moe_weights *tiled, void *stream);

/* Router GEMM and top-k gating (the "gated routing" of the AFD page, section
 * 3; ASAP's expert IDs of Table 2).
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h]   (fp32 accumulation)
 * or, when logits_in != NULL, logits = logits_in (x and w_router are then
 * ignored and may be NULL).
 *   softmax: z_e = logits[t][e] + bias[e] (bias may be NULL), p = softmax(z);
 *            the selection key of expert e is z_e, its raw score p_e.
 *   sigmoid: s_e = 1 / (1 + exp(-logits[t][e])); key s_e + bias[e]; raw s_e.
 *   group limit (n_groups > 1): group g = experts [g*E/G, (g+1)*E/G); group
 *            score = sum of its two largest keys (TOP2_SUM) or its largest
 *            (MAX); the topk_groups best groups are kept (ties: lower group).
 *   top-k:   the k best keys among kept experts, slot j = j-th best, ties to the
 *            lower expert index; keys are fp32 values.
 *   weight:  w_j = raw_j / sum(raw over the k) if renormalize else raw_j,
 *            times routed_scale.
 * x [T][H] act_dtype (F32 or BF16), w_router [E][H] same dtype, bias [E] fp32
 * or NULL, logits_in [T][E] fp32 or NULL, logits_out [T][E] fp32 or NULL
 * (written when non-NULL), topk_ids [T][k] int32, topk_w [T][k] fp32.
 * ws: moe_workspace_bytes(cfg, MOE_STAGE_ROUTE) (it holds the K-split partial
 * logits; unused, and may be NULL, when logits_in != NULL). */
moe_status moe_route(const moe_cfg *cfg, const void *x, const void *w_router, const float *bias,
                     const float *logits_in, float *logits_out, int32_t *topk_ids,
                     float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* moe_route on bf16 x that also writes x's per-token e4m3 quantisation, the
 * rule and outputs of moe_quantize_fp8 (x_q [T][H] OCP e4m3 codes, x_scale
 * [T][H/128] fp32), from the router's own pass over x: the "fp8 route" of a
 * layer whose expert GEMMs run in fp8 (the AFD page, section 1, the figure
 * caption on MoE MFU; section 7, W8A8), with no second read of x for the
 * quantiser.  topk_ids, topk_w and logits_out (NULL: not written) are those of
 * moe_route with logits_in == NULL; x_q and x_scale equal moe_quantize_fp8's
 * bit for bit.  Takes act_dtype MOE_BF16 and H a multiple of 128; x and
 * w_router 16-byte aligned, x_q 8-byte aligned, x_scale 4-byte aligned
 * (MOE_ERR_INVALID_ARG otherwise).
 * ws: moe_workspace_bytes(cfg, MOE_STAGE_ROUTE). */
moe_status moe_route_quantize(const moe_cfg *cfg, const void *x, const void *w_router, const float *bias,
                              float *logits_out, int32_t *topk_ids, float *topk_w, uint8_t *x_q,
                              float *x_scale, void *ws, size_t ws_bytes, void *stream);

/* Dispatch: a deterministic counting sort of the (token, choice) pairs by
 * expert (ASAP section 3.2.1: token counts per expert plus the token payload).
 *   expert_counts[e]  = #{(t, j) : topk_ids[t][j] == e}
 *   expert_offsets[e] = sum_{e' < e} ceil(count[e'] / m_tile) * m_tile   (E + 1 entries)
 *   inside an expert the rows follow ascending token index:
 *   row(t, j)         = expert_offsets[e] + #{t' < t : e in topk_ids[t']}
 *   row_src[row]      = t * k + j, or -1 for a padding row (moe_max_rows entries)
 *   tok_row[t*k + j]  = row(t, j)
 *   x_perm[row]       = x[t] (bit copy), zero rows where row_src == -1
 *   x_perm_scale[row] = x_scale[t] (fp8 activations only; [rows][H/128])
 * x_perm is laid out as cfg->x_layout says (moe_x_perm_bytes bytes); the tiled
 * layout also receives the shared expert's copy of x when has_shared, and its
 * column padding up to a multiple of 32 is zero.  With MOE_LAYOUT_INDEXED
 * x_perm is not written and may be NULL.
 * topk_ids must hold distinct ids in [0, E) per token.
 * ws: moe_workspace_bytes(cfg, MOE_STAGE_PERMUTE). */
moe_status moe_permute(const moe_cfg *cfg, const void *x, const float *x_scale,
                       const int32_t *topk_ids, int32_t *expert_counts,
                       int32_t *expert_offsets, int32_t *row_src, int32_t *tok_row,
                       void *x_perm, float *x_perm_scale, void *ws, size_t ws_bytes,
                       void *stream);

/* moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and layouts as moe_permute,
 * without ws / ws_bytes: the per-block counts of the counting sort live in a
 * static device array of the library, 4 MiB on each GPU it runs on, held until
 * the process ends.  Limit: 2 * ceil(T / 256) * E <= 1048576 (for example
 * T <= 524288 at E = 256), else MOE_ERR_UNSUPPORTED before anything is
 * enqueued.  The first call on a device looks up that array's address on the
 * current device (which must be the stream's device); no call allocates,
 * frees or synchronises.  Every call on one GPU shares the array, so calls
 * that overlap on one GPU (work of two of them in flight at once, e.g. on two
 * streams) race and give undefined results: order them on one stream. */
moe_status moe_permute_noalloc(const moe_cfg *cfg, const void *x, const float *x_scale,
                               const int32_t *topk_ids, int32_t *expert_counts,
                               int32_t *expert_offsets, int32_t *row_src, int32_t *tok_row,
                               void *x_perm, float *x_perm_scale, void *stream);

/* Grouped SwiGLU FFN over expert-contiguous rows (ASAP section 3.4.2's GMM).
 * For every expert e and every row r in [expert_offsets[e], expert_offsets[e+1]):
 *   g_i = sum_h x_rows[r][h] * w_gate[e][i][h],  u_i = sum_h x_rows[r][h] * w_up[e][i][h]
 *   a_i = silu(g_i) * u_i,  silu(z) = z / (1 + exp(-z))
 *   y_rows[r][h] = sum_i a_i * w_down[e][h][i]
 * with fp32 accumulation.  The intermediate a is stored as bf16 (bf16
 * operands), fp32 (fp32 operands) or, for fp8 operands, as e4m3 with one fp32
 * scale per row and 128 columns: s = max|a| / 448 (1 if the block is zero),
 * q = e4m3_rne_sat(a / s).  fp8 operands are dequantised as code * scale with
 * x_scale [n_rows_cap][H/128] (1 x 128 per-row blocks) and the 128 x 128
 * weight block scales.  Offsets may be unpadded (any alignment) and rows of
 * x_rows outside [0, expert_offsets[E]) are neither read nor written.
 * When cfg->has_shared, the shared expert is applied to every token of
 * x_tokens [T][H] into y_shared [T][H] (weight 1).
 * cfg->x_layout MOE_LAYOUT_TILED: x_rows is the tiled x_perm of moe_permute
 * with the same cfg, n_rows_cap must equal moe_max_rows(cfg), the expert
 * offsets must be multiples of 16 (results are undefined otherwise, accesses
 * stay inside x_rows), and the shared expert reads its copy of the tokens
 * inside x_rows (x_tokens is ignored and may be NULL).
 * cfg->x_layout MOE_LAYOUT_INDEXED: x_rows is x [T][H] itself and row_src
 * [n_rows_cap] (int32, as written by moe_permute) maps row r to token
 * row_src[r] / k, a zero row where row_src[r] < 0; the shared expert reads
 * x_rows too (x_tokens is ignored and may be NULL).  row_src is unused (may
 * be NULL) for the other layouts.
 * y_rows [n_rows_cap][H] and y_shared in cfg->y_dtype.  n_rows_cap is the
 * row count of x_rows and y_rows, independent of T (rows may arrive already
 * dispatched); expert_offsets[E] <= n_rows_cap.
 * ws: moe_ffn_workspace_bytes(cfg, n_rows_cap). */
moe_status moe_grouped_ffn(const moe_cfg *cfg, int64_t n_rows_cap, const void *x_rows,
                           const float *x_scale, const int32_t *expert_offsets,
                           const int32_t *row_src, const moe_weights *w, const void *x_tokens,
                           void *y_rows, void *y_shared, void *ws, size_t ws_bytes,
                           void *stream);

/* Combine: the weighted gather-reduce back to token order (ASAP section
 * 3.2.2's expert results per token and choice).
 *   out[t][h] = sum_{j=0..k-1} topk_w[t][j] * y_rows[tok_row[t*k+j]][h]  (+ y_shared[t][h])
 * accumulated in fp32 in slot order, the shared term last.
 * y_rows, y_shared in cfg->y_dtype; out [T][H] in cfg->out_dtype.  The
 * shared term is added whenever y_shared != NULL; y_shared must not be NULL
 * when cfg->has_shared.  y_rows, y_shared and out are 16-byte aligned
 * (MOE_ERR_INVALID_ARG otherwise). */
moe_status moe_combine(const moe_cfg *cfg, const void *y_rows, const int32_t *tok_row,
                       const float *topk_w, const void *y_shared, void *out, void *stream);

/* Per-token quantisation of activations for fp8 experts.  The AFD page runs
 * its MoE GEMMs in fp8 (section 1, the figure caption on MoE MFU: "fp8
 * DeepGEMM"; section 7: W8A8) without printing the quantiser; the fp8
 * expert-parallel workload this library is measured on states per-token
 * 1 x 128 activation scales.  The rule is the one the grouped FFN applies to
 * its intermediate.  For each row t and 128-column block b of
 * x [T][H] bf16: s = max|x| / 448 over the block (1 when the block is all
 * zero), q = e4m3_rne_sat(x / s), the divisions in fp32; x_q [T][H] OCP e4m3
 * codes, x_scale [T][H/128] fp32 (x, x_q, x_scale 16-, 8- and 4-byte
 * aligned, device).  Takes act_dtype MOE_BF16 and H a multiple of 128. */
moe_status moe_quantize_fp8(const moe_cfg *cfg, const void *x, uint8_t *x_q, float *x_scale, void *stream);

/* The whole layer: moe_route -> moe_permute -> moe_grouped_ffn -> moe_combine,
 * enqueued on `stream` with no host synchronisation.  x [T][H] in act_dtype
 * (F32 or BF16); out [T][H] in out_dtype.  All intermediates live in ws.
 * The stages run with m_tile = 16 and, for bf16, x_layout =
 * MOE_LAYOUT_INDEXED while x is under 2 GiB (MOE_LAYOUT_TILED beyond, which
 * the workspace size accounts for), whatever cfg->m_tile and cfg->x_layout say
 * (those shape the standalone stage calls only); the result equals that of
 * the four stage calls made with those two fields.  With bf16 y, a shared
 * expert, T >= 4096 and the environment variable MOE_FUSED_COMBINE set to 1
 * (read at each call) the combine runs inside the shared expert's GEMM2 (its
 * tiles own token rows of out; the same arithmetic, so the same bits); by
 * default it runs as the separate combine pass, which times as fast or
 * faster.  w may be row-major or tiled.  x, w_router and out are 16-byte aligned.
 * Low-precision experts (act_dtype MOE_BF16, w_dtype MOE_FP8_E4M3 or
 * MOE_FP4_E2M1, row-major weights with their scales, x 16-byte aligned): the
 * route and the quantisation of x in one pass (moe_route_quantize), moe_permute's maps (m_tile 16,
 * MOE_LAYOUT_INDEXED: the routed GEMM1 reads the e4m3 token rows and their
 * scales through row_src; for quantised tokens of 2 GiB or more, a row-major
 * x_perm with its scales), the grouped FFN over the routed rows and, with a
 * shared expert, a second one over the T quantised tokens, then
 * moe_combine.  With pointer-table weights (moe_weights.table) the FFN
 * kernels take the layer from *w->layer when they run.
 * ws: moe_workspace_bytes(cfg, MOE_STAGE_LAYER). */
moe_status moe_layer(const moe_cfg *cfg, const void *w_router, const float *bias,
                     const moe_weights *w, const void *x, void *out, void *ws,
                     size_t ws_bytes, void *stream);

/* Static text of a status code. */
const char *moe_status_string(moe_status status);

/* Message of the last failed call on the calling thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXPERT_LAYER_AMD_MOE_H */
