/*
 * veda.h -- C ABI of the MI355X (gfx950) Veda-style block-sparse attention library.
 *
 * One attention layer of a video diffusion transformer, split as the method
 * splits it:
 *   selection  (a lightweight predictor, "Training the Selector, Not the
 *              Generator" in the Affine launch article: the selector's query and
 *              key projections pick which attention blocks are computed), and
 *   attention  over the selected key tiles plus key ranges that stay dense
 *              (Veda R2VA record, first paragraph: reference and current-video
 *              tiles are chosen independently with fixed budgets per query tile
 *              and head; text, VLM conditioning and audio attention stay dense).
 *
 * Conventions shared by every entry point
 *   - Every buffer is caller-owned device memory (hipMalloc'd or torch-allocated).
 *     The library never allocates or frees device memory, keeps no pointer after
 *     a call returns and has no mutable global state: calls are re-entrant.  The one
 *     exception is veda_select_noalloc, whose workspace is a library-owned device array
 *     per GPU (see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *     work is enqueued asynchronously on it; nothing is synchronised.  A device
 *     fault surfaces at the caller's next synchronisation.
 *   - Arguments are validated completely on the host before any device call; an
 *     invalid call returns a negative veda_status and enqueues nothing.
 *   - Q, K, V and the attention output are bfloat16 tensors addressed as
 *       elem(b, n, h, c) = base + b*stride_b + n*stride_n + h*stride_h + c
 *     (strides in elements, the head dimension c contiguous).  The natural
 *     layout is [B, n_tokens, H, d] contiguous.  Base pointers must be 16-byte
 *     aligned, the three strides multiples of 8 elements and stride_n below 2^24.
 *   - Tiles: the query segment is cut into Tq = ceil(query.len / tile) tiles
 *     starting at query.start; key segment s into T_s = ceil(seg[s].len / tile)
 *     tiles starting at seg[s].start.  The last tile of a segment may be partial.
 */
#ifndef VEDA_H
#define VEDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VEDA_ABI_VERSION 6
#define VEDA_MAX_SEGMENTS 4
#define VEDA_MAX_DENSE 8
#define VEDA_MAX_KEY_TILES 8192   /* sum over segments of T_s accepted by selection */

typedef enum veda_status {
  VEDA_OK = 0,
  VEDA_EINVAL = -1,        /* null pointer, non-positive size, misaligned pointer or stride */
  VEDA_EUNSUPPORTED = -2,  /* d not in {64,128}, tile not in {64,128}, p not a multiple of 16
                              in [16, 384], more than VEDA_MAX_SEGMENTS / VEDA_MAX_DENSE,
                              more than VEDA_MAX_KEY_TILES key tiles, stride_n >= 2^24;
                              size limits: B*H, Tq and sum_s T_s at most 2^31 - 1, and
                              B*H*Tq*max(1, sum_s T_s) at most 2^40 */
  VEDA_EWORKSPACE = -3,    /* workspace smaller than veda_select_workspace_bytes() */
  VEDA_ERANGE = -4,        /* a range leaves [0, n_tokens), key segments overlap each other,
                              or a dense range overlaps a key segment or another dense range */
  VEDA_ENOKEYS = -5,       /* a query tile would attend to no key at all */
  VEDA_EHIP = -6,          /* the HIP runtime reported an error at launch */
  VEDA_EIO = -7,           /* a file could not be opened or read */
  VEDA_EFORMAT = -8        /* a file is not a well-formed safetensors file */
} veda_status;

/* Token range [start, start + len). */
typedef struct veda_range {
  int64_t start;
  int64_t len;
} veda_range;

/* Element type of the predictor weights Wq, Wk. */
typedef enum veda_wdtype {
  VEDA_W_BF16 = 0,         /* bfloat16 (also the result of veda_dequant_fp8_e4m3) */
  VEDA_W_F16 = 1           /* IEEE float16, as the competition's selector files store them */
} veda_wdtype;

/* Shape of one attention layer. */
typedef struct veda_layer {
  int32_t B;          /* batch                                                   */
  int32_t H;          /* heads (K/V have as many heads as Q)                      */
  int32_t d;          /* head dimension: 64 or 128                                */
  int32_t p;          /* predictor dimension (rows of Wq[h], Wk[h]); selection only */
  int32_t tile;       /* tokens per tile: 64 or 128                               */
  int32_t n_seg;      /* key segments, 1..VEDA_MAX_SEGMENTS (0 allowed for attention
                         when dense ranges exist)                                 */
  int64_t n_tokens;   /* sequence length of Q, K, V                               */
  int64_t stride_b, stride_n, stride_h;   /* element strides of Q, K, V and out  */
  veda_range query;   /* the sparse query segment (generated video)               */
  veda_range seg[VEDA_MAX_SEGMENTS];      /* key segments, in call order          */
  int32_t budget[VEDA_MAX_SEGMENTS];      /* top-k budget per segment, >= 0; a budget
                                             above T_s selects every tile          */
  int32_t wdtype;     /* veda_wdtype of Wq, Wk (selection only); 0 = bf16          */
  int32_t reserved;   /* must be 0                                                */
} veda_layer;

/* Ktot = sum_s min(budget[s], T_s): index entries per (b, h, query tile).  -1 for a null
 * layer, tile <= 0, n_seg outside [0, VEDA_MAX_SEGMENTS], or a negative segment length or
 * budget.  No other check is made (veda_layer_check does those). */
int64_t veda_k_total(const veda_layer* layer);

/* Library ABI version (VEDA_ABI_VERSION of the build). */
int veda_abi_version(void);

/* Static text for a veda_status value. */
const char* veda_status_string(int status);

/* Host-only check of a layer description for selection (checks p) or for
 * attention only (for_select = 0).  Returns VEDA_OK or the error code the
 * corresponding entry point would return for this layer.  No device call. */
int veda_layer_check(const veda_layer* layer, int for_select);

/* Bytes of workspace veda_select needs: the projected pooled vectors
 * q_hat [B,H,Tq,p] and k_hat [B,H,sum T_s,p] in fp32, 256-byte aligned.
 * Returns 0 for an invalid layer. */
size_t veda_select_workspace_bytes(const veda_layer* layer);

/*
 * Pool and project (steps a1 + a2).  Affine launch article, "Training the Selector,
 * Not the Generator": the trained selector is a query projection and a key projection
 * (one tensor each per layer, "How the SN120 Competition Works"); the pooling to one
 * vector per token tile is this library's reading of its "lightweight predictor".
 * For every (b, h) and tile i of the query segment:
 *     q_bar[i] = mean of Q[b, n, h, :] over the real tokens n of tile i (fp32 sums),
 *     q_hat[b, h, i, :] = Wq[h] q_bar[i]      (Wq[h] is p x d, row-major, no bias);
 * likewise k_hat[b, h, j, :] = Wk[h] k_bar[j] for every tile j of every key
 * segment, segments concatenated in call order.
 *   q, k   : bf16, strided as described above
 *   wq, wk : [H, p, d] contiguous, 16-byte aligned, bf16 or f16 (layer->wdtype);
 *            both types convert to fp32 exactly
 *   q_hat  : fp32 [B, H, Tq, p] contiguous (output)
 *   k_hat  : fp32 [B, H, sum_s T_s, p] contiguous (output)
 */
int veda_pool_project(const veda_layer* layer, const void* q, const void* k,
                      const void* wq, const void* wk, float* q_hat, float* k_hat,
                      void* stream);

/*
 * Score and select (steps a3 + a4), from veda_pool_project's outputs.  Veda R2VA
 * record, first paragraph: a fixed budget of key tiles per query tile and head, the
 * reference and current-video segments chosen independently (one budget per segment).
 *     S[b, h, i, j] = <q_hat[b,h,i,:], k_hat[b,h,j,:]>    (unscaled)
 * For every (b, h, i) and segment s, the min(budget[s], T_s) tiles of segment s
 * with the largest S; equal scores go to the lower tile index (-0 equals +0).
 * They are written ascending, as segment-local tile ids, segment blocks in call
 * order:  idx int32 [B, H, Tq, Ktot] contiguous (output).
 *   scores_opt : NULL, or fp32 [B, H, Tq, sum_s T_s] contiguous receiving S.
 * S is computed on bf16 matrix cores with each fp32 operand split into a high
 * and a low bf16 part (three products), fp32 accumulation.
 */
int veda_score_topk(const veda_layer* layer, const float* q_hat, const float* k_hat,
                    int32_t* idx, float* scores_opt, void* stream);

/*
 * Full selection: veda_pool_project into the workspace, then veda_score_topk (the
 * selector of the Affine launch article, "Training the Selector, Not the Generator",
 * with the per-segment budgets of the Veda R2VA record, first paragraph).
 *   ws, ws_bytes : device workspace of at least veda_select_workspace_bytes(layer),
 *                  256-byte aligned.  Its contents are scratch.
 */
int veda_select(const veda_layer* layer, const void* q, const void* k,
                const void* wq, const void* wk, int32_t* idx, float* scores_opt,
                void* ws, size_t ws_bytes, void* stream);

/*
 * veda_select for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * results, with the workspace taken from a library-owned device array of
 * VEDA_NOALLOC_SCRATCH_BYTES per GPU instead of a caller buffer.  The caller still
 * passes the inputs and outputs (q, k, wq, wk, idx, scores_opt as for veda_select).
 *   - Allocates nothing: no hipMalloc/hipFree, no allocating library call.  The array
 *     is held by every GPU the library runs on until the process ends.
 *   - The array of the device current on the calling thread is used; `stream` must
 *     belong to that device.  Its device address is looked up once per device (the
 *     first call on a device makes that lookup, a HIP runtime call).
 *   - Layers whose veda_select_workspace_bytes() exceeds VEDA_NOALLOC_SCRATCH_BYTES
 *     return VEDA_EWORKSPACE before any device call (64 MiB covers q_hat + k_hat of
 *     H = 40, p = 64 with 2741 query and 2741 key tiles).
 *   - Calls that overlap in time on one GPU (concurrent streams or threads) share the
 *     array and race; serialise them.  No contents need clearing between calls: every
 *     workspace entry a call reads is written earlier in the same call.
 */
#define VEDA_NOALLOC_SCRATCH_BYTES (64u << 20)
int veda_select_noalloc(const veda_layer* layer, const void* q, const void* k,
                        const void* wq, const void* wk, int32_t* idx, float* scores_opt,
                        void* stream);

/*
 * Block-sparse attention (step a5).  Affine launch article, "Training the Selector,
 * Not the Generator": the selected blocks feed a sparse execution kernel; Veda R2VA
 * record, first paragraph: text, VLM conditioning and audio keys stay dense (the
 * `dense` ranges).  For every (b, h) and query tile i, the key
 * set A(b,h,i) is the union of the tokens of the tiles idx[b,h,i,:] selects
 * (segment-local ids, segment blocks in call order, as veda_score_topk writes
 * them) and of every dense range.  For each query row n of tile i:
 *     out[b, n, h, :] = sum_{m in A} softmax_m(scale * <Q[b,n,h,:], K[b,m,h,:]>) V[b,m,h,:]
 * computed with bf16 matrix cores, fp32 online softmax and fp32 accumulation,
 * rounded to bf16 (nearest even).  Only the query segment's rows of `out` are
 * written.
 *   idx        : int32 [B, H, Tq, Ktot] contiguous.  An entry of -1 is padding: it
 *                and every later entry of the same segment's block select nothing
 *                (producers with fewer tiles for some query tiles end those rows'
 *                segment blocks with -1; the kernel skips the rest of the block at
 *                once).  Other entries are NOT re-validated:
 *                an id outside [0, T_s) is undefined behaviour.  A query tile left with
 *                no key at all (all padding, no dense range) gets zero output rows.
 *                idx may be NULL when every budget[s] >= T_s: every tile of every
 *                segment is then attended (dense attention over the segments).
 *   order      : NULL, or int32 [B, H, Tq] contiguous, 4-byte aligned (needs idx): for
 *                every (b, h), the query tiles in the order the kernel starts them, as
 *                veda_tile_order writes it.  Results do not depend on it; it decides
 *                how often gathered K/V blocks are found in L2.  It should be a
 *                permutation of 0 .. Tq-1: an entry outside that range is skipped (the
 *                rows of a tile no entry names are not written), a tile named twice is
 *                computed twice.  NULL is the natural order 0 .. Tq-1.
 *   dense      : host array of n_dense ranges (0 <= n_dense <= VEDA_MAX_DENSE),
 *                disjoint from the key segments and from each other.
 *   scale      : softmax scale; 0 selects 1/sqrt(d).
 *   out        : bf16 with the same strides as q.
 *   lse_opt    : NULL, or fp32 [B, H, query.len] receiving the natural-log
 *                log-sum-exp of each row's scaled logits.
 * q, k and v must hold finite values: a non-finite K or V value read by one query
 * tile's workgroup may make every row of that (b, h, query tile) non-finite, not only
 * the rows whose keys include it (key blocks are multiplied with zero weights where
 * a block is partial or missing).
 */
int veda_sparse_attn(const veda_layer* layer, const void* q, const void* k, const void* v,
                     const int32_t* idx, const int32_t* order, const veda_range* dense,
                     int32_t n_dense, float scale, void* out, float* lse_opt, void* stream);

/*
 * Processing order of the query tiles for the attention calls (their `order`
 * argument).  The pages fix what the sparse execution kernel computes per query tile
 * (Affine launch article, "Training the Selector, Not the Generator"), not the order
 * in which tiles run; this one puts tiles whose selections start alike side by side,
 * so that workgroups running at the same time on an XCD gather the same K/V blocks.
 * For every (b, h): the query tiles sorted by their index rows, lexicographically, on
 * the first segment (call order) with budget[s] < T_s: the segment block's first
 * E = min(50 / bits, K_s) entries packed into a key, bits = the bit width of T_s - 1
 * (at least 4), an entry at or after the block's first -1 taken as 2^bits - 1; equal
 * keys by lower tile id.  Without such a segment, or with Tq > 16384, the
 * identity order.
 *   idx   : int32 [B, H, Tq, Ktot] as veda_score_topk writes it (device, 16-byte aligned)
 *   order : int32 [B, H, Tq] contiguous (device, 4-byte aligned, output), a permutation
 *           of 0 .. Tq-1 for every (b, h)
 * One launch on `stream` (a workgroup per 256 query tiles of a (b, h)), no workspace.
 */
int veda_tile_order(const veda_layer* layer, const int32_t* idx, int32_t* order, void* stream);

/*
 * FP8 variant of veda_sparse_attn's first product (row f4 of the scope: the pages'
 * FP8 paths, R2VA record first paragraph and the VDN article's fp8 transformer, store
 * weights in FP8; this extends it to the logits, which the pages do not describe).
 * q8 and k8 hold OCP E4M3FN codes of Q and K at the same element offsets as the bf16
 * tensors (layer strides, one byte per element; strides must be multiples of 16),
 * each with a per-tensor scale in device memory (one float, as veda_quantize_fp8_e4m3
 * writes it).  Logits are
 *     scale * q_scale * k_scale * sum_c e4m3(q8[b,n,h,c]) * e4m3(k8[b,m,h,c])
 * on the FP8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation; its
 * sum of 64 products is not exact: measured within 2^-12 of the largest product).
 * Softmax, P (bf16) . V (bf16) and every other argument are as in veda_sparse_attn.
 * Needs 128-row tiles and at most 3072 64-key blocks per query tile (selected tiles
 * plus dense ranges); else VEDA_EUNSUPPORTED.
 */
int veda_sparse_attn_fp8qk(const veda_layer* layer, const uint8_t* q8, const uint8_t* k8, const void* v,
                           const float* q_scale, const float* k_scale, const int32_t* idx,
                           const int32_t* order, const veda_range* dense, int32_t n_dense, float scale,
                           void* out, float* lse_opt, void* stream);

/*
 * Per-tensor FP8 quantisation for veda_sparse_attn_fp8qk: x is a bf16 tensor
 * [B, n_tokens, H, d] with the layer's strides (every token, not only the query rows),
 * x8 receives E4M3FN codes at the same element offsets (one byte each, 16-byte
 * aligned), and *scale (device float) the power of two 2^e with e the smallest integer
 * such that max|x| <= 448 * 2^e (2^0 for an all-zero x).  x8 = nearest E4M3FN value of
 * x / 2^e, ties to the even code, sign kept (-0 -> 0x80); the division is exact and no
 * code saturates.  Four launches on `stream`; x must be finite.
 */
int veda_quantize_fp8_e4m3(const veda_layer* layer, const void* x, uint8_t* x8, float* scale,
                           void* stream);

/*
 * FP8 attention with both products on the FP8 matrix cores (row f4 of the scope: the
 * VDN article "VDN-H3 Renders Video Faster Than It Plays", section "Where it falls
 * down", names a dedicated FP8 path; the Veda R2VA record, first paragraph, and the
 * OpenVDN/vdn-minimax-h3 card, "Download the weights", ship FP8 streams.  The pages do
 * not say how P is held; here it is E4M3FN).
 * q8, k8, q_scale, k_scale as in veda_sparse_attn_fp8qk; vt and v_scale as
 * veda_quantize_fp8_e4m3_vt writes them (vt device, veda_fp8_vt_bytes bytes, 16-byte
 * aligned).  Per (b, h, query row) with the logits s_m of veda_sparse_attn_fp8qk over
 * the same key set:
 *     w_m = e4m3(16 exp(s_m - M)),  out = v_scale * sum_m w_m v8_m / sum_m w_m
 * where v8_m is the decoded code of V row m, M a running maximum of the row's logits
 * (one of them, at most 4.5 ln 2 below the largest logit of the key block, so
 * w_m < 2^8.5) and e4m3 rounds to nearest even; the normaliser sums exactly the rounded
 * weights.  Scaled so that the row's largest exact weight exp(s_m - max s) is 1, each
 * weight is off its exact value p_m by at most 2^-4 p_m where p_m >= 2^-10, and by at
 * most min(p_m, 2^-14) below that (subnormal codes; weights under 2^-14 may round to 0),
 * by a rounding that depends on the block order (callers cannot predict it).  lse_opt
 * (if given) is log(sum_m w_m exp(M) / 16), the row's log-sum-exp over the rounded
 * weights.
 * Needs 128-row tiles, segment and dense-range starts on multiples of 64 tokens, at
 * most 3072 64-key blocks per query tile (else VEDA_EUNSUPPORTED); strides of q8, k8 as
 * for veda_sparse_attn_fp8qk.  Every other argument and status as in veda_sparse_attn.
 */
int veda_sparse_attn_fp8(const veda_layer* layer, const uint8_t* q8, const uint8_t* k8, const uint8_t* vt,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         const int32_t* idx, const int32_t* order, const veda_range* dense,
                         int32_t n_dense, float scale, void* out, float* lse_opt, void* stream);

/*
 * V for veda_sparse_attn_fp8: v bf16 [B, n_tokens, H, d] (layer strides, 16-byte
 * aligned) -> vt, E4M3FN codes in d-major blocks of 64 tokens, [B, H, ceil(n_tokens /
 * 64), d, 64] bytes with each 64-byte row's four 16-byte chunks permuted: row c of block
 * g keeps the codes of tokens 64 g + 16 j .. 64 g + 16 j + 15 in chunk j ^ ((c >> 1) & 3).
 * Tokens past n_tokens are code 0.  *v_scale and the codes as veda_quantize_fp8_e4m3
 * (the same per-tensor power of two, the same rounding).  Four launches on `stream`.
 */
int veda_quantize_fp8_e4m3_vt(const veda_layer* layer, const void* v, uint8_t* vt, float* v_scale,
                              void* stream);

/* Bytes of veda_quantize_fp8_e4m3_vt's output for this layer: B * H * ceil(n_tokens / 64)
 * * d * 64.  Returns 0 for an invalid layer, or when B * H * ceil(n_tokens / 64) exceeds
 * 2^31 - 1 (the two FP8-V entry points then return VEDA_EUNSUPPORTED). */
size_t veda_fp8_vt_bytes(const veda_layer* layer);

/*
 * Host-only check of a veda_sparse_attn call: returns the status veda_sparse_attn
 * would return for these arguments without launching anything (lse_opt and stream
 * are not needed).  No device call.
 */
int veda_sparse_attn_check(const veda_layer* layer, const void* q, const void* k, const void* v,
                           const int32_t* idx, const int32_t* order, const veda_range* dense,
                           int32_t n_dense, float scale, const void* out);

/*
 * One full attention layer as the video model runs it (Veda R2VA record, first
 * paragraph: the video queries use the selected reference and video tiles; text,
 * VLM conditioning and audio attention stay dense):
 *   1. veda_select for the query segment (the generated video)  -> idx;
 *   2. veda_tile_order into the workspace (free after step 1), then veda_sparse_attn
 *      for the query segment's rows in that order;
 *   3. for each of the n_dense_queries ranges (text, VLM, audio or reference query
 *      rows), dense attention over every token of every key segment and every
 *      dense key range, written at those rows of `out`.
 * All checks of the three stages are done before the first launch.
 *   dense_queries : host array (<= VEDA_MAX_DENSE) of query ranges, disjoint from
 *                   layer->query and from each other (they may overlap key ranges).
 *   idx, ws, ws_bytes : as for veda_select (idx receives the selection).
 * Other arguments as for veda_select / veda_sparse_attn.
 */
int veda_layer_attn(const veda_layer* layer, const void* q, const void* k, const void* v,
                    const void* wq, const void* wk, const veda_range* dense, int32_t n_dense,
                    const veda_range* dense_queries, int32_t n_dense_queries, float scale,
                    void* out, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Teacher block attention mass (the full-attention pattern Veda distils its predictor
 * from: Affine launch article, "Training the Selector, Not the Generator").  For every
 * (b, h, query tile i) and every key tile j of every segment (all tiles, budgets are
 * ignored), with P_n the dense softmax of query row n over ALL keys (every segment
 * token and every dense range) at `scale` (0 selects 1/sqrt(d)):
 *     mass[b,h,i,j]      = (1/rows_i) * sum_{n in tile i} sum_{m in tile j} P_n(m)
 *     dense_mass[b,h,i]  = (1/rows_i) * sum_{n in tile i} sum_{m in dense ranges} P_n(m)
 *     lse[b,h,n]         = log sum_m exp(scale * <q_n, k_m>)   (natural log)
 * so each mass row plus its dense_mass sums to 1.  Column j runs over the key tiles
 * of all segments in call order (segment s starts at sum_{t<s} T_t), as the score
 * block of veda_score_topk.
 *   q, k       : bf16 [B, N, H, d] with the layer's strides (device, 16-byte aligned).
 *   lse        : fp32 [B, H, query.len] (output, also the second pass's input).
 *   mass       : fp32 [B, H, Tq, Tk] (output);  dense_mass_opt: fp32 [B, H, Tq] or NULL.
 * Two passes over all keys, bf16 matrix cores with fp32 accumulation and fp32 exp2.
 * Same argument checks as veda_sparse_attn on the layer with full budgets.
 * Asynchronous on `stream`; all buffers caller-owned.
 */
int veda_block_mass(const veda_layer* layer, const void* q, const void* k, const veda_range* dense,
                    int32_t n_dense, float scale, float* lse, float* mass, float* dense_mass_opt,
                    void* stream);

/*
 * Recall of an index set under the teacher mass: for every (b, h, query tile i)
 *     recall[b,h,i] = sum of mass[b,h,i, toff_s + t] over the tiles t that idx selects
 *                     in segment s (a -1 ends that segment's block), over all s,
 *                     divided by sum_j mass[b,h,i,j]   (1 when that sum is 0).
 *   mass   : fp32 [B, H, Tq, Tk] from veda_block_mass on the same segments.
 *   idx    : int32 [B, H, Tq, Ktot] as veda_sparse_attn reads it (Ktot from the
 *            layer's budgets); ids are not re-validated.
 *   recall : fp32 [B, H, Tq] (output).  Device pointers, 16-byte aligned.
 */
int veda_block_recall(const veda_layer* layer, const float* mass, const int32_t* idx, float* recall,
                      void* stream);

/*
 * Fixed-pattern index producer: sliding windows of frame chunks with boundary
 * anchors (the VDN analysis, "The mechanism: solving instead of stepping": chunks
 * of consecutive latent frames attend to themselves and their neighbouring chunks;
 * every frame also attends to the first and last frames, which attend to
 * everything).  Produced at tile granularity for veda_sparse_attn: query tile i
 * takes every key tile that overlaps a key frame of any of its query frames.
 *   layer        : one key segment equal to the query segment (the video); frames
 *                  count from its start, frame_tokens tokens each.
 *   chunk_frames : frames per chunk (>= 1); halo_chunks: neighbours on each side (>= 0);
 *   anchors      : 1 to add the first/last-frame anchors, 0 for windows only.
 * veda_window_width returns the longest row in tiles, or a negative status
 * (VEDA_EUNSUPPORTED unless n_seg == 1, VEDA_ERANGE unless seg[0] equals the query
 * segment, VEDA_EINVAL for a bad pattern).  veda_window_indices writes
 * idx int32 [B, H, Tq, width] (device, 16-byte aligned, caller-owned): each row
 * ascending, then -1 padding; every (b, h) gets the same rows.  It needs
 * longest row <= width <= ceil(seg[0].len / tile) (else VEDA_EINVAL) and is
 * asynchronous on `stream`.  Feed idx to veda_sparse_attn on the same layer with
 * budget[0] = width.
 */
int64_t veda_window_width(const veda_layer* layer, int64_t frame_tokens, int32_t chunk_frames,
                          int32_t halo_chunks, int32_t anchors);
int veda_window_indices(const veda_layer* layer, int64_t frame_tokens, int32_t chunk_frames,
                        int32_t halo_chunks, int32_t anchors, int32_t* idx, int32_t width,
                        void* stream);

/*
 * FP8 predictor weights to bf16 at load (step a0; Veda R2VA record: the
 * predictor is stored in FP8 and dequantised to BF16 at load).
 *     dst[i] = E4M3FN(src[i]) * 2^pow2_exp, exactly representable in bf16.
 * E4M3FN is the OCP FP8 format (bias 7, 3 mantissa bits, subnormals, max 448,
 * S.1111.111 = NaN, no infinities); NaN codes produce a bf16 quiet NaN.
 *   src : n bytes;  dst : n bf16 values (2-byte aligned);  -24 <= pow2_exp <= 24.
 */
int veda_dequant_fp8_e4m3(const uint8_t* src, void* dst_bf16, int64_t n, int32_t pow2_exp,
                          void* stream);

/*
 * safetensors reader (host only) for predictor files: the competition's selector
 * file holds float16 query/key projections per layer (Affine launch article, "How
 * the SN120 Competition Works"); the R2VA predictor is stored in FP8 and turned into
 * bf16 at load (Veda R2VA record, first paragraph; veda_dequant_fp8_e4m3 does that on
 * the device).  Layout: 8-byte little-endian header length, a JSON header mapping
 * names to {dtype, shape, data_offsets} plus an optional "__metadata__" string map,
 * then the data.  veda_st_open checks the whole header (offsets inside the file,
 * byte counts = dtype size x shape, the tensors tiling the data without holes or
 * overlap) and returns VEDA_EIO (cannot open/read) or VEDA_EFORMAT (malformed).
 * A string holding U+0000 is rejected (VEDA_EFORMAT): names and metadata come back
 * as C strings.  Names, metadata strings and the handle stay valid until veda_st_close.  Tensors
 * keep the file's order.  veda_st_read copies a tensor's raw little-endian bytes into
 * host memory of exactly veda_st_info's nbytes.
 */
typedef struct veda_st_file veda_st_file;
typedef enum veda_st_dtype {
  VEDA_ST_UNKNOWN = 0, VEDA_ST_F16 = 1, VEDA_ST_BF16 = 2, VEDA_ST_F32 = 3, VEDA_ST_F64 = 4,
  VEDA_ST_F8_E4M3 = 5, VEDA_ST_F8_E5M2 = 6, VEDA_ST_I8 = 7, VEDA_ST_U8 = 8, VEDA_ST_I16 = 9,
  VEDA_ST_U16 = 10, VEDA_ST_I32 = 11, VEDA_ST_U32 = 12, VEDA_ST_I64 = 13, VEDA_ST_U64 = 14,
  VEDA_ST_BOOL = 15
} veda_st_dtype;
#define VEDA_ST_MAX_DIMS 8
int veda_st_open(const char* path, veda_st_file** out);
void veda_st_close(veda_st_file* file);
int64_t veda_st_count(const veda_st_file* file);
int veda_st_info(const veda_st_file* file, int64_t i, const char** name, int32_t* dtype,
                 int32_t* ndim, int64_t* shape /* [VEDA_ST_MAX_DIMS] */, int64_t* nbytes);
/* index of the tensor called name, or VEDA_ERANGE when there is none */
int64_t veda_st_find(const veda_st_file* file, const char* name);
int veda_st_read(const veda_st_file* file, int64_t i, void* dst_host, int64_t nbytes);
int64_t veda_st_metadata_count(const veda_st_file* file);
int veda_st_metadata_at(const veda_st_file* file, int64_t i, const char** key, const char** value);

#ifdef __cplusplus
}
#endif
#endif /* VEDA_H */
