/*
 * librelattn: fused forward of relation-aware self-attention on AMD MI355X
 * (gfx950), plus the T5 bucketed scalar-bias variant and the related
 * operators listed below.
 *
 * What is computed (one head; q_i, k_j, v_j are rows of q, k, v):
 *
 *   Shaw et al. ("Self-Attention with Relative Position Representations",
 *   section 3.4, Eq. 3 and Eq. 4, with the tables of section "Relative Position
 *   Representations: From Arbitrary Edges to Sequences"):
 *       r(i, j) = clip(j - i, k) = max(-k, min(k, j - i))
 *       e_ij    = scale * q_i . (k_j + wK[r(i, j) + k])
 *       alpha   = softmax over the visible keys j of e_i.
 *       z_i     = sum_j alpha_ij * (v_j + wV[r(i, j) + k])
 *     A missing table (NULL) counts as all zeros.  scale <= 0 selects
 *     1/sqrt(d).  The scale multiplies both terms of e (Eq. 5); wV is unscaled.
 *
 *   T5 ("Relative position embeddings", section "T5"):
 *       e_ij = scale * q_i . k_j + bias[beta(j - i), h],  scale <= 0 selects 1
 *     where beta is the bucket function of that section.  Bidirectional: half
 *     = num_buckets/2 buckets per sign, keys after the query (j > i) use the
 *     upper half; unidirectional: all buckets for j <= i, bucket 0 for j > i.
 *     B_exact = half/2; the floor in beta is taken of the exact real value.
 *
 *   Around these, each declared below with its own formula: incremental
 *   decoding against a key/value cache (relattn_decode, _offset_bias, _xl), a
 *   scalar bias by clipped offset such as ALiBi (relattn_fwd_offset_bias), the
 *   backward with the table and bias gradients (relattn_bwd, _offset_bias),
 *   Transformer-XL relative logits (relattn_fwd_xl), the 2-D window bias of
 *   windowed vision models (relattn_fwd_grid_bias), and per-pair edge labels as a
 *   scalar bias (relattn_fwd_edge_bias) or with key and value tables
 *   (relattn_fwd_edge_tables); each of these forwards has an _lse variant and a
 *   backward (relattn_bwd_xl, _grid_bias, _edge_bias, _edge_tables).
 *
 *   Masks (no page defines them): causal hides keys j > i; key_lens[b] hides
 *   keys j >= key_lens[b] (clamped to [0, n]) of batch b.  A hidden key adds
 *   neither v_j nor wV.  A query row with no visible key outputs zeros.
 *
 * Conventions for every entry point:
 *   - All tensor data pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing and keeps no state between calls; it is
 *     thread-safe.  Equal inputs give bit-identical outputs.
 *   - Entry points that launch kernels only enqueue work on `stream` (a
 *     hipStream_t, NULL = the default stream) and return.  Buffers must stay
 *     alive until the stream has passed that point.  Faults during execution surface at the caller's
 *     next synchronisation.
 *   - Return value: RELATTN_OK (0) or a negative relattn_status.  A message
 *     with the detail is kept per thread (relattn_last_error).  No exception or
 *     abort crosses this interface.
 */
#ifndef RELATTN_H
#define RELATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RELATTN_VERSION 1

typedef enum {
  RELATTN_OK = 0,
  RELATTN_ERR_INVALID_ARGUMENT = -1, /* null/shape/stride/parameter error     */
  RELATTN_ERR_UNSUPPORTED = -2,      /* valid, but outside what is built      */
  RELATTN_ERR_NO_DEVICE = -3,        /* no usable HIP device                  */
  RELATTN_ERR_LAUNCH_FAILED = -4     /* HIP reported an error at launch        */
} relattn_status;

/* RELATTN_U8 is taken only by the label matrix of relattn_fwd_edge_bias. */
typedef enum { RELATTN_F32 = 0, RELATTN_BF16 = 1, RELATTN_U8 = 2 } relattn_dtype;

/* A strided tensor view.  `stride` counts ELEMENTS, not bytes.  The last
 * dimension must be contiguous (stride 1).  Dimensions past `ndim` are ignored. */
typedef struct {
  void* data;          /* device pointer (may be NULL only if the view is empty) */
  int32_t dtype;       /* relattn_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} relattn_tensor;

typedef struct {
  int32_t causal;            /* nonzero: hide keys j > i                    */
  const int32_t* key_lens;   /* device int32[B] or NULL (all n keys visible) */
} relattn_mask;

typedef struct {
  int32_t num_buckets;       /* B of the T5 section; even when bidirectional */
  int32_t max_distance;      /* D_max; must exceed B_exact                   */
  int32_t bidirectional;     /* nonzero: split buckets by sign of j - i      */
} relattn_t5_params;

/*
 * relattn_fwd: enqueue the forward pass.
 *
 *   q, k, v, out : [B, H, n, d], one dtype (F32 or BF16), d in {16,32,64,128}.
 *                  Rows must start 16-byte aligned (data pointer and the
 *                  strides of dims 0..2 in bytes are multiples of 16).
 *   wK, wV       : Shaw tables [Ht, 2*clip_k + 1, d] of the same dtype, with
 *                  Ht = H (one table per head) or Ht = 1 (shared by all
 *                  heads).  Row r holds offset r - clip_k.  Either may be NULL.
 *   t5_bias, t5  : T5 bias table [num_buckets, H] (F32) and its parameters.
 *                  Given together or not at all; excludes wK and wV.
 *   clip_k       : k >= 0 of clip(j - i, k) (ignored for T5).
 *   scale        : logit scale; <= 0 picks 1/sqrt(d) (Shaw) or 1 (T5).
 *   mask         : NULL = no mask.
 *   stream       : hipStream_t to enqueue on (NULL = default stream).
 *
 * Errors: INVALID_ARGUMENT for inconsistent shapes, dtypes, strides or
 * parameters; UNSUPPORTED for a head size outside {16,32,64,128}, misaligned
 * rows, or a label window (2*clip_k+1, or 2n-1 when clip_k >= n) or T5 bias
 * window too large for on-chip memory; NO_DEVICE; LAUNCH_FAILED.  Empty
 * problems (B, H or n equal to 0) return RELATTN_OK and launch nothing.
 */
int relattn_fwd(const relattn_tensor* q, const relattn_tensor* k,
                const relattn_tensor* v, const relattn_tensor* wK,
                const relattn_tensor* wV, const relattn_tensor* t5_bias,
                const relattn_t5_params* t5, int32_t clip_k, float scale,
                const relattn_mask* mask, relattn_tensor* out, void* stream);

/* relattn_validate: the argument checks of relattn_fwd, run on the host only.
 * Makes no HIP call and touches no device memory, so it works without a GPU.
 * Returns the status relattn_fwd would return before launching. */
int relattn_validate(const relattn_tensor* q, const relattn_tensor* k,
                     const relattn_tensor* v, const relattn_tensor* wK,
                     const relattn_tensor* wV, const relattn_tensor* t5_bias,
                     const relattn_t5_params* t5, int32_t clip_k, float scale,
                     const relattn_mask* mask, const relattn_tensor* out);

/* relattn_debug_indices: write, for every offset delta = j - i in
 * [-(n-1), n-1], the integer index the kernels use for that offset into
 * out_dev[delta + n - 1] (device int32[2n-1]):
 *   t5 == NULL : the table row clip(delta, clip_k) + clip_k   (clip section)
 *   t5 != NULL : the bucket beta(delta)                       (T5 section)
 * computed on the device by the same functions the attention kernels use.
 * Enqueued on `stream`; same error codes as relattn_fwd. */
int relattn_debug_indices(int32_t n, int32_t clip_k, const relattn_t5_params* t5,
                          int32_t* out_dev, void* stream);

/*
 * relattn_fwd_offset_bias: attention with a scalar bias by clipped offset, the
 * T5 bias with its bucket table replaced by a function of the offset (survey
 * page "Relative position embeddings", section "Placement in the taxonomy";
 * ALiBi is bias[h, window + delta] = -m_h * |delta|):
 *
 *       e_ij = scale * q_i . k_j + bias[h', clip(j - i, window) + window]
 *
 *   q, k, v, out : as for relattn_fwd.
 *   bias         : [Hb, 2*window + 1] F32, Hb = H (one row per head) or 1
 *                  (shared); entry window + delta holds offset delta, and
 *                  offsets beyond +-window take the end entries.
 *   window       : >= 0.
 *   scale        : logit scale; <= 0 picks 1/sqrt(d).
 *   mask, stream : as for relattn_fwd.
 * Errors as for relattn_fwd; UNSUPPORTED when the window clipped to n - 1 does
 * not fit on chip (2*min(window, n-1)+1 entries).  No value term.
 */
int relattn_fwd_offset_bias(const relattn_tensor* q, const relattn_tensor* k,
                            const relattn_tensor* v, const relattn_tensor* bias,
                            int32_t window, float scale, const relattn_mask* mask,
                            relattn_tensor* out, void* stream);

/*
 * relattn_fwd_xl: Transformer-XL relative logits (the transformer-xl page's
 * four-term score; survey page, section "Transformer-XL"):
 *
 *       e_ij = scale * [ q_i.k_j + q_i.R_{i-j} + u.k_j + v.R_{i-j} ]
 *            = scale * [ (q_i + u).k_j + (q_i + v).R_{i-j} ]
 *
 *   q, k, v, out : as for relattn_fwd.  No value term: z_i = sum_j alpha_ij v_j.
 *   R            : [Hr, 2*window + 1, d] position table (the projected
 *                  relative encodings W_R r), dtype of q, Hr in {H, 1}; row
 *                  window + (i - j) holds distance i - j; distances beyond
 *                  +-window take the end rows (window >= n - 1 clips nothing).
 *   u, vb        : [Hu, d] global biases (dtype of q, Hu in {H, 1}, rows
 *                  16-byte aligned): u for the content logit, vb for the
 *                  relative logit.  q + u and q + vb are rounded once to the
 *                  input dtype.
 *   scale        : multiplies the whole score; <= 0 picks 1/sqrt(d).
 *   mask, stream : as for relattn_fwd.
 * The segment memory of Transformer-XL (keys longer than the queries) is not
 * part of this call.  Errors as for relattn_fwd.
 */
int relattn_fwd_xl(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                   const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                   int32_t window, float scale, const relattn_mask* mask, relattn_tensor* out,
                   void* stream);

/* relattn_validate_xl: the argument checks of relattn_fwd_xl, host only. */
int relattn_validate_xl(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                        const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                        int32_t window, float scale, const relattn_mask* mask,
                        const relattn_tensor* out);

/*
 * relattn_fwd_grid_bias: a relative position bias on an M x M window of
 * tokens (survey page "Relative position embeddings", Swin paragraph: the T5
 * scalar bias ported to a grid, the table indexed by the flattened 2-D offset):
 *
 *       e_ij = scale * q_i.k_j + bias[h', (y_j - y_i + M - 1)(2M - 1) + (x_j - x_i + M - 1)]
 *
 *   with token p at (y, x) = (p / M, p % M), raster order, n = M * M.
 *   q, k, v, out : as for relattn_fwd; the batch dimension holds the windows.
 *   bias         : [Hb, (2M-1)^2] F32, Hb in {H, 1}.
 *   window_side  : M >= 1 (at most 2048).
 *   scale        : <= 0 picks 1/sqrt(d).
 *   mask         : key lengths only; a causal mask is INVALID_ARGUMENT.
 * Errors as for relattn_fwd.  No value term.
 */
int relattn_fwd_grid_bias(const relattn_tensor* q, const relattn_tensor* k,
                          const relattn_tensor* v, const relattn_tensor* bias,
                          int32_t window_side, float scale, const relattn_mask* mask,
                          relattn_tensor* out, void* stream);

/* relattn_validate_grid_bias: the argument checks of relattn_fwd_grid_bias,
 * host only. */
int relattn_validate_grid_bias(const relattn_tensor* q, const relattn_tensor* k,
                               const relattn_tensor* v, const relattn_tensor* bias,
                               int32_t window_side, float scale, const relattn_mask* mask,
                               const relattn_tensor* out);

/*
 * relattn_fwd_edge_bias: a scalar bias indexed by a label given per (query,
 * key) pair ("Self-Attention with Relative Position Representations", summary
 * page: the input as a labeled, directed, fully connected graph whose edge
 * labels need not be positions; survey page "Relative position embeddings",
 * section "Placement in the taxonomy": the bias looked up per pair):
 *
 *       e_ij = scale * q_i.k_j + bias[h', labels[b, i, j]]
 *
 *   q, k, v, out : as for relattn_fwd.  No value term.
 *   labels       : [B, n, n] U8 device matrix, the label of the edge from query
 *                  i to key j, shared by the heads of a batch entry.  Rows are
 *                  read in whole 16-byte chunks: the data pointer is 16-byte
 *                  aligned, stride[0] and stride[1] are multiples of 16 (stride[0]
 *                  may be 0: one matrix for all batch entries), stride[1] >= n
 *                  rounded up to 16, stride[2] = 1, and every row is readable up to
 *                  that rounded length (bytes past column n - 1 are read, never
 *                  used).  A label >= NL is read as NL - 1.
 *   bias         : [Hb, NL] F32, Hb in {H, 1}, 1 <= NL <= 256.
 *   scale        : multiplies q.k only; <= 0 picks 1/sqrt(d).
 *   mask, stream : as for relattn_fwd.
 * Errors as for relattn_fwd; a layout of labels outside the rules above is
 * UNSUPPORTED.
 */
int relattn_fwd_edge_bias(const relattn_tensor* q, const relattn_tensor* k,
                          const relattn_tensor* v, const relattn_tensor* labels,
                          const relattn_tensor* bias, float scale, const relattn_mask* mask,
                          relattn_tensor* out, void* stream);

/* relattn_validate_edge_bias: the argument checks of relattn_fwd_edge_bias,
 * host only. */
int relattn_validate_edge_bias(const relattn_tensor* q, const relattn_tensor* k,
                               const relattn_tensor* v, const relattn_tensor* labels,
                               const relattn_tensor* bias, float scale,
                               const relattn_mask* mask, const relattn_tensor* out);

/*
 * relattn_fwd_edge_tables: relation-aware self-attention over a labeled graph
 * ("Self-Attention with Relative Position Representations", summary page: Eq. 4
 * and Eq. 3 with the edge representations a^K_ij, a^V_ij taken from the label
 * of the pair, which need not be a clipped offset):
 *
 *       e_ij = scale * q_i.(k_j + wK[h', E_ij]),   z_i = sum_j alpha_ij (v_j + wV[h', E_ij])
 *
 *   with E_ij = labels[b, i, j].
 *   q, k, v, out : as for relattn_fwd.
 *   labels       : [B, n, n] U8, the layout rules of relattn_fwd_edge_bias; a
 *                  label >= NL is read as NL - 1.
 *   wK, wV       : [Ht, NL, d] in the dtype of q, Ht in {H, 1}, 1 <= NL <= 256
 *                  (the same NL for both); either may be NULL (absent = zero),
 *                  not both.  Rows 16-byte aligned as for relattn_fwd's tables.
 *   scale        : multiplies both terms of the logit; <= 0 picks 1/sqrt(d).
 *   mask, stream : as for relattn_fwd.
 * Errors as for relattn_fwd; UNSUPPORTED when the NL-entry rows of a workgroup's
 * queries do not fit on chip.
 */
int relattn_fwd_edge_tables(const relattn_tensor* q, const relattn_tensor* k,
                            const relattn_tensor* v, const relattn_tensor* labels,
                            const relattn_tensor* wK, const relattn_tensor* wV, float scale,
                            const relattn_mask* mask, relattn_tensor* out, void* stream);

/* relattn_validate_edge_tables: the argument checks of relattn_fwd_edge_tables,
 * host only. */
int relattn_validate_edge_tables(const relattn_tensor* q, const relattn_tensor* k,
                                 const relattn_tensor* v, const relattn_tensor* labels,
                                 const relattn_tensor* wK, const relattn_tensor* wV, float scale,
                                 const relattn_mask* mask, const relattn_tensor* out);

/* relattn_validate_offset_bias: the argument checks of relattn_fwd_offset_bias,
 * host only (no HIP call). */
int relattn_validate_offset_bias(const relattn_tensor* q, const relattn_tensor* k,
                                 const relattn_tensor* v, const relattn_tensor* bias,
                                 int32_t window, float scale, const relattn_mask* mask,
                                 const relattn_tensor* out);

/*
 * relattn_decode: incremental decoding.  The newest Tq positions of each
 * sequence attend over its key/value cache with the causal mask; each output
 * row is the row relattn_fwd would compute for that position with causal = 1
 * (same formulas, tables and T5 bias as above).
 *
 *   q, out       : [B, H, Tq, d].  Query t of batch b sits at position
 *                  i = cache_lens[b] - Tq + t and sees the keys j <= i.
 *   k, v         : [B, H, L, d] caches, L >= 1 rows; rows j < cache_lens[b]
 *                  must hold the keys and values of positions 0..j (the new
 *                  positions included); later rows are never read.
 *   wK, wV, t5_bias, t5, clip_k, scale: as for relattn_fwd.
 *   cache_lens   : device int32[B] (4-byte aligned), clamped to [0, L]; NULL
 *                  means L for every batch.  A query whose position is
 *                  negative (cache_lens[b] < Tq - t) sees no key and outputs
 *                  zeros.
 *   workspace    : device buffer of at least workspace_bytes, 16-byte
 *                  aligned, owned by the caller; its contents on entry do not
 *                  matter and are overwritten.  Its size comes from
 *                  relattn_decode_workspace_size (0 for empty problems, where
 *                  NULL is accepted).  Calls that share a workspace must be
 *                  ordered (same stream).
 *   stream       : hipStream_t to enqueue on (NULL = default stream).
 *
 * Dtypes, head sizes, alignment and error codes as for relattn_fwd; the
 * cache may be longer than 65535 * 32768 / (d * element bytes) rows only
 * with UNSUPPORTED.  Enqueues two kernels and returns.
 */
int relattn_decode(const relattn_tensor* q, const relattn_tensor* k,
                   const relattn_tensor* v, const relattn_tensor* wK,
                   const relattn_tensor* wV, const relattn_tensor* t5_bias,
                   const relattn_t5_params* t5, int32_t clip_k, float scale,
                   const int32_t* cache_lens, relattn_tensor* out,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * relattn_decode_noalloc: relattn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results, dtypes and errors as
 * relattn_decode, without workspace: the split rows' partial results go to a
 * static scratch array of 4 MiB that the library holds on each device it runs
 * on until the process ends.  Shapes whose relattn_decode_workspace_size
 * exceeds 4 MiB return RELATTN_ERR_UNSUPPORTED.  The call allocates nothing
 * (no hipMalloc, no hipFree).  Every call on a device shares that device's
 * scratch, whose contents on entry do not matter: calls on one device that
 * overlap in time (different streams, or different host threads without
 * ordering) race and must be serialised by the caller.  The first call on a
 * device resolves that device's copy of the array (hipGetSymbolAddress).
 */
int relattn_decode_noalloc(const relattn_tensor* q, const relattn_tensor* k,
                           const relattn_tensor* v, const relattn_tensor* wK,
                           const relattn_tensor* wV, const relattn_tensor* t5_bias,
                           const relattn_t5_params* t5, int32_t clip_k, float scale,
                           const int32_t* cache_lens, relattn_tensor* out, void* stream);

/*
 * relattn_decode_xl: incremental decoding with Transformer-XL relative logits
 * (the transformer-xl page's four-term score; the newest positions attend over
 * everything before them):
 *
 *       e_j = scale * [ (q + u).k_j + (q + vb).R_{i-j} ],  j <= i
 *
 *   q, k, v, out, cache_lens, workspace, stream : as for relattn_decode.
 *   R, u, vb, window : as for relattn_fwd_xl (R [Hr, 2*window + 1, d], row
 *                  window + (i - j); u, vb [Hu, d]; q + u and q + vb rounded
 *                  once to the input dtype).
 *   scale        : multiplies the whole score; <= 0 picks 1/sqrt(d).
 * relattn_decode_xl_workspace_size gives the workspace bytes.  Errors as for
 * relattn_decode.  No value term; the segment memory is the cache itself.
 */
int relattn_decode_xl(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                      const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                      int32_t window, float scale, const int32_t* cache_lens, relattn_tensor* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* relattn_decode_xl_workspace_size: host only; *bytes receives the workspace
 * relattn_decode_xl needs for these shapes (0 when none). */
int relattn_decode_xl_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                     const relattn_tensor* v, const relattn_tensor* R,
                                     const relattn_tensor* u, const relattn_tensor* vb,
                                     int32_t window, float scale, const relattn_tensor* out,
                                     size_t* bytes);

/*
 * relattn_decode_offset_bias: incremental decoding with a scalar bias by clipped
 * offset (survey page "Relative position embeddings", section "Placement in
 * the taxonomy": ALiBi is the bias -m_h |delta| written as such a table):
 *
 *       e_j = scale * q.k_j + bias[h', clip(j - i, window) + window],  j <= i
 *
 *   q, k, v, out, cache_lens, workspace, stream : as for relattn_decode (query t
 *                  of batch b at position len_b - Tq + t over keys 0 .. that
 *                  position).
 *   bias         : [Hb, 2*window + 1] F32, Hb in {H, 1}; window >= 0.
 *   scale        : multiplies q.k only; <= 0 picks 1/sqrt(d).
 * relattn_decode_offset_bias_workspace_size gives the workspace bytes.  Errors
 * as for relattn_decode.  No value term.
 */
int relattn_decode_offset_bias(const relattn_tensor* q, const relattn_tensor* k,
                               const relattn_tensor* v, const relattn_tensor* bias, int32_t window,
                               float scale, const int32_t* cache_lens, relattn_tensor* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* relattn_decode_offset_bias_workspace_size: host only; *bytes receives the
 * workspace relattn_decode_offset_bias needs for these shapes (0 when none). */
int relattn_decode_offset_bias_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                              const relattn_tensor* v, const relattn_tensor* bias,
                                              int32_t window, float scale,
                                              const relattn_tensor* out, size_t* bytes);

/* relattn_decode_workspace_size: the argument checks of relattn_decode (host
 * only: no HIP call, works without a GPU) and the workspace it needs, written
 * to *bytes.  The size depends only on the shapes, dtype and tables. */
int relattn_decode_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                  const relattn_tensor* v, const relattn_tensor* wK,
                                  const relattn_tensor* wV,
                                  const relattn_tensor* t5_bias,
                                  const relattn_t5_params* t5, int32_t clip_k,
                                  float scale, const relattn_tensor* out,
                                  size_t* bytes);

/*
 * Training.  The backward pass needs each query row's log-sum-exp of its
 * logits, lse_i = log sum_{visible j} exp(e_ij) (natural log; -inf for a row
 * that sees no key), which these forward variants also write:
 *
 * relattn_fwd_lse / relattn_fwd_offset_bias_lse: relattn_fwd /
 *   relattn_fwd_offset_bias plus lse: [B, H, n] F32, innermost dimension
 *   contiguous, device memory owned by the caller.  Same errors.
 */
int relattn_fwd_lse(const relattn_tensor* q, const relattn_tensor* k,
                    const relattn_tensor* v, const relattn_tensor* wK,
                    const relattn_tensor* wV, const relattn_tensor* t5_bias,
                    const relattn_t5_params* t5, int32_t clip_k, float scale,
                    const relattn_mask* mask, relattn_tensor* out, relattn_tensor* lse,
                    void* stream);
int relattn_fwd_offset_bias_lse(const relattn_tensor* q, const relattn_tensor* k,
                                const relattn_tensor* v, const relattn_tensor* bias,
                                int32_t window, float scale, const relattn_mask* mask,
                                relattn_tensor* out, relattn_tensor* lse, void* stream);

/*
 * relattn_bwd: enqueue the backward pass: the gradients of a scalar loss L
 * given dout = dL/dz for the attention relattn_fwd_lse computed (Eq. 3 and
 * Eq. 4 of the Shaw section 3.4, or the T5 bias, differentiated by the chain
 * rule; the papers train these models end to end).  With P the weights,
 * dP_ij = dout_i.(v_j + wV[r]), D_i = dout_i.z_i and dS_ij = P_ij (dP_ij - D_i):
 *     dq_i = s sum_j dS_ij (k_j + wK[r])    dk_j = s sum_i dS_ij q_i
 *     dv_j = sum_i P_ij dout_i
 *     dwK[r] = s sum over pairs of label r of dS_ij q_i
 *     dwV[r] = sum over pairs of label r of P_ij dout_i
 *     dbias[beta, h] = sum over pairs of bucket beta of dS_ij
 * Table gradients of a shared table (Ht = 1) sum over the heads.  Pairs that
 * are hidden by the mask contribute nothing.
 *
 *   q .. mask      : exactly the arguments of the forward call.
 *   out, lse       : that call's output and row log-sum-exp (unchanged).
 *   dout           : [B, H, n, d], dtype and alignment of q.
 *   dq, dk, dv     : outputs like q (16-byte aligned rows).
 *   dwK, dwV       : outputs [Ht, 2*clip_k + 1, d] F32 (innermost contiguous),
 *                    or NULL to skip; a non-NULL one needs its table.  Rows of
 *                    labels no pair reaches are set to zero.
 *   dbias          : output like t5_bias (F32), or NULL to skip.
 *   workspace      : device buffer of at least the bytes that
 *                    relattn_bwd_workspace_size reports (16-byte aligned,
 *                    caller-owned; contents on entry do not matter).  Calls
 *                    that share a workspace must be ordered (same stream).
 * All outputs are fully overwritten; the results are bitwise reproducible
 * (no atomics).  Errors as for relattn_fwd; UNSUPPORTED also when the
 * per-workgroup state of the label window (or of the T5 buckets) does not
 * fit on chip.  Enqueues up to three kernels and returns.
 */
int relattn_bwd(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                const relattn_tensor* wK, const relattn_tensor* wV,
                const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
                float scale, const relattn_mask* mask, const relattn_tensor* out,
                const relattn_tensor* dout, const relattn_tensor* lse, relattn_tensor* dq,
                relattn_tensor* dk, relattn_tensor* dv, relattn_tensor* dwK,
                relattn_tensor* dwV, relattn_tensor* dbias, void* workspace,
                size_t workspace_bytes, void* stream);

/* relattn_bwd_workspace_size: the argument checks of relattn_bwd (host only:
 * no HIP call) and the workspace bytes it needs, written to *bytes (0 for
 * empty problems).  Depends only on shapes, dtype, tables and mask kind. */
int relattn_bwd_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                               const relattn_tensor* v, const relattn_tensor* wK,
                               const relattn_tensor* wV, const relattn_tensor* t5_bias,
                               const relattn_t5_params* t5, int32_t clip_k, float scale,
                               const relattn_mask* mask, const relattn_tensor* out,
                               const relattn_tensor* dout, const relattn_tensor* lse,
                               const relattn_tensor* dq, const relattn_tensor* dk,
                               const relattn_tensor* dv, const relattn_tensor* dwK,
                               const relattn_tensor* dwV, const relattn_tensor* dbias,
                               size_t* bytes);

/* relattn_bwd_offset_bias and its workspace size: the same for
 * relattn_fwd_offset_bias_lse; dbias is [Hb, 2*window + 1] F32 or NULL (e.g.
 * fixed ALiBi slopes).  A bias gradient needs per-workgroup sums over
 * 2*min(window, n-1)+1 entries on chip: larger windows give UNSUPPORTED
 * unless dbias is NULL. */
int relattn_bwd_offset_bias(const relattn_tensor* q, const relattn_tensor* k,
                            const relattn_tensor* v, const relattn_tensor* bias,
                            int32_t window, float scale, const relattn_mask* mask,
                            const relattn_tensor* out, const relattn_tensor* dout,
                            const relattn_tensor* lse, relattn_tensor* dq, relattn_tensor* dk,
                            relattn_tensor* dv, relattn_tensor* dbias, void* workspace,
                            size_t workspace_bytes, void* stream);
int relattn_bwd_offset_bias_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                           const relattn_tensor* v, const relattn_tensor* bias,
                                           int32_t window, float scale,
                                           const relattn_mask* mask, const relattn_tensor* out,
                                           const relattn_tensor* dout,
                                           const relattn_tensor* lse, const relattn_tensor* dq,
                                           const relattn_tensor* dk, const relattn_tensor* dv,
                                           const relattn_tensor* dbias, size_t* bytes);

/* relattn_fwd_grid_bias_lse, relattn_bwd_grid_bias and its workspace size: the
 * same for the 2-D window bias of relattn_fwd_grid_bias (survey page "Relative
 * position embeddings", Swin paragraph), differentiated by the chain rule:
 *     dbias[h', e] = sum over the heads h' covers, the windows and the pairs
 *                    (i, j) whose 2-D offset is entry e of dS_ij
 * lse as for relattn_fwd_lse; dbias is [Hb, (2M-1)^2] F32 or NULL.  The
 * backward holds the head's (2M-1)^2 entries on chip, and with dbias a
 * per-wave sum over them: large windows give UNSUPPORTED (head size 64 in
 * BF16: M up to 40 with dbias, 74 without). */
int relattn_fwd_grid_bias_lse(const relattn_tensor* q, const relattn_tensor* k,
                              const relattn_tensor* v, const relattn_tensor* bias,
                              int32_t window_side, float scale, const relattn_mask* mask,
                              relattn_tensor* out, relattn_tensor* lse, void* stream);
int relattn_bwd_grid_bias(const relattn_tensor* q, const relattn_tensor* k,
                          const relattn_tensor* v, const relattn_tensor* bias,
                          int32_t window_side, float scale, const relattn_mask* mask,
                          const relattn_tensor* out, const relattn_tensor* dout,
                          const relattn_tensor* lse, relattn_tensor* dq, relattn_tensor* dk,
                          relattn_tensor* dv, relattn_tensor* dbias, void* workspace,
                          size_t workspace_bytes, void* stream);
int relattn_bwd_grid_bias_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                         const relattn_tensor* v, const relattn_tensor* bias,
                                         int32_t window_side, float scale,
                                         const relattn_mask* mask, const relattn_tensor* out,
                                         const relattn_tensor* dout,
                                         const relattn_tensor* lse, const relattn_tensor* dq,
                                         const relattn_tensor* dk, const relattn_tensor* dv,
                                         const relattn_tensor* dbias, size_t* bytes);

/* relattn_fwd_edge_bias_lse, relattn_bwd_edge_bias and its workspace size: the
 * same for the scalar bias by per-pair edge label of relattn_fwd_edge_bias
 * (summary page of "Self-Attention with Relative Position Representations",
 * the labeled-graph reading; survey page, "Placement in the taxonomy"),
 * differentiated by the chain rule:
 *     dbias[h', l] = sum over the heads h' covers, the batch and the pairs
 *                    (i, j) labelled l of dS_ij
 * labels and their layout rules as for relattn_fwd_edge_bias (a label >= NL
 * counts as NL - 1 here too); lse as for relattn_fwd_lse; dbias is [Hb, NL]
 * F32 or NULL, and a label no visible pair carries gets 0.  The backward
 * holds the head's NL entries on chip, and with dbias one sum over them per
 * query and lane half: tables too long for on-chip memory give UNSUPPORTED
 * (every NL up to 256 fits, except BF16 at head size 64 with dbias: NL up to
 * 253). */
int relattn_fwd_edge_bias_lse(const relattn_tensor* q, const relattn_tensor* k,
                              const relattn_tensor* v, const relattn_tensor* labels,
                              const relattn_tensor* bias, float scale, const relattn_mask* mask,
                              relattn_tensor* out, relattn_tensor* lse, void* stream);
int relattn_bwd_edge_bias(const relattn_tensor* q, const relattn_tensor* k,
                          const relattn_tensor* v, const relattn_tensor* labels,
                          const relattn_tensor* bias, float scale, const relattn_mask* mask,
                          const relattn_tensor* out, const relattn_tensor* dout,
                          const relattn_tensor* lse, relattn_tensor* dq, relattn_tensor* dk,
                          relattn_tensor* dv, relattn_tensor* dbias, void* workspace,
                          size_t workspace_bytes, void* stream);
int relattn_bwd_edge_bias_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                         const relattn_tensor* v, const relattn_tensor* labels,
                                         const relattn_tensor* bias, float scale,
                                         const relattn_mask* mask, const relattn_tensor* out,
                                         const relattn_tensor* dout,
                                         const relattn_tensor* lse, const relattn_tensor* dq,
                                         const relattn_tensor* dk, const relattn_tensor* dv,
                                         const relattn_tensor* dbias, size_t* bytes);

/* relattn_fwd_xl_lse, relattn_bwd_xl and its workspace size: the same for the
 * Transformer-XL logits of relattn_fwd_xl ("Relative Position Encoding in
 * Transformer-XL", the four-term score), differentiated by the chain rule with
 * the score written as s [(q_i + u).k_j + (q_i + v).R_{i-j}]:
 *     dq_i = s sum_j dS_ij (k_j + R_{i-j})     dk_j = s sum_i dS_ij (q_i + u)
 *     dR_r = s sum over pairs at row r of dS_ij (q_i + v)
 *     du = s sum_ij dS_ij k_j                  dv = s sum_ij dS_ij R_{i-j}
 * (dv here is the gradient of the position bias v; the value gradient is the
 * argument dv of relattn_bwd's list, named dv as there).
 *   q .. mask      : exactly the arguments of the forward call.
 *   dR             : [Hr, 2*window + 1, d] F32 (innermost contiguous), or NULL.
 *   du, dvb        : [Hu, d] and [Hv, d] F32 (innermost contiguous), or NULL.
 * A shared R, u or v (leading dimension 1) gets the sum over the heads; rows
 * of distances no pair reaches are set to zero.  The backward holds one row
 * of relative logits per query over the reachable distances on chip:
 * distances past what fits give UNSUPPORTED (bf16 at d = 64: every distance
 * of a 512-token causal segment fits, with one wave per query tile).
 * Errors, workspace and reproducibility as for relattn_bwd. */
int relattn_fwd_xl_lse(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                       const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                       int32_t window, float scale, const relattn_mask* mask, relattn_tensor* out,
                       relattn_tensor* lse, void* stream);
int relattn_bwd_xl(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                   const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                   int32_t window, float scale, const relattn_mask* mask,
                   const relattn_tensor* out, const relattn_tensor* dout,
                   const relattn_tensor* lse, relattn_tensor* dq, relattn_tensor* dk,
                   relattn_tensor* dv, relattn_tensor* dR, relattn_tensor* du,
                   relattn_tensor* dvb, void* workspace, size_t workspace_bytes, void* stream);
int relattn_bwd_xl_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                  const relattn_tensor* v, const relattn_tensor* R,
                                  const relattn_tensor* u, const relattn_tensor* vb,
                                  int32_t window, float scale, const relattn_mask* mask,
                                  const relattn_tensor* out, const relattn_tensor* dout,
                                  const relattn_tensor* lse, const relattn_tensor* dq,
                                  const relattn_tensor* dk, const relattn_tensor* dv,
                                  const relattn_tensor* dR, const relattn_tensor* du,
                                  const relattn_tensor* dvb, size_t* bytes);

/* relattn_fwd_edge_tables_lse, relattn_bwd_edge_tables and its workspace size:
 * the same for relation-aware attention over a labeled graph,
 * relattn_fwd_edge_tables (summary page of "Self-Attention with Relative
 * Position Representations", Eq. 3 and Eq. 4 with each pair's table rows read
 * by its label), differentiated by the chain rule as relattn_bwd does for the
 * clipped offset:
 *     dwK[l] = s sum over the pairs labelled l of dS_ij q_i
 *     dwV[l] = sum over the pairs labelled l of P_ij dout_i
 * labels and tables as for relattn_fwd_edge_tables (a label >= NL counts as
 * NL - 1); dwK, dwV: [Ht, NL, d] F32 (innermost contiguous) or NULL, a NULL
 * one needing no table.  The dq workgroup keeps, per query row, the label sums
 * of dS and of P on chip: tables too long give UNSUPPORTED (key and value
 * tables in bf16 at d = 64: NL up to 64).  Errors, workspace and
 * reproducibility as for relattn_bwd. */
int relattn_fwd_edge_tables_lse(const relattn_tensor* q, const relattn_tensor* k,
                                const relattn_tensor* v, const relattn_tensor* labels,
                                const relattn_tensor* wK, const relattn_tensor* wV, float scale,
                                const relattn_mask* mask, relattn_tensor* out,
                                relattn_tensor* lse, void* stream);
int relattn_bwd_edge_tables(const relattn_tensor* q, const relattn_tensor* k,
                            const relattn_tensor* v, const relattn_tensor* labels,
                            const relattn_tensor* wK, const relattn_tensor* wV, float scale,
                            const relattn_mask* mask, const relattn_tensor* out,
                            const relattn_tensor* dout, const relattn_tensor* lse,
                            relattn_tensor* dq, relattn_tensor* dk, relattn_tensor* dv,
                            relattn_tensor* dwK, relattn_tensor* dwV, void* workspace,
                            size_t workspace_bytes, void* stream);
int relattn_bwd_edge_tables_workspace_size(
    const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
    const relattn_tensor* labels, const relattn_tensor* wK, const relattn_tensor* wV, float scale,
    const relattn_mask* mask, const relattn_tensor* out, const relattn_tensor* dout,
    const relattn_tensor* lse, const relattn_tensor* dq, const relattn_tensor* dk,
    const relattn_tensor* dv, const relattn_tensor* dwK, const relattn_tensor* dwV,
    size_t* bytes);

/* Static text for a status code. */
const char* relattn_strerror(int status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* relattn_last_error(void);

/* RELATTN_VERSION of the built library. */
int relattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RELATTN_H */
