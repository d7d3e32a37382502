/*
 * lacache.h -- C ABI of the exact layer-0 cached block step (LaCache) on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (LaCache, "Exact Caching and Precision-Adaptive Inference for
 * Diffusion Large Language Models", arXiv 2607.16339):
 *   - Section 3.3.1 (Notation): a sequence of N tokens; C is the current
 *     block [block_start, block_end); U is every other token.
 *   - Section 3.3.2, Eq. (1): EmbedCache H = Embed(x) and RoPECache
 *     Q, K = RoPE(Norm(H) W_{Q,K}), V = Norm(H) W_V, recomputed for C only.
 *   - Section 3.3.3, Eqs. (2)-(6): FACache, the online-softmax state
 *     (m, l, O~) of every row of U over the keys of U; in later steps a row of
 *     U starts from that state and streams only the keys of C.
 *   - Algorithm 1 ("the first layer's Flash-Attention"): output O and the
 *     log-sum-exp L of every row; the cache is written at the first step of a
 *     block only.
 * The block-row attention over [prefix | fresh block | suffix] keys is the
 * inner step of Fast-dLLM's block-wise DualCache (DantinoX documentation,
 * "Block-wise Generation" and "Building the Dual Cache Manually"); the flat,
 * pre-allocated, token-major cache with a per-sample block table follows the
 * Flash-dLLM article ("Flash-Cache", block table and flat cache layout).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every device buffer is owned by the caller and stays owned by the
 *   caller.  The library keeps only the context (configuration, a device
 *   RoPE table and a device status word, allocated by lacache_create).
 *   Pointers marked "device" must be device memory aligned to 16 bytes;
 *   pointers marked "host" are read before the call returns.
 * Layouts (row-major, token-major, one flat buffer for the whole batch):
 *   embed  [vocab, d_model]                   dtype
 *   gamma  [d_model]                          dtype
 *   w_qkv  [(H + 2 H_kv) d_h, d_model]        dtype; output features of the Q
 *          heads, then K heads, then V heads, each head's d_h rows contiguous
 *   h      [n_rows, d_model]                  dtype  (EmbedCache)
 *   q      [n_rows, H, d_h]                   ctype  (RoPECache, after RoPE)
 *   k, v   [n_rows, H_kv, d_h]                ctype  (RoPECache; v not rotated)
 *   m, l   [n_rows, H]                        fp32   (FACache running max in
 *          natural-log units of the scaled scores, and normaliser)
 *   o      [n_rows, H, d_h]                   ctype  (FACache output O~ / l: the
 *          unnormalised accumulator divided by the normaliser l)
 *   out    [n_rows, H, d_h]                   dtype
 *   lse    [n_rows, H]                        fp32   (natural log)
 *   dtype is fp32 or bf16 (lacache_config.dtype).  ctype, the RoPECache
 *   element type, is fp32 for fp32 and IEEE fp16 for bf16: fp16 carries 3 more
 *   mantissa bits than bf16 at the same size and MFMA rate (magnitudes above
 *   65504 set LACACHE_DEVFLAG_CACHE_RANGE).  Sample b owns rows
 *   seq_offset .. seq_offset + seq_len - 1; its token positions are
 *   0 .. seq_len - 1 (layout [prompt | block 0 | ...]).  Keys never cross
 *   samples.
 * Streams.  `stream` is a hipStream_t (NULL: the default stream).  Every
 *   compute call only enqueues kernels on it and returns; results are valid
 *   once the stream has reached them.  No call synchronises the device,
 *   except lacache_read_device_status.
 * Errors.  Arguments are validated before anything is enqueued; on an error
 *   nothing is launched, the status is returned and lacache_last_error(ctx)
 *   describes it.  A failed launch returns LACACHE_ERR_HIP.  Token ids are
 *   device data and cannot be checked on the host: an id outside
 *   [0, vocab) is read as an all-zero embedding row and sets
 *   LACACHE_DEVFLAG_BAD_TOKEN_ID in the context's device status word.
 * Threads.  Calls on different contexts are independent.  One context may
 *   be used from several threads if each call has its own workspace and
 *   stream; lacache_last_error then reports whichever call failed last.
 */
#ifndef LACACHE_H
#define LACACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef LACACHE_API
#define LACACHE_API __attribute__((visibility("default")))
#endif

typedef enum {
  LACACHE_OK = 0,
  LACACHE_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, bad block table */
  LACACHE_ERR_UNSUPPORTED = 2,   /* valid request this build does not serve  */
  LACACHE_ERR_WORKSPACE = 3,     /* workspace missing or too small           */
  LACACHE_ERR_HIP = 4            /* a HIP runtime call or launch failed      */
} lacache_status;

typedef enum { LACACHE_F32 = 0, LACACHE_BF16 = 1 } lacache_dtype;

/* Device status flags (lacache_read_device_status). */
#define LACACHE_DEVFLAG_BAD_TOKEN_ID 1u
#define LACACHE_DEVFLAG_CACHE_RANGE 2u   /* a q/k/v value exceeded the fp16 range */
#define LACACHE_DEVFLAG_SEARCH_ORDER 4u  /* lacache_verify_accept: search positions not increasing
                                            or outside the sample (nothing accepted there) */

/* First-layer shape (Section 3.3.2).  Supported: head_dim 64 or 128,
 * d_model a multiple of 256 up to 8192, n_heads a multiple of n_kv_heads,
 * 1 <= max_seq_len <= 1<<20.  sm_scale <= 0 selects 1/sqrt(head_dim).
 * rope_theta > 0: feature i of a head is paired with feature i + d_h/2 and
 * rotated by position * rope_theta^(-2i/d_h).  rms_eps >= 0:
 * Norm(x) = gamma * x / sqrt(mean(x^2) + rms_eps). */
typedef struct {
  int32_t d_model;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t vocab;
  int32_t max_seq_len;
  float rope_theta;
  float rms_eps;
  float sm_scale;
  int32_t dtype;                  /* lacache_dtype */
} lacache_config;

/* Layer-0 parameters, device, layouts above.  w_qkv_packed is optional:
 * NULL, or w_qkv as converted by lacache_pack_qkv_weight.  Calls that
 * project 128 or more tokens at once (prefill, block steps with that many
 * block tokens; bf16 contexts with d_model a multiple of 512) then read it
 * instead of converting w_qkv to fp16 tile by tile inside the projection;
 * both forms hold the same fp16 values, and the projections differ only in
 * the order of the fp32 accumulation.  It must be packed from this w_qkv. */
typedef struct {
  const void *embed;
  const void *gamma;
  const void *w_qkv;
  const void *w_qkv_packed;
} lacache_weights;

/* The caches (device), layouts above; n_rows = rows every buffer holds. */
typedef struct {
  void *h;
  void *q;
  void *k;
  void *v;
  float *m;
  float *l;
  void *o;
  int64_t n_rows;
} lacache_cache;

/* One row of the block table (host): sample rows
 * [seq_offset, seq_offset + seq_len) and current block
 * [block_start, block_end) in positions of the sample.  Rules:
 * 0 <= block_start < block_end <= seq_len <= max_seq_len,
 * block_end - block_start <= 128, row ranges of different samples disjoint
 * and inside [0, n_rows), seq_offset + seq_len <= 2^31 - 1 (rows are indexed
 * in 32 bits; byte offsets into the buffers are 64-bit, so a buffer may hold
 * any number of bytes). */
typedef struct {
  int32_t seq_offset;
  int32_t seq_len;
  int32_t block_start;
  int32_t block_end;
} lacache_seq;

typedef struct lacache_ctx lacache_ctx;

/* Operations, for lacache_workspace_size. */
typedef enum {
  LACACHE_OP_PREFILL = 0,
  LACACHE_OP_BLOCK_STEP = 1,
  LACACHE_OP_DUALCACHE_ATTN = 2,
  LACACHE_OP_REFRESH_BLOCK = 3,    /* seqs: the table of the rows to re-project (proj) */
  LACACHE_OP_PROJECT_BLOCK = 4
} lacache_op;

/* Creates a context on the current HIP device: validates the configuration,
 * builds the RoPE cos/sin table (computed in double on the host, stored as
 * fp32 [max_seq_len, head_dim/2] pairs) and a device status word.  The
 * context must be used on that device only.  *out is NULL on failure.
 * Diagnostics: the environment variable LACACHE_SPLIT_KEYS (a multiple of
 * 32), read here, fixes the key chunk of the block rows' split-KV partials
 * for the context's lifetime instead of the per-call choice; results stay
 * within the parity tolerances, not bit-identical.  LACACHE_GEMM_TILE
 * ("whole", "half" or "wide"), also read here, fixes the tile of the
 * packed-weight projection GEMM used for 128 or more tokens (128 x 192,
 * 128 x 96 or 256 x 192 tokens x columns per workgroup) instead of the
 * choice by launch size; the results are the same up to fp32 summation
 * order (within the parity tolerances).  LACACHE_REFRESH_ROWS (64 or 128),
 * also read here, fixes the rows per workgroup of the bf16 refresh attention
 * instead of the choice by launch size (bit-identical results: the rows per
 * workgroup do not change any row's arithmetic).  LACACHE_LOG (non-empty and
 * not "0"), also read here, makes every later kernel launch of the process
 * print one line "lacache launch: <kernel instantiation> grid <workgroups>"
 * to stderr; unset or "0" by the next lacache_create switches it off. */
LACACHE_API lacache_status lacache_create(const lacache_config *cfg, lacache_ctx **out);

/* Frees the context's device memory (synchronises the device first).
 * NULL is accepted. */
LACACHE_API lacache_status lacache_destroy(lacache_ctx *ctx);

/* Bytes of device workspace an operation needs for this block table
 * (0 is possible).  seqs: host, `batch` rows.  The block step and the
 * DualCache attention keep partial softmax states of the block rows there:
 * per block row, head and chunk of keys a (max, normaliser) pair in fp32 and
 * d_h outputs in ctype; the chunk length is chosen per call from the table
 * (128 keys while that gives at most ~4 workgroups per CU, longer beyond). */
LACACHE_API lacache_status lacache_workspace_size(const lacache_ctx *ctx, int32_t op,
                                      const lacache_seq *seqs, int32_t batch,
                                      size_t *bytes);

/* Refresh at the first denoising step of a block (Section 3.3, "populated at
 * the first denoising step of each SAR block"; Algorithm 1 with its first-step
 * flag set): the full layer-0 forward of every row of every sample.
 *   ids      device int32 [n_rows]: token id of every row (rows outside all
 *            samples are not read).
 * Writes h, q, k, v for every row of every sample; m, l, o for every row
 * of U (the state over the keys of U only); out and lse (lse may be NULL) for
 * every row.  FACache rows of C are left unspecified. */
LACACHE_API lacache_status lacache_prefill_cache(lacache_ctx *ctx, const lacache_weights *w,
                                     const int32_t *ids, const lacache_seq *seqs,
                                     int32_t batch, const lacache_cache *cache,
                                     void *out, float *lse, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* One cached inner step (Section 3.3.2 and 3.3.3; Figure 3 right):
 *   block_ids device int32 [sum_b (block_end - block_start)]: the current
 *            ids of every sample's block, concatenated in sample order.
 * Writes h, q, k, v of the block rows only (EmbedCache / RoPECache update);
 * block rows attend over all keys of their sample; every row of U is finished
 * from its FACache state plus the block's keys.  Writes out and lse (may be
 * NULL) for every row of every sample.  Reads, never writes, the FACache.
 * The result equals a full recompute of layer 0 on the new ids, up to
 * rounding, provided the caches were filled by lacache_prefill_cache for the
 * same block table and only block ids changed since. */
LACACHE_API lacache_status lacache_block_step(lacache_ctx *ctx, const lacache_weights *w,
                                  const int32_t *block_ids, const lacache_seq *seqs,
                                  int32_t batch, const lacache_cache *cache,
                                  void *out, float *lse, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* lacache_block_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Its scratch (the split-KV partial states
 * and the projection's activation tiles) is a static device array of
 * 32 MiB (33554432 bytes) that each GPU the library runs on holds from its
 * first lacache_create on that GPU until the process ends; the call itself
 * allocates nothing.  Arguments, results and the other errors are those of
 * lacache_block_step.  Returns LACACHE_ERR_UNSUPPORTED, with nothing
 * launched, when the block table needs more scratch than that (the message
 * gives both sizes; lacache_workspace_size(LACACHE_OP_BLOCK_STEP) bounds the
 * need from above), and LACACHE_ERR_INVALID_ARG while per-kernel profiling is
 * enabled on the context (its events are created on demand).  Every call on
 * one GPU shares that GPU's scratch, which keeps the last call's contents (no
 * kernel needs it cleared: every partial state and activation tile is written
 * before it is read): calls that overlap on one GPU (other streams, other
 * threads, other contexts) race and must be serialised by the caller. */
LACACHE_API lacache_status lacache_block_step_noalloc(lacache_ctx *ctx, const lacache_weights *w,
                                                      const int32_t *block_ids, const lacache_seq *seqs,
                                                      int32_t batch, const lacache_cache *cache, void *out,
                                                      float *lse, void *stream);

/* Refresh at a block boundary when only some rows' ids changed since their
 * last projection (normally the block just finished: its final ids are
 * chosen after its last inner step).  Layer-0 q, k, v of a row depend only on
 * its id and position (Section 3.3.2, EmbedCache and RoPECache), so only the
 * rows of proj are re-projected; the attention is the full refresh of
 * lacache_prefill_cache for the new block table seqs (the invariant set
 * changes at the boundary and keys cannot leave an online-softmax state).
 *   proj_ids device int32 [sum_b (proj[b].block_end - proj[b].block_start)]:
 *            the ids of the rows to re-project, concatenated in sample order.
 *   proj     host [batch]: per sample, the same seq_offset and seq_len as
 *            seqs, and as block the rows [block_start, block_end) to
 *            re-project (non-empty, at most 128 rows).
 *   seqs     host [batch]: the block table from now on (the new block).
 * Writes h, q, k, v of the proj rows; m, l, o for every row of the new U;
 * out and lse (lse may be NULL) for every row.  The result equals
 * lacache_prefill_cache on the full new ids up to rounding, provided the
 * other rows' cache entries are those of their current ids.  Workspace:
 * lacache_workspace_size(LACACHE_OP_REFRESH_BLOCK, proj, batch). */
LACACHE_API lacache_status lacache_refresh_block(lacache_ctx *ctx, const lacache_weights *w,
                                     const int32_t *proj_ids, const lacache_seq *proj,
                                     const lacache_seq *seqs, int32_t batch,
                                     const lacache_cache *cache, void *out, float *lse,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* Block-query attention over [prefix | fresh block | suffix] keys: the
 * attention of Fast-dLLM's DualCache inner step (decode_block), exact at
 * layer 0.
 *   q_block   device [sum_b B_b, H, d_h] ctype: the block rows' queries,
 *             concatenated in sample order.
 *   k, v      device [n_rows, H_kv, d_h] ctype: every sample's keys/values
 *             at its rows (prefix, block and suffix), as in the cache.
 *   n_rows    rows k and v hold.
 *   out_block device [sum_b B_b, H, d_h] dtype; lse_block [sum_b B_b, H]
 *             fp32 or NULL. */
LACACHE_API lacache_status lacache_dualcache_attn(lacache_ctx *ctx, const void *q_block,
                                      const void *k, const void *v, int64_t n_rows,
                                      const lacache_seq *seqs, int32_t batch,
                                      void *out_block, float *lse_block,
                                      void *workspace, size_t workspace_bytes,
                                      void *stream);

/* Steps a1-a5 alone for the block rows: gathers the rows of w->embed named
 * by block_ids, writes them to cache->h, and writes the block rows' RoPE'd
 * q, k, v into the RoPECache, exactly as lacache_block_step does, with no
 * attention (cache->m, l, o are not read and may be NULL).  For a layer
 * after the first, w->embed is that layer's input rows (the previous layer's
 * output, [rows, d_model]) and block_ids the rows' own indices, so the
 * "embedding" of a token is its hidden row: the block's fresh q, k, v of
 * that layer, to be attended by lacache_dualcache_attn over the layer's
 * cached keys (the DualCache inner step of the DualCache page, "Block-wise
 * Generation"; approximate at layers after the first, where the other rows'
 * keys are those of the last refresh).  Workspace:
 * lacache_workspace_size(LACACHE_OP_PROJECT_BLOCK). */
LACACHE_API lacache_status lacache_project_block(lacache_ctx *ctx, const lacache_weights *w, const int32_t *block_ids,
                                                 const lacache_seq *seqs, int32_t batch, const lacache_cache *cache,
                                                 void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Per-group FP8 FFN of the layers after the first (LaCache Section 3.4,
 * "Mixed precision strategy", Eqs. (7)-(8), and Figure 2): per-group FP8
 * quantization before the gate-up and ffout linears, fused with the
 * feed-forward AddNorm and with SwiGLU, and both linears on FP8 operands.
 *   Quantization: groups of 128 consecutive features of one token
 *   (activations) or 128 x 128 blocks (weights); scale = max |x| / 448 and
 *   code = E4M3(clip(x / scale, -448, 448)), OCP E4M3, round to nearest
 *   even, scale and x / scale in fp32; an all-zero group has scale 0.
 *   Layer: r = bf16(h + attn_out); x = RMSNorm(r) with gamma and the
 *   context's rms_eps; [gate; up] = Q(x) Q(W_gate_up)^T; y = silu(gate) * up;
 *   out = bf16(r + Q(y) Q(W_down)^T), every product of quantized operands
 *   dequantized group by group in fp32.
 * The context must be bf16 with d_model a multiple of 512; d_ff a multiple of
 * 128.  Shapes: w_gate, w_up [d_ff, d_model] bf16, w_down [d_model, d_ff]
 * bf16 (row-major, out-features major), gamma [d_model] bf16; h, attn_out,
 * r_out, out [n_rows, d_model] bf16.  The FFN runs on whole sequences: the
 * rows of the layer (no block table). */
typedef struct {
  const void *gamma;         /* feed-forward RMSNorm gain, [d_model] bf16               */
  const void *gate_up;       /* packed FP8 [w_gate; w_up] (lacache_ffn_pack_weights)    */
  const float *s_gate_up;    /* its block scales                                        */
  const void *down;          /* packed FP8 w_down                                       */
  const float *s_down;       /* its block scales                                        */
} lacache_ffn_weights;

/* Bytes of the packed FP8 weights and of their block scales for d_ff. */
LACACHE_API lacache_status lacache_ffn_weight_bytes(const lacache_ctx *ctx, int32_t d_ff, size_t *gate_up_bytes,
                                                    size_t *gate_up_scale_bytes, size_t *down_bytes,
                                                    size_t *down_scale_bytes);

/* Enqueues the one-time quantization of a layer's FFN weights (device, bf16)
 * into the packed FP8 form lacache_ffn_fp8 reads (device, caller-owned, at
 * least the sizes above), with one fp32 scale per 128 x 128 block. */
LACACHE_API lacache_status lacache_ffn_pack_weights(lacache_ctx *ctx, int32_t d_ff, const void *w_gate,
                                                    const void *w_up, const void *w_down, void *gate_up,
                                                    float *s_gate_up, void *down, float *s_down, void *stream);

/* Workspace bytes of lacache_ffn_fp8 for n_rows rows (1 <= n_rows <= 2^24);
 * keeps_residual: whether the call will be given r_out (else r lives in the
 * workspace). */
LACACHE_API lacache_status lacache_ffn_workspace_size(const lacache_ctx *ctx, int32_t d_ff, int64_t n_rows,
                                                      int32_t keeps_residual, size_t *bytes);

/* One FFN sub-block: writes out (and r_out unless NULL) for every row.  The
 * diagnostic environment variable LACACHE_FP8_TILE ("256" or "128"), read by
 * lacache_create, fixes the down projection's output tile instead of the
 * choice by launch size.
 * Packed FP8 layout (the weights, and the quantized activations in the
 * workspace): element (i, k) of an [N rows, K] operand (i: a row of the
 * activations or an output feature of the weight, k: the contraction index)
 * is byte ((i/256) (K/128) + k/128) 32768 + ((i/16) % 16) 2048 +
 * ((k/16) % 2) 1024 + (16 ((k % 128)/32) + i % 16) 16 + k % 16 (N padded to a
 * multiple of 256 with zero codes).  The packed gate-up weight holds, in its
 * 256-row tile j, rows 128 j .. 128 j + 127 of w_gate then the same rows of
 * w_up; its scales are [d_model/128][2 d_ff/128] with column 2 j for the gate
 * block and 2 j + 1 for the up block of tile j; the down weight's scales are
 * [d_ff/128][d_model/128].
 * Workspace after the call (M_pad = n_rows rounded up to 256; each part
 * starts at a multiple of 256 bytes, in this order): the packed codes of
 * x = RMSNorm(r) [M_pad, d_model]; their scales [d_model/128][M_pad] fp32;
 * the packed codes of y = silu(gate) * up [M_pad, d_ff]; their scales
 * [d_ff/128][M_pad] fp32; r [n_rows, d_model] bf16 when r_out is NULL. */
LACACHE_API lacache_status lacache_ffn_fp8(lacache_ctx *ctx, int32_t d_ff, const lacache_ffn_weights *w,
                                           const void *h, const void *attn_out, int64_t n_rows, void *r_out,
                                           void *out, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The rest of layer 0 after its attention, and the sampler cut (LaCache
 * Figure 2; Section 3.4: the first layer keeps the parameter precision, and
 * at the sampling stage only the current block's rows of the transformer
 * output go through the final norm, the lm-head and the float softmax).
 * bf16 throughout, fp32 accumulation, every operator's output rounded to bf16
 * (round to nearest even):
 *   a = bf16(attn_out W_o^T); r = bf16(h + a);
 *   x = bf16(gamma r / sqrt(mean(r^2) + rms_eps));
 *   gate = bf16(x W_gate^T), up = bf16(x W_up^T), y = bf16(silu(gate) up);
 *   out = bf16(r + bf16(y W_down^T)).
 * Shapes (row-major, bf16): w_o [d_model, n_heads head_dim]; gamma
 * [d_model]; w_gate, w_up [d_ff, d_model]; w_down [d_model, d_ff]; h, r_out,
 * out [n_rows, d_model] (h: the layer's input rows, i.e. the EmbedCache at
 * layer 0); attn_out [n_rows, n_heads head_dim] (the attention output, heads
 * concatenated: the `out` rows of lacache_block_step).  Every row of the
 * sequences is computed: each row's attention output changes with the
 * block's keys.  The context must be bf16 with d_model in {512, 1024, 2048,
 * 4096, 8192}, n_heads head_dim a multiple of 64; d_ff a multiple of 128. */
typedef struct {
  const void *w_o;           /* attention output projection                             */
  const void *gamma;         /* feed-forward RMSNorm gain                               */
  const void *w_gate;        /* gate linear                                             */
  const void *w_up;          /* up linear                                               */
  const void *w_down;        /* down (ffout) linear                                     */
} lacache_layer_weights;

/* Workspace bytes of lacache_layer_finish for n_rows rows (1 <= n_rows <=
 * 2^24); keeps_residual: whether the call will be given r_out. */
LACACHE_API lacache_status lacache_layer_finish_workspace_size(const lacache_ctx *ctx, int32_t d_ff, int64_t n_rows,
                                                               int32_t keeps_residual, size_t *bytes);

/* Enqueues the rest of the layer for n_rows rows: out (and r_out unless
 * NULL).  The diagnostic environment variable LACACHE_LAYER_TILE ("256",
 * "128", "64" or "128w4"), read by lacache_create, fixes the output tile of
 * the bf16 GEMMs here and in lacache_sampler_cut (256 x 256, 128 x 128,
 * 64 x 256, or 128 x 128 with four waves; the SwiGLU GEMM takes 64 x 256 for
 * "128") instead of the choice by launch size.  GEMMs whose tiles leave
 * compute units idle split their contraction (at most 64 rows on 64 x 256
 * tiles; a long contraction on 128 x 128 tiles) and sum fp32 partials in
 * the workspace.  Workspace after the call (each part at a multiple of 256
 * bytes, in this order): r [n_rows, d_model] when r_out is NULL; x [n_rows,
 * d_model]; y [n_rows, d_ff]. */
LACACHE_API lacache_status lacache_layer_finish(lacache_ctx *ctx, int32_t d_ff, const lacache_layer_weights *w,
                                                const void *h, const void *attn_out, int64_t n_rows, void *r_out,
                                                void *out, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of lacache_sampler_cut for this block table and vocabulary
 * (a multiple of 8).  The table's blocks may be any size here (a block that
 * spans a whole sequence gives the sampler without the cut). */
LACACHE_API lacache_status lacache_sampler_workspace_size(const lacache_ctx *ctx, int32_t vocab,
                                                          const lacache_seq *seqs, int32_t batch, size_t *bytes);

/* The sampler on the block rows only.  For block row t of the table (rows
 * seq_offset + [block_start, block_end), sample by sample; M rows in all) of
 * hidden [n_rows, d_model] bf16: z = bf16(gamma_final row / sqrt(mean(row^2)
 * + rms_eps)); logits = z w_lm^T in fp32 (w_lm [vocab, d_model] bf16);
 * token[t] = the argmax (the first index among equal maxima), confidence[t]
 * = its softmax probability 1 / sum_v exp(logit_v - max); probs [M, vocab]
 * fp32, unless NULL, every probability.  Workspace after the call (each
 * part at a multiple of 256 bytes, in this order): z [M, d_model] bf16; the
 * logits [M, vocab] fp32; the softmax's per-chunk (max, sum exp(l - max))
 * [M, ceil(vocab / 4096)] float pairs and chunk argmaxes int32; the rows'
 * (max, sum) [M] float pairs. */
LACACHE_API lacache_status lacache_sampler_cut(lacache_ctx *ctx, const void *hidden, int64_t n_rows,
                                               const lacache_seq *seqs, int32_t batch, const void *gamma_final,
                                               const void *w_lm, int32_t vocab, int32_t *token, float *confidence,
                                               float *probs, void *workspace, size_t workspace_bytes,
                                               void *stream);

/* ---------------------------------------------------------------------------
 * Flash-dLLM's selective cache update and two-view verify (the Flash-dLLM
 * article: the third element of "Flash-Cache: Fusing Projection, RoPE, and
 * Cache Writes into One Kernel", and "Flash-Verify: Making the Diffusion
 * Model Its Own Verifier").  bf16 contexts (fp16 RoPECache), head_dim 64 or
 * 128.
 * ------------------------------------------------------------------------- */

/* Workspace bytes of lacache_track_select for buffers of n_rows rows. */
LACACHE_API lacache_status lacache_track_workspace_size(const lacache_ctx *ctx, int64_t n_rows, size_t *bytes);

/* Attention importance and the tracking set.  For each sample b of the
 * table and each of its rows j: importance[seq_offset + j] = sum over heads h
 * and the block's queries i of exp(scale q_ih . k_jh - lse_ih), the softmax
 * weight row j receives from the current block (cache->q and cache->k: the
 * RoPECache after the step; lse [n_rows, n_heads]: the block rows' LSE as
 * lacache_block_step writes it).  tracked[b budget + r], r < budget: the
 * budget rows outside the block (positions within the sample) of largest
 * importance, the lower position on ties, in increasing position; -1 where
 * fewer rows are eligible.  budget in [1, 64]; sequences of at most 16384
 * rows.  Workspace: lacache_track_workspace_size(cache->n_rows). */
LACACHE_API lacache_status lacache_track_select(lacache_ctx *ctx, const lacache_cache *cache, const float *lse,
                                                const lacache_seq *seqs, int32_t batch, int32_t budget,
                                                float *importance, int32_t *tracked, void *workspace,
                                                size_t workspace_bytes, void *stream);

/* Two-view verify attention.  Sample b's verify tokens are rows
 * ver_start[b] .. ver_start[b+1]-1 (ver_start: host, non-decreasing) of
 * q_ver, k_ver, v_ver ([*, n_heads / n_kv_heads, head_dim] fp16, RoPE'd at
 * their positions: the projection of the verify query), with view[t] (0
 * tracking, 1 draft view, 2 mask view) and pos[t] (the position within the
 * sample it carries).  Each verify query attends over the sample's cached
 * rows (cache->k, cache->v) except the positions its sample's verify tokens
 * carry, and over the verify tokens' own keys of view 0 or of its own view.
 * out [*, n_heads, head_dim] bf16 and lse [*, n_heads] (natural log, or NULL)
 * at the verify tokens' rows.  Sequences of at most 32768 rows. */
LACACHE_API lacache_status lacache_verify_attn(lacache_ctx *ctx, const void *q_ver, const void *k_ver,
                                               const void *v_ver, const int32_t *view, const int32_t *pos,
                                               const int32_t *ver_start, const lacache_cache *cache,
                                               const lacache_seq *seqs, int32_t batch, void *out, float *lse,
                                               void *stream);

/* Verify acceptance.  Sample b's search positions are entries
 * search_start[b] .. search_start[b+1]-1 (host, non-decreasing; at most 64
 * per sample) of pos (increasing positions within the sample), draft and
 * mask_tok (the argmax tokens of the draft and mask views) and mask_conf (the
 * mask view's confidence).  n_accepted[b] = the length of the longest prefix
 * whose draft and mask tokens agree with mask_conf > gamma; the accepted
 * draft tokens are written to ids[seq_offset + pos] (ids: the flat token ids
 * of the table's rows).  Positions not increasing or outside the sample set
 * LACACHE_DEVFLAG_SEARCH_ORDER and accept nothing in that sample. */
LACACHE_API lacache_status lacache_verify_accept(lacache_ctx *ctx, const int32_t *draft, const int32_t *mask_tok,
                                                 const float *mask_conf, const int32_t *pos,
                                                 const int32_t *search_start, const lacache_seq *seqs,
                                                 int32_t batch, float gamma, int32_t *ids, int32_t *n_accepted,
                                                 void *stream);

/* Bytes of the packed projection weight for this context: 0 where the
 * configuration has no many-token projection (fp32, or d_model not a
 * multiple of 512). */
LACACHE_API lacache_status lacache_packed_weight_size(const lacache_ctx *ctx, size_t *bytes);

/* Enqueues the conversion of w_qkv (device, bf16, layout above) into
 * w_packed (device, caller-owned, at least lacache_packed_weight_size bytes):
 * every weight as IEEE fp16 (round to nearest even; exact for weights of
 * magnitude in [2^-14, 65504], the fp16 normal range), arranged in the
 * column-tile / contraction-tile order the many-token projection copies
 * from, so each copy reads contiguous memory.  A one-time step per weight
 * set: pass the result as lacache_weights.w_qkv_packed.  Returns
 * LACACHE_ERR_UNSUPPORTED where the size is 0 and LACACHE_ERR_INVALID_ARG
 * for a NULL or unaligned pointer or packed_bytes below the size. */
LACACHE_API lacache_status lacache_pack_qkv_weight(lacache_ctx *ctx, const void *w_qkv, void *w_packed,
                                                   size_t packed_bytes, void *stream);

/* Reads and clears the device status word (LACACHE_DEVFLAG_*), after
 * synchronising `stream`. */
LACACHE_API lacache_status lacache_read_device_status(lacache_ctx *ctx, void *stream,
                                          uint32_t *flags);

/* Optional per-kernel timing (diagnostics, off by default).  While enabled,
 * every kernel launch of this context carries two HIP events that the
 * dispatch itself stamps with its start and end (hipExtLaunchKernelGGL).
 * lacache_profile_read synchronises those events and returns,
 * for one kernel class, the summed event time in milliseconds and the number
 * of launches since the last read of that class (then resets that class). */
typedef enum {
  LACACHE_KERNEL_QKV = 0,            /* embed + RMSNorm + QKV + RoPE + cache write  */
  LACACHE_KERNEL_BLOCK_ROWS = 1,     /* block rows x key chunks: partial states     */
  LACACHE_KERNEL_INVARIANT_ROWS = 2, /* block step: invariant rows from FACache and
                                        the merge of the block rows' partials      */
  LACACHE_KERNEL_MERGE = 3,          /* DualCache: merge of the partials            */
  LACACHE_KERNEL_REFRESH_ATTN = 4,   /* refresh attention with FACache snapshot     */
  LACACHE_KERNEL_QKV_PREP = 5,       /* gather, EmbedCache, RMSNorm (GEMM path)     */
  LACACHE_KERNEL_QKV_GEMM = 6,       /* prep'd tokens: QKV GEMM + RoPE + cache write */
  LACACHE_KERNEL_ATTN = 7,           /* small block steps: block-row partials and
                                        invariant rows in one launch               */
  LACACHE_KERNEL_FFN_NORM = 8,       /* FP8 FFN: AddNorm + quantization             */
  LACACHE_KERNEL_FFN_GATE_UP = 9,    /* FP8 FFN: gate-up GEMM + SwiGLU + quantization */
  LACACHE_KERNEL_FFN_DOWN = 10,      /* FP8 FFN: down GEMM + residual               */
  LACACHE_KERNEL_LAYER_OPROJ = 11,   /* layer finish: W_o GEMM + residual           */
  LACACHE_KERNEL_LAYER_NORM = 12,    /* layer finish: feed-forward RMSNorm          */
  LACACHE_KERNEL_LAYER_GATE_UP = 13, /* layer finish: gate-up GEMM + SwiGLU         */
  LACACHE_KERNEL_LAYER_DOWN = 14,    /* layer finish: down GEMM + residual          */
  LACACHE_KERNEL_SAMPLER_NORM = 15,  /* sampler: final norm of the block rows       */
  LACACHE_KERNEL_SAMPLER_LMHEAD = 16, /* sampler: lm-head GEMM (fp32 logits)        */
  LACACHE_KERNEL_SAMPLER_SOFTMAX = 17, /* sampler: float softmax and argmax         */
  LACACHE_KERNEL_TRACK_IMPORTANCE = 18, /* selective update: attention importance   */
  LACACHE_KERNEL_TRACK_SELECT = 19,  /* selective update: the tracking set          */
  LACACHE_KERNEL_VERIFY_ATTN = 20,   /* two-view verify attention                   */
  LACACHE_KERNEL_VERIFY_ACCEPT = 21, /* verify acceptance                           */
  LACACHE_KERNEL_COUNT = 22
} lacache_kernel;

LACACHE_API lacache_status lacache_profile_enable(lacache_ctx *ctx, int enable);
LACACHE_API lacache_status lacache_profile_read(lacache_ctx *ctx, int32_t kernel, double *total_ms,
                                                int64_t *launches);

/* Static description of a status code. */
LACACHE_API const char *lacache_status_string(lacache_status s);

/* Description of the last failed call on this context ("" if none). */
LACACHE_API const char *lacache_last_error(const lacache_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* LACACHE_H */
