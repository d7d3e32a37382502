// Internal interface between the C-ABI front end (api.hip) and the kernel
// launchers (qkv.hip, attn.hip).  Plain pointers and sizes only.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace lc {

enum DType { kF32 = 0, kBF16 = 1 };

// Fused embedding gather + RMSNorm + QKV projection + RoPE + cache write.
struct QkvArgs {
  const int *ids;          // mode 0: [tokens of launch] block ids; mode 1: flat ids by row
  const void *E;           // [vocab, D]
  const void *gamma;       // [D]
  const void *W;           // [F, D]
  void *h;                 // EmbedCache [rows, D]
  void *q, *k, *v;         // RoPECache
  const float2 *rope;      // [max_pos, dh/2] (cos, sin)
  unsigned *flags;         // device status word
  int mode;                // 0: block step, 1: prefill
  int M;                   // tokens in this launch
  int ids_base;            // mode 0: index of the launch's first token in `ids`
  int vocab, D, H, Hkv, dh;
  float eps;
};

// Many-token path (bf16 parameters): prep kernel (gather, EmbedCache write,
// normalised fp16 activation, per-token cache row and position), then the
// MFMA GEMM with RoPE and the cache write in its epilogue.
struct PrepArgs {
  const int *ids;          // as QkvArgs
  const void *E, *gamma;   // bf16
  void *h;                 // EmbedCache
  void *A;                 // [M_pad, D] fp16 normalised activations, GEMM tile order (workspace)
  int2 *map;               // [M_pad] (cache row, position) per token (workspace)
  float2 *cs;              // [M_pad, dh/2] (cos, sin) of each token's position (workspace)
  const float2 *rope;      // [max_pos, dh/2] (cos, sin)
  unsigned *flags;
  int mode;                // 0: block step, 1: prefill
  int M, M_pad;            // tokens of this launch, rounded up to the GEMM row tile
  int row0;                // index of the launch's first token among the slice's tokens
  int ids_base;            // mode 0: index of the slice's first token in `ids`
  int vocab, D, dh;
  float eps;
};
struct GemmArgs {
  const void *A;           // fp16 activations, tiled: [M_pad/128][D/64][128 x 64] (see a_piece)
  const void *W;           // [F, D] bf16 (used when Wp is null)
  const void *Wp;          // fp16 weights in GEMM tile order (launch_pack_qkv_weight), or null
  const int2 *map;         // [M] (cache row, position)
  const float2 *cs;        // [M_pad, dh/2] (cos, sin) per token
  void *q, *k, *v;         // fp16 RoPECache
  unsigned *flags;
  int M, D, F, H, Hkv;
};
constexpr int kGemmMinTokens = 128;    // block steps with fewer tokens use the streaming kernel
constexpr int kPrefillChunk = 4096;    // refresh rows per prep + GEMM pass
int gemm_rows_padded(int M);

// Attention kernels: block-row split partials (type A), invariant rows from
// FACache (type B), the refresh, and the merge of partials.
struct AttnArgs {
  const void *q;           // qmode 0: q cache [rows, H, dh]; qmode 1: q_block [M, H, dh]
  const void *k, *v;       // [rows, Hkv, dh]
  void *out;               // omode 0: [rows, H, dh]; omode 1: out_block [M, H, dh]
  float *lse;              // matching rows, [.., H], or null
  const float *m_c, *l_c;  // FACache read (block step): max (natural log), normaliser
  const void *o_c;         //   O~ / l in the cache type [rows, H, dh]
  float *m_w, *l_w;        // FACache write (refresh)
  void *o_w;
  float2 *part_ml;         // [P, H] (max in log2 units, normaliser)
  void *part_o;            // [P, H, dh] O~ / l of the chunk, cache type
  int qmode, omode;
  int row_base;            // index of the slice's first block row in q_block/out_block
  int part_base;           // index of the slice's first partial row
  int H, Hkv;
  int split_keys;          // keys per type-A chunk (multiple of 32)
  int seg_rows;            // streaming type B: invariant rows per workgroup (multiple of 16)
  int direct;              // streaming type A: chunks are whole sequences, write O and LSE
  float scale_log2;        // sm_scale * log2(e)
};

// Optional timing events attached to a launch: when set, the kernel is
// dispatched with hipExtLaunchKernelGGL, which stamps the events with the
// dispatch's own start and end times.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Launch log (diagnostics): when on, every launch prints its kernel
// instantiation and grid size to stderr.  Switched on by lacache_create when
// the environment variable LACACHE_LOG is set to a non-empty value other than
// "0"; process-wide.
void set_launch_log(bool on);
bool launch_log_enabled();
void log_launch(const void *kernel, hipStream_t s, unsigned grid);

// Launch kernel K on stream s, with events if requested.
template <auto K, typename... Args>
inline void lc_launch(dim3 grid, dim3 block, unsigned shmem, hipStream_t s, const LaunchEvents &ev, Args... args) {
  if (launch_log_enabled()) log_launch(reinterpret_cast<const void *>(K), s, grid.x * grid.y * grid.z);
  if (ev.start || ev.stop)                 // either stamp may be absent (launch sequences share one pair)
    hipExtLaunchKernelGGL(K, grid, block, shmem, s, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(K, grid, block, shmem, s, args...);
}

// Launchers: return hipSuccess or the launch error.
hipError_t launch_qkv(DType dt, const SeqArgs &sa, const QkvArgs &a, int F, hipStream_t s, const LaunchEvents &ev);
hipError_t launch_qkv_prep(const SeqArgs &sa, const PrepArgs &a, hipStream_t s, const LaunchEvents &ev);
// At most 64 tokens with the packed weight and an embedding table below 4 GB.
bool skinny_fused_supported(int M, int D, int vocab);
// At most 64 tokens with the packed weight: prep folded into the skinny GEMM
// (p.M == a.M, p.D == a.D; p.A, p.map, p.cs unused).
hipError_t launch_qkv_skinny_fused(int dh, const SeqArgs &sa, const PrepArgs &p, const GemmArgs &a, hipStream_t s,
                                   const LaunchEvents &ev);
// Tile of the packed-weight GEMM (>= 128 tokens): automatic by launch size,
// or fixed (diagnostics): whole 128 x 192, half-width 128 x 96, wide 256 x 192.
enum GemmTile { kGemmTileAuto = 0, kGemmTileWhole = 1, kGemmTileHalf = 2, kGemmTileWide = 3 };
hipError_t launch_qkv_gemm(int dh, const GemmArgs &a, int tile, hipStream_t s, const LaunchEvents &ev);
size_t packed_qkv_weight_bytes(int D, int F);
bool skinny_supported(int M, int D);      // the packed-weight projection for <= 64 tokens
int prep_rows(int M, int D, bool packed); // rows the prep kernel writes (zero rows past M included)
hipError_t launch_pack_qkv_weight(const void *W, void *Wp, int D, int F, int dh, hipStream_t s);
hipError_t setup_gemm_attributes();
int device_cus();                         // compute units of the current device (cached; 256 if unknown)
hipError_t launch_block_rows(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks,
                             hipStream_t s, const LaunchEvents &ev);
hipError_t launch_invariant_rows(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks, int M,
                                 hipStream_t s, const LaunchEvents &ev);
hipError_t launch_merge(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int M, hipStream_t s,
                        const LaunchEvents &ev);
// Workgroups of a combined (type A + type B) launch resident on the chip at once.
int attn_ab_capacity(DType dt, int dh, const SeqArgs &sa);
hipError_t launch_attn_ab(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int nA, int nB, hipStream_t s,
                          const LaunchEvents &ev);
constexpr int kStreamMaxBlock = 64;   // largest block the streaming type-B kernel serves
hipError_t launch_invariant_stream(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, hipStream_t s,
                                   const LaunchEvents &ev);
hipError_t launch_refresh_attn(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks,
                               hipStream_t s, const LaunchEvents &ev);
// Streaming refresh (bf16 parameters, 16-bit caches): items of 64 * mb rows
// (mb = 1 or 2 row blocks of 16 per wave), a 2-stage ring of 64-key tiles
// (two workgroups per CU).
hipError_t launch_refresh_stream(int dh, int mb, const SeqArgs &sa, const AttnArgs &a, int n_blocks, hipStream_t s,
                                 const LaunchEvents &ev);
hipError_t setup_kernel_attributes();

// Per-group FP8 FFN (layers after the first): AddNorm + quantization, FP8
// GEMMs with SwiGLU + quantization or residual epilogues, weight packing.
struct Fp8NormArgs {
  const void *h, *a;       // [M, D] bf16: residual stream and the attention block's output
  const void *gamma;       // [D] bf16
  void *r;                 // [M, D] bf16: r = bf16(h + a)
  void *xq;                // packed FP8 codes of RMSNorm(r) (M_pad rows)
  float *sx;               // [D/128][M_pad] scales
  int M, M_pad, D;
  float eps;
};
struct Fp8GemmArgs {
  const void *A;           // packed FP8 activations (M_pad rows, K contraction)
  const float *sa;         // [K/128][M_pad]
  const void *B;           // packed FP8 weight (N rows, K contraction)
  const float *sw;         // [K/128][N/128]
  int M, M_pad, N, K;
  void *yq;                // SwiGLU epilogue: packed FP8 of silu(gate) * up (M_pad rows, N/2 contraction)
  float *sy;               //   [N/256][M_pad]
  const void *res;         // residual epilogue: out = bf16(res + A W^T), [M, N] bf16
  void *out;
  float *part;             // residual epilogue, split contraction: fp32 partials [splits][M][N] (workspace), or null
  int splits;              // set by the launcher
};
size_t fp8_packed_bytes(int N, int K);                     // bytes of a packed FP8 operand of N rows
hipError_t launch_fp8_pack_weight(const void *W, int N, int K, int mode, void *Wp, float *sw, int Np, hipStream_t s);
hipError_t launch_fp8_addnorm_quant(const Fp8NormArgs &a, hipStream_t s, const LaunchEvents &ev);
hipError_t launch_fp8_gemm_swiglu(const Fp8GemmArgs &a, hipStream_t s, const LaunchEvents &ev);
// tile: 0 automatic, 1 = 256 x 256, 2 = 128 x 128.  With a.part set, a
// launch of 128 x 128 tiles that leaves CUs idle and contracts over many
// groups is split (fp8_part_bytes bytes of partials).
hipError_t launch_fp8_gemm_resid(const Fp8GemmArgs &a, int tile, hipStream_t s, const LaunchEvents &ev);
size_t fp8_part_bytes(int M, int M_pad, int N, int K, int tile);
hipError_t setup_fp8_attributes();

// The rest of layer 0 and the sampler cut (layer.hip).
struct Bf16GemmArgs {
  const bf16_t *A;         // [M, K] row-major, leading dimension lda (elements)
  const bf16_t *B;         // [N, K] row-major (SwiGLU: the gate rows), leading dimension ldb
  const bf16_t *B2;        // SwiGLU: the up rows [N, K]; else unused
  const bf16_t *res;       // bf16 output: residual [M, N] (leading dimension ldr) added after rounding, or null
  void *out;               // [M, N] bf16 or fp32 (SwiGLU: [M, N] bf16 with N the features), leading dimension ldo
  int M, N, K;
  int lda, ldb, ldr, ldo;
  // Split contraction (set by the launcher): `splits` workgroups share each
  // output tile, split s summing contraction steps [s KG / splits, (s+1) KG /
  // splits) of the KG 64-wide steps into part[s][M][ldp] (fp32, the tiles'
  // columns in the kernel's own order); a second kernel adds the splits in
  // order and applies the epilogue.
  float *part;
  int splits, ldp;
};
enum { kGemmOutBf16 = 0, kGemmOutF32 = 1, kGemmOutSwiglu = 2 };
// tile: 0 automatic, 1 256 x 256, 2 128 x 128, 3 64 x 256, 4 128 x 128 with four waves (rows x columns of the output)
hipError_t launch_bf16_gemm(const Bf16GemmArgs &a, int out_kind, int tile, hipStream_t s, const LaunchEvents &ev);
// Bytes of split-contraction partials launch_bf16_gemm may use for this
// shape (0: it never splits); a.part must then hold that many bytes, or be
// null to forbid splitting.
size_t bf16_gemm_part_bytes(int M, int N, int K, int out_kind);
struct RowNormArgs {
  const bf16_t *src;       // rows, leading dimension lds (elements)
  const bf16_t *gamma;     // [D]
  bf16_t *out;             // [M, D]
  int lds, M, D;
  float eps;
  int gather;              // 1: output row m is block row m of sa (pre[0]: block-token prefix sums)
  SeqArgs sa;
};
hipError_t launch_rmsnorm_rows(const RowNormArgs &a, hipStream_t s, const LaunchEvents &ev);
struct SoftmaxArgs {
  const float *logits;     // [M, V], leading dimension ld
  int *token;              // [M] argmax (first index among equal maxima)
  float *conf;             // [M] its probability
  float *probs;            // [M, V] probabilities (leading dimension ldp), or null
  float2 *part;            // [M, softmax_chunks(V)] chunk (max, sum exp(l - max)) (workspace)
  int *part_idx;           // [M, softmax_chunks(V)] chunk argmax (workspace)
  float2 *row_stat;        // [M] row (max, sum exp(l - max)) (workspace)
  int M, V, ld, ldp;
};
int softmax_chunks(int V);
hipError_t launch_softmax_argmax(const SoftmaxArgs &a, hipStream_t s, const LaunchEvents &ev);
hipError_t setup_layer_attributes();

// Selective cache update and two-view verify (flashdllm.hip); fp16 RoPECache.
constexpr int kTrackMaxKeys = 16384;     // rows per sample the tracking selection holds in LDS
constexpr int kVerifyMaxKeys = 32768;    // rows per sample the verify attention's carried-position bitmap covers
struct TrackArgs {
  const void *q;           // RoPECache q [n_rows, H, dh] (the block rows' fresh queries)
  const float *lse;        // [n_rows, H] the block rows' log-sum-exp (natural log)
  const void *k;           // RoPECache k [n_rows, Hkv, dh]
  float *partial;          // [n_rows, H] per-head importance (workspace)
  float *importance;       // [n_rows] importance of every row of the table's samples
  int *tracked;            // [batch, budget] selected rows within their sample, in row order; -1 pads
  int64_t n_rows;
  int H, Hkv, budget, sample_base;
  float scale_log2;
};
hipError_t launch_importance(int dh, const SeqArgs &sa, const TrackArgs &a, hipStream_t s, const LaunchEvents &ev);
hipError_t launch_track_select(const SeqArgs &sa, const TrackArgs &a, int max_len, hipStream_t s,
                               const LaunchEvents &ev);
struct VerifyArgs {
  const void *q;           // [V, H, dh] verify queries (fp16, RoPE'd at their positions); sample b: rows pre[0][b] ..
  const void *k_ver, *v_ver;  // [V, Hkv, dh] their own keys and values
  const int *view;         // [V] 0 tracking, 1 draft view, 2 mask view
  const int *pos;          // [V] position within the sample each verify token carries
  const void *k, *v;       // RoPECache [n_rows, Hkv, dh]: the context
  void *out;               // [V, H, dh] bf16
  float *lse;              // [V, H] natural log, or null
  int H, Hkv;
  float scale_log2;
};
hipError_t launch_verify_attn(int dh, const SeqArgs &sa, const VerifyArgs &a, hipStream_t s, const LaunchEvents &ev);
struct AcceptArgs {
  const int *draft, *mask_tok;  // [S] argmax tokens of the two views at the search positions
  const float *mask_conf;  // [S] the mask view's confidence
  const int *pos;          // [S] search positions within the sample, increasing
  int *ids;                // [n_rows] token ids; accepted draft tokens are written at off + pos
  int *n_accepted;         // [batch]
  unsigned *flags;
  float gamma;
};
hipError_t launch_verify_accept(const SeqArgs &sa, const AcceptArgs &a, hipStream_t s, const LaunchEvents &ev);
hipError_t setup_flashdllm_attributes();

// Work decomposition shared by the planner and the kernels.
constexpr int kRowsA = 32;     // block rows per type-A item
constexpr int kRowsB = 64;     // invariant rows per type-B item
constexpr int kRowsR = 64;     // rows per refresh item (fp32)
constexpr int kRefreshMB = 2;  // row blocks of 16 per wave in the streaming refresh (1 for small launches)
constexpr int kQkvRows = 32;   // token rows per QKV tile
constexpr int kQkvNB = 3;      // 16-feature column blocks per QKV tile
constexpr int kQkvWaves = 8;   // waves splitting the contraction
constexpr int kQkvMaxD = 8192; // largest d_model (gamma is staged in LDS)

}  // namespace lc
