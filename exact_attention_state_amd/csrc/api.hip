// C ABI of the exact layer-0 cached block step (declared in include/lacache.h).
//
// Host side only: argument validation (all before any launch), the work
// decomposition computed from the host block table (no device->host sync),
// the RoPE table, and the kernel launches on the caller's stream.  The block
// table of each launch travels inside the kernel arguments; batches larger
// than lc::kMaxInline samples are launched in slices.

#include <algorithm>
#include <cxxabi.h>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"
#include "lacache.h"

struct lacache_ctx {
  lacache_config cfg;
  int device;
  float2 *rope;
  unsigned *flags;
  int split_keys;          // keys per type-A chunk if fixed by LACACHE_SPLIT_KEYS, else 0 (per call)
  int gemm_tile;           // packed GEMM tile fixed by LACACHE_GEMM_TILE (lc::GemmTile), else automatic
  int refresh_rows;        // streaming refresh item rows fixed by LACACHE_REFRESH_ROWS (64 or 128), else 0
  void *scratch;           // device address of this device's static scratch (lacache_block_step_noalloc)
  int fp8_tile;            // down-projection FP8 GEMM tile fixed by LACACHE_FP8_TILE (1: 256, 2: 128), else 0
  int layer_tile;          // bf16 layer GEMM tile fixed by LACACHE_LAYER_TILE (1: 256, 2: 128, 3: 64 x 256,
                           // 4: 128 x 128 with four waves), else 0
  std::string last_error;
  // Diagnostics: event pairs stamped by each launch while profiling is on.
  bool profiling = false;
  struct Mark { int kernel; hipEvent_t start, stop; };
  std::vector<Mark> marks;
  std::vector<hipEvent_t> free_events;
  double prof_ms[LACACHE_KERNEL_COUNT] = {};
  int64_t prof_n[LACACHE_KERNEL_COUNT] = {};
};

namespace lc {
namespace {
bool g_launch_log = false;
}
void set_launch_log(bool on) { g_launch_log = on; }
bool launch_log_enabled() { return g_launch_log; }
void log_launch(const void *kernel, hipStream_t s, unsigned grid) {
  // The runtime's (mangled) name of the kernel, demangled:
  // "void lc::name<args>(params)" -> "lc::name<args>".
  const char *mangled = hipKernelNameRefByPtr(kernel, s);
  std::string m = mangled ? mangled : "?";
  // _Float16 is mangled DF16_, which the host demangler may not know: read it
  // as the half type (Dh).
  for (size_t p = m.find("DF16_"); p != std::string::npos; p = m.find("DF16_", p)) m.replace(p, 5, "Dh");
  int status = -1;
  char *dem = abi::__cxa_demangle(m.c_str(), nullptr, nullptr, &status);
  std::string name = status == 0 && dem ? dem : m;
  std::free(dem);
  if (name.compare(0, 5, "void ") == 0) name.erase(0, 5);
  const size_t args = name.rfind(">(");
  if (args != std::string::npos) name.erase(args + 1);
  std::fprintf(stderr, "lacache launch: %s grid %u\n", name.c_str(), grid);
}
}  // namespace lc

// Scratch of lacache_block_step_noalloc (callers that cannot allocate): one
// array per device, which every GPU the library runs on holds until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device.
namespace {
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) __attribute__((used)) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;

// Device address of `scratch` on device `dev` (the current device), looked
// up on the first request for that device.
hipError_t static_scratch_address(int dev, void **out) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!addr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}
}  // namespace

namespace {

using lc::kMaxInline;
using lc::bf16_t;

lacache_status fail(const lacache_ctx *ctx, lacache_status st, const char *fmt, ...)
    __attribute__((format(printf, 3, 4)));

lacache_status fail(const lacache_ctx *ctx, lacache_status st, const char *fmt, ...) {
  if (ctx) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    const_cast<lacache_ctx *>(ctx)->last_error = buf;
  }
  return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lacache_status check_device(lacache_ctx *ctx) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ctx, LACACHE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev != ctx->device)
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "context was created on device %d but device %d is current",
                ctx->device, dev);
  return LACACHE_OK;
}

// Block-table checks shared by every call.  n_rows < 0: no row bound.
lacache_status check_table(lacache_ctx *ctx, const lacache_seq *seqs, int32_t batch, int64_t n_rows,
                           int max_block = 128) {
  if (!seqs) return fail(ctx, LACACHE_ERR_INVALID_ARG, "seqs is NULL");
  if (batch < 1) return fail(ctx, LACACHE_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  std::vector<std::pair<int64_t, int64_t>> ranges;
  ranges.reserve(batch);
  for (int i = 0; i < batch; ++i) {
    const lacache_seq &s = seqs[i];
    if (s.seq_offset < 0 || s.seq_len < 1)
      return fail(ctx, LACACHE_ERR_INVALID_ARG, "sample %d: seq_offset %d / seq_len %d invalid", i, s.seq_offset,
                  s.seq_len);
    if (s.seq_len > ctx->cfg.max_seq_len)
      return fail(ctx, LACACHE_ERR_INVALID_ARG, "sample %d: seq_len %d exceeds max_seq_len %d", i, s.seq_len,
                  ctx->cfg.max_seq_len);
    if (!(0 <= s.block_start && s.block_start < s.block_end && s.block_end <= s.seq_len))
      return fail(ctx, LACACHE_ERR_INVALID_ARG, "sample %d: block [%d, %d) not inside [0, %d) or empty", i,
                  s.block_start, s.block_end, s.seq_len);
    if (s.block_end - s.block_start > max_block)
      return fail(ctx, LACACHE_ERR_UNSUPPORTED, "sample %d: block of %d tokens (at most %d supported)", i,
                  s.block_end - s.block_start, max_block);
    const int64_t end = (int64_t)s.seq_offset + s.seq_len;
    // Kernels index rows in 32 bits (offsets into the buffers are 64-bit).
    if (end > INT32_MAX)
      return fail(ctx, LACACHE_ERR_INVALID_ARG, "sample %d: rows [%d, %lld) end past row 2^31 - 1", i, s.seq_offset,
                  (long long)end);
    if (n_rows >= 0 && end > n_rows)
      return fail(ctx, LACACHE_ERR_INVALID_ARG, "sample %d: rows [%d, %lld) exceed the %lld rows of the buffers", i,
                  s.seq_offset, (long long)end, (long long)n_rows);
    ranges.emplace_back(s.seq_offset, end);
  }
  std::sort(ranges.begin(), ranges.end());
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].first < ranges[i - 1].second)
      return fail(ctx, LACACHE_ERR_INVALID_ARG, "row ranges of two samples overlap at row %lld",
                  (long long)ranges[i].first);
  return LACACHE_OK;
}

int nchunks(int split, int len) { return (len + split - 1) / split; }

// Keys per type-A chunk for a batch: one 128-key tile per workgroup while
// that leaves at most ~4 workgroups per CU; longer chunks (and fewer partial
// rows to merge) beyond that.  LACACHE_SPLIT_KEYS (a multiple of 32) fixes it.
// Keys per type-A chunk.  bf16: one chunk per sequence when that still gives
// every CU a workgroup; then *direct is set and the streaming block-row
// kernel writes O and LSE itself (no merge).  Otherwise chunks of 128 keys
// and more, doubled while the launch keeps about 1024 items.
constexpr int64_t kStreamAItems = 256;
int split_keys(const lacache_ctx *ctx, const lacache_seq *seqs, int32_t batch, int *direct = nullptr) {
  if (direct) *direct = 0;
  if (ctx->split_keys > 0) return ctx->split_keys;
  auto items = [&](int split) {
    int64_t n = 0;
    for (int i = 0; i < batch; ++i) {
      const int B = seqs[i].block_end - seqs[i].block_start;
      n += (int64_t)nchunks(split, seqs[i].seq_len) * ((B + lc::kRowsA - 1) / lc::kRowsA);
    }
    return n * ctx->cfg.n_heads;
  };
  int max_len = 1;
  for (int i = 0; i < batch; ++i) max_len = std::max(max_len, seqs[i].seq_len);
  if (ctx->cfg.dtype == LACACHE_BF16) {
    const int whole = (max_len + 63) / 64 * 64;
    if (items(whole) >= kStreamAItems) {
      if (direct) *direct = 1;
      return whole;
    }
  }
  int split = 128;
  while (split < max_len && items(2 * split) >= 1024) split *= 2;
  return split;
}

int64_t partial_rows(int split, const lacache_seq *seqs, int32_t batch) {
  int64_t p = 0;
  for (int i = 0; i < batch; ++i) p += (int64_t)nchunks(split, seqs[i].seq_len) * (seqs[i].block_end - seqs[i].block_start);
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t cache_elem_bytes(const lacache_ctx *ctx) { return ctx->cfg.dtype == LACACHE_BF16 ? 2 : 4; }

// Workspace layout for type-A partials: part_ml [P, H] float2, part_o [P, H, d_h] in the cache type.
struct Partials {
  float2 *ml;
  void *o;
};
size_t partial_bytes(const lacache_ctx *ctx, int64_t P) {
  const size_t H = ctx->cfg.n_heads, d = ctx->cfg.head_dim;
  return align256((size_t)P * H * sizeof(float2)) + align256((size_t)P * H * d * cache_elem_bytes(ctx));
}
Partials partial_layout(const lacache_ctx *ctx, void *ws, int64_t P) {
  const size_t H = ctx->cfg.n_heads;
  char *p = static_cast<char *>(ws);
  Partials r;
  r.ml = reinterpret_cast<float2 *>(p);
  p += align256((size_t)P * H * sizeof(float2));
  r.o = p;
  return r;
}

// Many-token QKV path (prep + MFMA GEMM): bf16 parameters with d_model a
// multiple of 512; always for the refresh, for block steps of at least
// kGemmMinTokens tokens.
bool gemm_capable(const lacache_ctx *ctx) { return ctx->cfg.dtype == LACACHE_BF16 && ctx->cfg.d_model % 512 == 0; }
bool step_uses_gemm(const lacache_ctx *ctx, int64_t M) { return gemm_capable(ctx) && M >= lc::kGemmMinTokens; }
// Block steps through the prep kernel and a GEMM: many tokens, or few
// tokens with the packed weight (the skinny GEMM).
bool step_uses_prep(const lacache_ctx *ctx, const lacache_weights *w, int64_t M) {
  return step_uses_gemm(ctx, M) ||
         (gemm_capable(ctx) && w->w_qkv_packed && lc::skinny_supported((int)M, ctx->cfg.d_model));
}
int64_t block_tokens(const lacache_seq *seqs, int32_t batch) {
  int64_t M = 0;
  for (int i = 0; i < batch; ++i) M += seqs[i].block_end - seqs[i].block_start;
  return M;
}
// Workspace of one prep + GEMM pass over up to `rows` tokens: A [rows_pad, D] fp16 and the token map.
size_t gemm_bytes(const lacache_ctx *ctx, int64_t rows) {
  const size_t Mp = (size_t)lc::gemm_rows_padded((int)rows);
  return align256(Mp * ctx->cfg.d_model * 2) + align256(Mp * sizeof(int2)) +
         align256(Mp * (ctx->cfg.head_dim / 2) * sizeof(float2));
}
struct GemmWs {
  void *A;
  int2 *map;
  float2 *cs;
};
GemmWs gemm_layout(const lacache_ctx *ctx, void *ws, int64_t rows) {
  const size_t Mp = (size_t)lc::gemm_rows_padded((int)rows);
  char *p = static_cast<char *>(ws);
  GemmWs g;
  g.A = p;
  p += align256(Mp * ctx->cfg.d_model * 2);
  g.map = reinterpret_cast<int2 *>(p);
  p += align256(Mp * sizeof(int2));
  g.cs = reinterpret_cast<float2 *>(p);
  return g;
}
// Largest number of rows one refresh pass handles for this table.
int64_t prefill_pass_rows(const lacache_seq *seqs, int32_t batch) {
  int64_t most = 0;
  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    int64_t t = 0;
    for (int i = s0; i < std::min(batch, s0 + kMaxInline); ++i) t += seqs[i].seq_len;
    most = std::max(most, std::min<int64_t>(t, lc::kPrefillChunk));
  }
  return most;
}

lc::SeqArgs slice_args(const lacache_seq *seqs, int s0, int ns) {
  lc::SeqArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  sa.n = ns;
  for (int i = 0; i < ns; ++i) {
    sa.off[i] = seqs[s0 + i].seq_offset;
    sa.len[i] = seqs[s0 + i].seq_len;
    sa.bs[i] = seqs[s0 + i].block_start;
    sa.be[i] = seqs[s0 + i].block_end;
  }
  return sa;
}

hipEvent_t take_event(lacache_ctx *ctx) {
  if (!ctx->free_events.empty()) {
    hipEvent_t e = ctx->free_events.back();
    ctx->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch(events)` (returning hipError_t); when profiling, the launch
// carries a start/stop event pair stamped by the dispatch itself.
template <typename F> hipError_t timed(lacache_ctx *ctx, int kernel, hipStream_t s, F &&launch) {
  (void)s;
  if (!ctx->profiling) return launch(lc::LaunchEvents{});
  lc::LaunchEvents ev;
  ev.start = take_event(ctx);
  ev.stop = take_event(ctx);
  if (!ev.start || !ev.stop) return hipErrorOutOfMemory;
  hipError_t e = launch(ev);
  if (e == hipSuccess) ctx->marks.push_back({kernel, ev.start, ev.stop});
  return e;
}

lc::DType dtype_of(const lacache_ctx *ctx) { return ctx->cfg.dtype == LACACHE_BF16 ? lc::kBF16 : lc::kF32; }

float scale_log2(const lacache_ctx *ctx) {
  const double s = ctx->cfg.sm_scale > 0 ? (double)ctx->cfg.sm_scale : 1.0 / std::sqrt((double)ctx->cfg.head_dim);
  return (float)(s * 1.4426950408889634);
}

lacache_status hip_fail(lacache_ctx *ctx, const char *what, hipError_t e) {
  return fail(ctx, LACACHE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

lacache_status check_cache(lacache_ctx *ctx, const lacache_cache *c, bool facache) {
  if (!c) return fail(ctx, LACACHE_ERR_INVALID_ARG, "cache is NULL");
  const void *ptrs[7] = {c->h, c->q, c->k, c->v, c->m, c->l, c->o};
  const char *names[7] = {"h", "q", "k", "v", "m", "l", "o"};
  for (int i = 0; i < (facache ? 7 : 4); ++i) {
    if (!ptrs[i]) return fail(ctx, LACACHE_ERR_INVALID_ARG, "cache.%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(ctx, LACACHE_ERR_INVALID_ARG, "cache.%s is not 16-byte aligned", names[i]);
  }
  if (c->n_rows < 1) return fail(ctx, LACACHE_ERR_INVALID_ARG, "cache.n_rows must be >= 1");
  return LACACHE_OK;
}

lacache_status check_weights(lacache_ctx *ctx, const lacache_weights *w) {
  if (!w || !w->embed || !w->gamma || !w->w_qkv) return fail(ctx, LACACHE_ERR_INVALID_ARG, "weights or a weight pointer is NULL");
  if (!aligned16(w->embed) || !aligned16(w->gamma) || !aligned16(w->w_qkv) || !aligned16(w->w_qkv_packed))
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  if (w->w_qkv_packed && !gemm_capable(ctx))
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "w_qkv_packed given, but this configuration has no packed form");
  return LACACHE_OK;
}

lc::QkvArgs qkv_args(lacache_ctx *ctx, const lacache_weights *w, const lacache_cache *c, const int32_t *ids, int mode) {
  lc::QkvArgs a;
  std::memset(&a, 0, sizeof(a));
  a.ids = ids;
  a.E = w->embed;
  a.gamma = w->gamma;
  a.W = w->w_qkv;
  a.h = c->h;
  a.q = c->q;
  a.k = c->k;
  a.v = c->v;
  a.rope = ctx->rope;
  a.flags = ctx->flags;
  a.mode = mode;
  a.vocab = ctx->cfg.vocab;
  a.D = ctx->cfg.d_model;
  a.H = ctx->cfg.n_heads;
  a.Hkv = ctx->cfg.n_kv_heads;
  a.dh = ctx->cfg.head_dim;
  a.eps = ctx->cfg.rms_eps;
  return a;
}

int features(const lacache_ctx *ctx) {
  return (ctx->cfg.n_heads + 2 * ctx->cfg.n_kv_heads) * ctx->cfg.head_dim;
}

}  // namespace

extern "C" {

const char *lacache_status_string(lacache_status s) {
  switch (s) {
    case LACACHE_OK: return "ok";
    case LACACHE_ERR_INVALID_ARG: return "invalid argument";
    case LACACHE_ERR_UNSUPPORTED: return "unsupported";
    case LACACHE_ERR_WORKSPACE: return "workspace missing or too small";
    case LACACHE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *lacache_last_error(const lacache_ctx *ctx) { return ctx ? ctx->last_error.c_str() : "NULL context"; }

lacache_status lacache_create(const lacache_config *cfg, lacache_ctx **out) {
  if (!out) return LACACHE_ERR_INVALID_ARG;
  *out = nullptr;
  if (!cfg) return LACACHE_ERR_INVALID_ARG;
  const lacache_config &c = *cfg;
  if (c.head_dim != 64 && c.head_dim != 128) return LACACHE_ERR_UNSUPPORTED;
  if (c.d_model < 256 || c.d_model % 256 != 0 || c.d_model > lc::kQkvMaxD) return LACACHE_ERR_UNSUPPORTED;
  if (c.n_heads < 1 || c.n_kv_heads < 1 || c.n_heads % c.n_kv_heads != 0) return LACACHE_ERR_INVALID_ARG;
  if (c.vocab < 1 || c.max_seq_len < 1 || c.max_seq_len > (1 << 20)) return LACACHE_ERR_INVALID_ARG;
  if (!(c.rope_theta > 0) || !(c.rms_eps >= 0) || !std::isfinite(c.sm_scale)) return LACACHE_ERR_INVALID_ARG;
  if (c.dtype != LACACHE_F32 && c.dtype != LACACHE_BF16) return LACACHE_ERR_INVALID_ARG;

  lacache_ctx *ctx = new lacache_ctx();
  ctx->cfg = c;
  ctx->rope = nullptr;
  ctx->flags = nullptr;
  ctx->split_keys = 0;
  if (const char *env = std::getenv("LACACHE_SPLIT_KEYS")) {
    const int v = std::atoi(env);
    if (v >= 32 && v % 32 == 0) ctx->split_keys = v;
  }
  ctx->refresh_rows = 0;
  if (const char *env = std::getenv("LACACHE_REFRESH_ROWS")) {
    const int v = std::atoi(env);
    if (v == 64 || v == 128) ctx->refresh_rows = v;
  }
  {
    const char *env = std::getenv("LACACHE_LOG");
    lc::set_launch_log(env && env[0] != 0 && std::strcmp(env, "0") != 0);
  }
  ctx->gemm_tile = lc::kGemmTileAuto;
  ctx->fp8_tile = 0;
  if (const char *env = std::getenv("LACACHE_FP8_TILE")) {
    if (!std::strcmp(env, "256")) ctx->fp8_tile = 1;
    else if (!std::strcmp(env, "128")) ctx->fp8_tile = 2;
  }
  ctx->layer_tile = 0;
  if (const char *env = std::getenv("LACACHE_LAYER_TILE")) {
    if (!std::strcmp(env, "256")) ctx->layer_tile = 1;
    else if (!std::strcmp(env, "128")) ctx->layer_tile = 2;
    else if (!std::strcmp(env, "64")) ctx->layer_tile = 3;
    else if (!std::strcmp(env, "128w4")) ctx->layer_tile = 4;
  }
  if (const char *env = std::getenv("LACACHE_GEMM_TILE")) {
    if (!std::strcmp(env, "whole")) ctx->gemm_tile = lc::kGemmTileWhole;
    else if (!std::strcmp(env, "half")) ctx->gemm_tile = lc::kGemmTileHalf;
    else if (!std::strcmp(env, "wide")) ctx->gemm_tile = lc::kGemmTileWide;
  }
  hipError_t e = hipGetDevice(&ctx->device);
  // RoPE angles in double on the host: position * theta^(-2i/d_h), stored as fp32 (cos, sin).
  const int half = c.head_dim / 2;
  std::vector<float2> tab((size_t)c.max_seq_len * half);
  for (int p = 0; p < c.max_seq_len; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * std::pow((double)c.rope_theta, -2.0 * i / (double)c.head_dim);
      tab[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  if (e == hipSuccess) e = hipMalloc(&ctx->rope, tab.size() * sizeof(float2));
  if (e == hipSuccess) e = hipMemcpy(ctx->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMalloc(&ctx->flags, 256);
  if (e == hipSuccess) e = hipMemset(ctx->flags, 0, 256);
  ctx->scratch = nullptr;
  if (e == hipSuccess) e = static_scratch_address(ctx->device, &ctx->scratch);
  if (e == hipSuccess) e = lc::setup_kernel_attributes();
  if (e == hipSuccess) e = lc::setup_gemm_attributes();
  if (e == hipSuccess) e = lc::setup_fp8_attributes();
  if (e == hipSuccess) e = lc::setup_layer_attributes();
  if (e == hipSuccess) e = lc::setup_flashdllm_attributes();
  if (e != hipSuccess) {
    if (ctx->rope) (void)hipFree(ctx->rope);
    if (ctx->flags) (void)hipFree(ctx->flags);
    delete ctx;
    return LACACHE_ERR_HIP;
  }
  *out = ctx;
  return LACACHE_OK;
}

lacache_status lacache_destroy(lacache_ctx *ctx) {
  if (!ctx) return LACACHE_OK;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(ctx->device);
  (void)hipDeviceSynchronize();
  (void)hipFree(ctx->rope);
  (void)hipFree(ctx->flags);
  for (auto &mk : ctx->marks) {
    (void)hipEventDestroy(mk.start);
    (void)hipEventDestroy(mk.stop);
  }
  for (auto e : ctx->free_events) (void)hipEventDestroy(e);
  if (prev >= 0) (void)hipSetDevice(prev);
  delete ctx;
  return LACACHE_OK;
}

lacache_status lacache_workspace_size(const lacache_ctx *cctx, int32_t op, const lacache_seq *seqs, int32_t batch,
                                      size_t *bytes) {
  lacache_ctx *ctx = const_cast<lacache_ctx *>(cctx);
  if (!ctx || !bytes) return LACACHE_ERR_INVALID_ARG;
  *bytes = 0;
  lacache_status st = check_table(ctx, seqs, batch, -1);
  if (st != LACACHE_OK) return st;
  switch (op) {
    case LACACHE_OP_PREFILL:
      *bytes = gemm_capable(ctx) ? gemm_bytes(ctx, prefill_pass_rows(seqs, batch)) : 0;
      return LACACHE_OK;
    case LACACHE_OP_BLOCK_STEP: {
      const int64_t M = block_tokens(seqs, batch);
      // The prep/GEMM workspace whenever the configuration has that path (the
      // weights, packed or not, are known only at the call).
      *bytes = partial_bytes(ctx, partial_rows(split_keys(ctx, seqs, batch), seqs, batch)) +
               (gemm_capable(ctx) ? gemm_bytes(ctx, M) : 0);
      return LACACHE_OK;
    }
    case LACACHE_OP_DUALCACHE_ATTN:
      *bytes = partial_bytes(ctx, partial_rows(split_keys(ctx, seqs, batch), seqs, batch));
      return LACACHE_OK;
    case LACACHE_OP_REFRESH_BLOCK:
      // seqs: the table of the rows to re-project (lacache_refresh_block's proj)
      *bytes = gemm_capable(ctx) ? gemm_bytes(ctx, block_tokens(seqs, batch)) : 0;
      return LACACHE_OK;
    case LACACHE_OP_PROJECT_BLOCK:
      *bytes = gemm_capable(ctx) ? gemm_bytes(ctx, block_tokens(seqs, batch)) : 0;
      return LACACHE_OK;
  }
  return fail(ctx, LACACHE_ERR_INVALID_ARG, "unknown op %d", op);
}

namespace {

// One prep + GEMM pass over tokens [row0, row0 + M) of a slice.
hipError_t run_qkv_gemm(lacache_ctx *ctx, const lacache_weights *w, const lacache_cache *c, const int32_t *ids,
                        const lc::SeqArgs &sa, int mode, int row0, int ids_base, int M, const GemmWs &gw,
                        hipStream_t s) {
  lc::PrepArgs pa;
  std::memset(&pa, 0, sizeof(pa));
  pa.ids = ids;
  pa.E = w->embed;
  pa.gamma = w->gamma;
  pa.h = c->h;
  pa.A = gw.A;
  pa.map = gw.map;
  pa.cs = gw.cs;
  pa.rope = ctx->rope;
  pa.flags = ctx->flags;
  pa.mode = mode;
  pa.M = M;
  pa.M_pad = lc::prep_rows(M, ctx->cfg.d_model, w->w_qkv_packed != nullptr);
  pa.row0 = row0;
  pa.ids_base = ids_base;
  pa.vocab = ctx->cfg.vocab;
  pa.D = ctx->cfg.d_model;
  pa.dh = ctx->cfg.head_dim;
  pa.eps = ctx->cfg.rms_eps;
  const bool fused = w->w_qkv_packed && lc::skinny_fused_supported(M, ctx->cfg.d_model, ctx->cfg.vocab);
  if (!fused) {
    hipError_t e = timed(ctx, LACACHE_KERNEL_QKV_PREP, s, [&](const lc::LaunchEvents &ev) { return lc::launch_qkv_prep(sa, pa, s, ev); });
    if (e != hipSuccess) return e;
  }
  lc::GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.A = gw.A;
  ga.W = w->w_qkv;
  ga.Wp = w->w_qkv_packed;
  ga.map = gw.map;
  ga.cs = gw.cs;
  ga.q = c->q;
  ga.k = c->k;
  ga.v = c->v;
  ga.flags = ctx->flags;
  ga.M = M;
  ga.D = ctx->cfg.d_model;
  ga.F = features(ctx);
  ga.H = ctx->cfg.n_heads;
  ga.Hkv = ctx->cfg.n_kv_heads;
  if (fused)
    return timed(ctx, LACACHE_KERNEL_QKV_GEMM, s, [&](const lc::LaunchEvents &ev) {
      return lc::launch_qkv_skinny_fused(ctx->cfg.head_dim, sa, pa, ga, s, ev);
    });
  return timed(ctx, LACACHE_KERNEL_QKV_GEMM, s, [&](const lc::LaunchEvents &ev) { return lc::launch_qkv_gemm(ctx->cfg.head_dim, ga, ctx->gemm_tile, s, ev); });
}

}  // namespace

namespace {
// The launch's samples reordered longest first, every prefix array rebuilt
// from the samples' own counts in the new order.  A launch whose items cost
// in proportion to their sample's length finishes sooner when the long ones
// start first (the dispatcher starts workgroups in index order).  Only for
// launches that address rows through each sample's seq_offset and block
// (qmode = omode = 0): pre[0] then no longer follows the caller's sample
// order of q_block / out_block.
lc::SeqArgs longest_first(const lc::SeqArgs &sa) {
  int idx[kMaxInline];
  for (int i = 0; i < sa.n; ++i) idx[i] = i;
  std::stable_sort(idx, idx + sa.n, [&](int x, int y) { return sa.len[x] > sa.len[y]; });
  lc::SeqArgs r = sa;
  for (int i = 0; i < sa.n; ++i) {
    const int j = idx[i];
    r.off[i] = sa.off[j];
    r.len[i] = sa.len[j];
    r.bs[i] = sa.bs[j];
    r.be[i] = sa.be[j];
    for (int k = 0; k < 4; ++k) r.pre[k][i + 1] = r.pre[k][i] + (sa.pre[k][j + 1] - sa.pre[k][j]);
  }
  return r;
}
// The refresh attention of one slice (block table sa, rows by seq_offset):
// every row against every key of its sample, invariant keys first, with the
// FACache snapshot of the invariant rows; O and LSE of every row.
hipError_t refresh_attention(lacache_ctx *ctx, const lacache_cache *cache, const lc::SeqArgs &slice, void *out,
                             float *lse, hipStream_t s) {
  const lc::DType dt = dtype_of(ctx);
  const int dh = ctx->cfg.head_dim, H = ctx->cfg.n_heads, ns = slice.n;
  // bf16 contexts (16-bit caches) run the streaming refresh: 128-row items
  // (two row blocks per wave), or 64-row items when 128-row ones would leave
  // compute units without a workgroup.
  const bool streaming = dt == lc::kBF16;
  auto items = [&](int rows) {
    int64_t n = 0;
    for (int i = 0; i < ns; ++i) n += (slice.len[i] + rows - 1) / rows;
    return n * H;
  };
  int mb = lc::kRefreshMB;
  if (streaming) {
    if (ctx->refresh_rows) mb = ctx->refresh_rows / 64;
    else if (items(64 * lc::kRefreshMB) < lc::device_cus()) mb = 1;
  }
  const int rows_item = streaming ? 64 * mb : lc::kRowsR;
  lc::SeqArgs sa = slice;
  for (int i = 0; i < ns; ++i) sa.pre[1][i + 1] = sa.pre[1][i] + (sa.len[i] + rows_item - 1) / rows_item;
  lc::AttnArgs aa;
  std::memset(&aa, 0, sizeof(aa));
  aa.q = cache->q;
  aa.k = cache->k;
  aa.v = cache->v;
  aa.out = out;
  aa.lse = lse;
  aa.m_w = cache->m;
  aa.l_w = cache->l;
  aa.o_w = cache->o;
  aa.H = H;
  aa.Hkv = ctx->cfg.n_kv_heads;
  aa.scale_log2 = scale_log2(ctx);
  // Every refresh item of a sample streams all of its keys: the streaming
  // launch takes the samples longest first.
  const lc::SeqArgs sr = streaming ? longest_first(sa) : sa;
  return timed(ctx, LACACHE_KERNEL_REFRESH_ATTN, s, [&](const lc::LaunchEvents &ev) {
    return streaming ? lc::launch_refresh_stream(dh, mb, sr, aa, sr.pre[1][ns] * H, s, ev)
                     : lc::launch_refresh_attn(dt, dh, sa, aa, sa.pre[1][ns] * H, s, ev);
  });
}

// The projection of the block rows of one slice (block table sa with pre[0]
// the prefix sums of its block lengths): embedding gather, RMSNorm, QKV,
// RoPE and the cache write of rows [block_start, block_end) of each sample;
// block_ids[row_base ..] are the slice's block ids.
hipError_t project_block_rows(lacache_ctx *ctx, const lacache_weights *w, const lacache_cache *cache,
                              const int32_t *block_ids, const lc::SeqArgs &sa, int row_base, bool gemm, char *gemm_ws,
                              hipStream_t s) {
  const int M = sa.pre[0][sa.n];
  if (gemm) return run_qkv_gemm(ctx, w, cache, block_ids, sa, 0, 0, row_base, M, gemm_layout(ctx, gemm_ws, M), s);
  lc::QkvArgs qa = qkv_args(ctx, w, cache, block_ids, 0);
  qa.M = M;
  qa.ids_base = row_base;
  const lc::DType dt = dtype_of(ctx);
  return timed(ctx, LACACHE_KERNEL_QKV, s,
               [&](const lc::LaunchEvents &ev) { return lc::launch_qkv(dt, sa, qa, features(ctx), s, ev); });
}
}  // namespace

lacache_status lacache_prefill_cache(lacache_ctx *ctx, const lacache_weights *w, const int32_t *ids,
                                     const lacache_seq *seqs, int32_t batch, const lacache_cache *cache, void *out,
                                     float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if ((st = check_weights(ctx, w)) != LACACHE_OK) return st;
  if ((st = check_cache(ctx, cache, true)) != LACACHE_OK) return st;
  if (!ids) return fail(ctx, LACACHE_ERR_INVALID_ARG, "ids is NULL");
  if (!out || !aligned16(out)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "out is NULL or not 16-byte aligned");
  if ((st = check_table(ctx, seqs, batch, cache->n_rows)) != LACACHE_OK) return st;
  const bool gemm = gemm_capable(ctx);
  const size_t need = gemm ? gemm_bytes(ctx, prefill_pass_rows(seqs, batch)) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(ctx, LACACHE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes,
                workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const lc::DType dt = dtype_of(ctx);

  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    const int ns = std::min(kMaxInline, batch - s0);
    lc::SeqArgs sa = slice_args(seqs, s0, ns);
    for (int i = 0; i < ns; ++i) sa.pre[0][i + 1] = sa.pre[0][i] + sa.len[i];
    hipError_t e = hipSuccess;
    if (gemm) {
      // Rows of the slice in passes of at most kPrefillChunk tokens.
      for (int r0 = 0; r0 < sa.pre[0][ns]; r0 += lc::kPrefillChunk) {
        const int Mc = std::min(lc::kPrefillChunk, sa.pre[0][ns] - r0);
        const GemmWs gw = gemm_layout(ctx, workspace, Mc);
        e = run_qkv_gemm(ctx, w, cache, ids, sa, 1, r0, 0, Mc, gw, s);
        if (e != hipSuccess) return hip_fail(ctx, "prefill qkv launch", e);
      }
    } else {
      lc::QkvArgs qa = qkv_args(ctx, w, cache, ids, 1);
      qa.M = sa.pre[0][ns];
      e = timed(ctx, LACACHE_KERNEL_QKV, s, [&](const lc::LaunchEvents &ev) { return lc::launch_qkv(dt, sa, qa, features(ctx), s, ev); });
      if (e != hipSuccess) return hip_fail(ctx, "prefill qkv launch", e);
    }

    e = refresh_attention(ctx, cache, sa, out, lse, s);
    if (e != hipSuccess) return hip_fail(ctx, "refresh attention launch", e);
  }
  return LACACHE_OK;
}

namespace {

// Rows per wave of the streaming invariant-row kernel (bf16 contexts).  0
// (the one-tile-per-workgroup kernel with the merge folded in) for fp32,
// where a block of the slice exceeds what the streaming kernel serves, or
// where the launch is small (at most kStreamItems 64-row tiles x heads): then
// nothing is left to overlap and the separate merge launch only adds.
// The launch lasts as long as its busiest CU, so the segments balance the
// work: equal batches split every (sample, head) into equal segments, about
// four per CU in all; batches of unequal lengths take short segments (192
// rows) that the dispatcher can spread evenly.  Measured on the batched16,
// long4 and varlen32 workloads against fixed segment lengths of 128..2432
// (and, with four waves per workgroup, 128..384 on varlen32).
constexpr int64_t kStreamItems = 2048;
int stream_segment_rows(const lc::SeqArgs &sa, int H, lc::DType dt) {
  if (dt != lc::kBF16) return 0;
  int64_t tiles = 0, rows = 0;
  int nu0 = -1;
  bool equal = true;
  for (int i = 0; i < sa.n; ++i) {
    const int B = sa.be[i] - sa.bs[i];
    if (B > lc::kStreamMaxBlock) return 0;
    const int nU = sa.len[i] - B;
    tiles += (nU + 63) / 64;
    rows += nU;
    if (nU > 0) {
      if (nu0 < 0) nu0 = nU;
      else if (nU != nu0) equal = false;
    }
  }
  if (tiles * H <= kStreamItems || nu0 <= 0) return 0;
  if (!equal) return 192;
  const int64_t target = std::max<int64_t>(16, rows * H / (4 * (int64_t)lc::device_cus()));
  const int nseg = std::max<int64_t>(1, (nu0 + target - 1) / target);
  return ((nu0 + nseg - 1) / nseg + 15) / 16 * 16;
}

// Workspace of one block step with these weights (the packed weight decides
// the projection path) and block table.
size_t block_step_bytes(const lacache_ctx *ctx, const lacache_weights *w, const lacache_seq *seqs, int32_t batch) {
  const int64_t M = block_tokens(seqs, batch);
  return partial_bytes(ctx, partial_rows(split_keys(ctx, seqs, batch), seqs, batch)) +
         (step_uses_prep(ctx, w, M) ? gemm_bytes(ctx, M) : 0);
}

void plan_block_rows(int split, lc::SeqArgs &sa) {
  for (int i = 0; i < sa.n; ++i) {
    const int B = sa.be[i] - sa.bs[i];
    const int nch = nchunks(split, sa.len[i]);
    sa.pre[0][i + 1] = sa.pre[0][i] + B;
    sa.pre[1][i + 1] = sa.pre[1][i] + nch * ((B + lc::kRowsA - 1) / lc::kRowsA);
    sa.pre[3][i + 1] = sa.pre[3][i] + nch * B;
  }
}

}  // namespace

lacache_status lacache_block_step(lacache_ctx *ctx, const lacache_weights *w, const int32_t *block_ids,
                                  const lacache_seq *seqs, int32_t batch, const lacache_cache *cache, void *out,
                                  float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if ((st = check_weights(ctx, w)) != LACACHE_OK) return st;
  if ((st = check_cache(ctx, cache, true)) != LACACHE_OK) return st;
  if (!block_ids) return fail(ctx, LACACHE_ERR_INVALID_ARG, "block_ids is NULL");
  if (!out || !aligned16(out)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "out is NULL or not 16-byte aligned");
  if ((st = check_table(ctx, seqs, batch, cache->n_rows)) != LACACHE_OK) return st;
  int direct = 0;
  const int split = split_keys(ctx, seqs, batch, &direct);
  const int64_t P = partial_rows(split, seqs, batch);
  const int64_t Mall = block_tokens(seqs, batch);
  const bool gemm = step_uses_prep(ctx, w, Mall);
  const size_t need = block_step_bytes(ctx, w, seqs, batch);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(ctx, LACACHE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes,
                workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const lc::DType dt = dtype_of(ctx);
  const int dh = ctx->cfg.head_dim, H = ctx->cfg.n_heads;
  const Partials part = partial_layout(ctx, workspace, P);
  char *gemm_ws = static_cast<char *>(workspace) + partial_bytes(ctx, P);

  int row_base = 0, part_base = 0;
  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    const int ns = std::min(kMaxInline, batch - s0);
    lc::SeqArgs sa = slice_args(seqs, s0, ns);
    plan_block_rows(split, sa);
    const int seg_rows = stream_segment_rows(sa, H, dt);
    for (int i = 0; i < ns; ++i) {
      const int nU = sa.len[i] - (sa.be[i] - sa.bs[i]);
      sa.pre[2][i + 1] = sa.pre[2][i] + (seg_rows ? (nU + seg_rows - 1) / seg_rows : (nU + lc::kRowsB - 1) / lc::kRowsB);
    }
    // Small launches run the block rows' partials and the invariant rows in
    // one launch.  A second round of workgroups would pay the memory latency
    // again, so the key chunks grow (fewer partials, more tiles per
    // workgroup) until the launch is resident at once, if it can be.  Fewer
    // partial rows than the workspace was sized for.
    const bool combined = !seg_rows && !direct;
    int split_s = split;
    if (combined && ctx->split_keys <= 0) {
      const int cap = lc::attn_ab_capacity(dt, dh, sa);
      int max_len = 1;
      for (int i = 0; i < ns; ++i) max_len = std::max(max_len, sa.len[i]);
      while (sa.pre[1][ns] * H + sa.pre[2][ns] * H > cap && split_s < max_len) {
        split_s *= 2;
        plan_block_rows(split_s, sa);
      }
    }
    const int M = sa.pre[0][ns];

    hipError_t e = project_block_rows(ctx, w, cache, block_ids, sa, row_base, gemm, gemm_ws, s);
    if (e != hipSuccess) return hip_fail(ctx, "block-step qkv launch", e);

    lc::AttnArgs aa;
    std::memset(&aa, 0, sizeof(aa));
    aa.q = cache->q;
    aa.k = cache->k;
    aa.v = cache->v;
    aa.out = out;
    aa.lse = lse;
    aa.m_c = cache->m;
    aa.l_c = cache->l;
    aa.o_c = cache->o;
    aa.part_ml = part.ml;
    aa.part_o = part.o;
    aa.qmode = 0;
    aa.omode = 0;
    aa.row_base = row_base;
    aa.part_base = part_base;
    aa.H = H;
    aa.Hkv = ctx->cfg.n_kv_heads;
    aa.split_keys = split_s;
    aa.seg_rows = seg_rows;
    aa.direct = direct;
    aa.scale_log2 = scale_log2(ctx);
    if (combined) {
      // Small launches: the block rows' partials and the invariant rows in one
      // launch (their latencies overlap), then the merge.
      e = timed(ctx, LACACHE_KERNEL_ATTN, s, [&](const lc::LaunchEvents &ev) {
        return lc::launch_attn_ab(dt, dh, sa, aa, sa.pre[1][ns] * H, sa.pre[2][ns] * H, s, ev);
      });
      if (e != hipSuccess) return hip_fail(ctx, "block-step attention launch", e);
      e = timed(ctx, LACACHE_KERNEL_MERGE, s, [&](const lc::LaunchEvents &ev) { return lc::launch_merge(dt, dh, sa, aa, M, s, ev); });
      if (e != hipSuccess) return hip_fail(ctx, "block-step merge launch", e);
      row_base += M;
      part_base += sa.pre[3][ns];
      continue;
    }
    // Whole-sequence items cost in proportion to their sample's length: the
    // launch takes them longest first (it writes O and LSE at each sample's
    // own rows, qmode = omode = 0).
    const lc::SeqArgs sb = direct ? longest_first(sa) : sa;
    e = timed(ctx, LACACHE_KERNEL_BLOCK_ROWS, s, [&](const lc::LaunchEvents &ev) {
      return lc::launch_block_rows(dt, dh, sb, aa, sb.pre[1][ns] * H, s, ev);
    });
    if (e != hipSuccess) return hip_fail(ctx, "block-step block-rows launch", e);
    if (seg_rows) {
      // Blocks of at most 64 keys: the block rows' merge (unless the block-row
      // kernel finished them), then the streaming invariant-row kernel.
      if (!aa.direct) {
        e = timed(ctx, LACACHE_KERNEL_MERGE, s, [&](const lc::LaunchEvents &ev) { return lc::launch_merge(dt, dh, sa, aa, M, s, ev); });
        if (e != hipSuccess) return hip_fail(ctx, "block-step merge launch", e);
      }
      e = timed(ctx, LACACHE_KERNEL_INVARIANT_ROWS, s, [&](const lc::LaunchEvents &ev) {
        return lc::launch_invariant_stream(dt, dh, sa, aa, s, ev);
      });
    } else {
      const int Mmerge = aa.direct ? 0 : M;
      e = timed(ctx, LACACHE_KERNEL_INVARIANT_ROWS, s, [&](const lc::LaunchEvents &ev) {
        return lc::launch_invariant_rows(dt, dh, sa, aa, sa.pre[2][ns] * H, Mmerge, s, ev);
      });
    }
    if (e != hipSuccess) return hip_fail(ctx, "block-step invariant-rows launch", e);
    row_base += M;
    part_base += sa.pre[3][ns];
  }
  return LACACHE_OK;
}

lacache_status lacache_project_block(lacache_ctx *ctx, const lacache_weights *w, const int32_t *block_ids,
                                     const lacache_seq *seqs, int32_t batch, const lacache_cache *cache,
                                     void *workspace, size_t workspace_bytes, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if ((st = check_weights(ctx, w)) != LACACHE_OK) return st;
  if ((st = check_cache(ctx, cache, false)) != LACACHE_OK) return st;
  if (!block_ids) return fail(ctx, LACACHE_ERR_INVALID_ARG, "block_ids is NULL");
  if ((st = check_table(ctx, seqs, batch, cache->n_rows)) != LACACHE_OK) return st;
  const int64_t Mall = block_tokens(seqs, batch);
  const bool gemm = step_uses_prep(ctx, w, Mall);
  const size_t need = gemm ? gemm_bytes(ctx, Mall) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(ctx, LACACHE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes,
                workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int row_base = 0;
  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    const int ns = std::min(kMaxInline, batch - s0);
    lc::SeqArgs sa = slice_args(seqs, s0, ns);
    for (int i = 0; i < ns; ++i) sa.pre[0][i + 1] = sa.pre[0][i] + (sa.be[i] - sa.bs[i]);
    hipError_t e = project_block_rows(ctx, w, cache, block_ids, sa, row_base, gemm, static_cast<char *>(workspace), s);
    if (e != hipSuccess) return hip_fail(ctx, "block projection launch", e);
    row_base += sa.pre[0][ns];
  }
  return LACACHE_OK;
}

lacache_status lacache_block_step_noalloc(lacache_ctx *ctx, const lacache_weights *w, const int32_t *block_ids,
                                          const lacache_seq *seqs, int32_t batch, const lacache_cache *cache,
                                          void *out, float *lse, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if (ctx->profiling)
    return fail(ctx, LACACHE_ERR_INVALID_ARG,
                "per-kernel profiling is on (it creates events on demand): switch it off for the no-allocation step");
  if (!ctx->scratch) return fail(ctx, LACACHE_ERR_HIP, "no static scratch on device %d", ctx->device);
  if ((st = check_weights(ctx, w)) != LACACHE_OK) return st;
  if ((st = check_cache(ctx, cache, true)) != LACACHE_OK) return st;
  if ((st = check_table(ctx, seqs, batch, cache->n_rows)) != LACACHE_OK) return st;
  const size_t need = block_step_bytes(ctx, w, seqs, batch);
  if (need > kStaticScratchBytes)
    return fail(ctx, LACACHE_ERR_UNSUPPORTED,
                "this block table needs %zu bytes of scratch, the static scratch holds %zu: "
                "use lacache_block_step with a workspace",
                need, kStaticScratchBytes);
  return lacache_block_step(ctx, w, block_ids, seqs, batch, cache, out, lse, ctx->scratch, kStaticScratchBytes,
                            stream);
}

lacache_status lacache_refresh_block(lacache_ctx *ctx, const lacache_weights *w, const int32_t *proj_ids,
                                     const lacache_seq *proj, const lacache_seq *seqs, int32_t batch,
                                     const lacache_cache *cache, void *out, float *lse, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if ((st = check_weights(ctx, w)) != LACACHE_OK) return st;
  if ((st = check_cache(ctx, cache, true)) != LACACHE_OK) return st;
  if (!proj_ids) return fail(ctx, LACACHE_ERR_INVALID_ARG, "proj_ids is NULL");
  if (!out || !aligned16(out)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "out is NULL or not 16-byte aligned");
  if ((st = check_table(ctx, proj, batch, cache->n_rows)) != LACACHE_OK) return st;
  if ((st = check_table(ctx, seqs, batch, cache->n_rows)) != LACACHE_OK) return st;
  for (int i = 0; i < batch; ++i)
    if (proj[i].seq_offset != seqs[i].seq_offset || proj[i].seq_len != seqs[i].seq_len)
      return fail(ctx, LACACHE_ERR_INVALID_ARG, "sample %d: proj and seqs differ in seq_offset or seq_len", i);
  const int64_t Mall = block_tokens(proj, batch);
  const bool gemm = step_uses_prep(ctx, w, Mall);
  const size_t need = gemm ? gemm_bytes(ctx, Mall) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(ctx, LACACHE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes,
                workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int row_base = 0;
  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    const int ns = std::min(kMaxInline, batch - s0);
    lc::SeqArgs sp = slice_args(proj, s0, ns);
    for (int i = 0; i < ns; ++i) sp.pre[0][i + 1] = sp.pre[0][i] + (sp.be[i] - sp.bs[i]);
    hipError_t e = project_block_rows(ctx, w, cache, proj_ids, sp, row_base, gemm, static_cast<char *>(workspace), s);
    if (e != hipSuccess) return hip_fail(ctx, "block-refresh qkv launch", e);
    row_base += sp.pre[0][ns];
    e = refresh_attention(ctx, cache, slice_args(seqs, s0, ns), out, lse, s);
    if (e != hipSuccess) return hip_fail(ctx, "block-refresh attention launch", e);
  }
  return LACACHE_OK;
}

lacache_status lacache_dualcache_attn(lacache_ctx *ctx, const void *q_block, const void *k, const void *v,
                                      int64_t n_rows, const lacache_seq *seqs, int32_t batch, void *out_block,
                                      float *lse_block, void *workspace, size_t workspace_bytes, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if (!q_block || !k || !v || !out_block)
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "q_block, k, v and out_block must not be NULL");
  if (!aligned16(q_block) || !aligned16(k) || !aligned16(v) || !aligned16(out_block))
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "q_block, k, v and out_block must be 16-byte aligned");
  if (n_rows < 1) return fail(ctx, LACACHE_ERR_INVALID_ARG, "n_rows must be >= 1");
  if ((st = check_table(ctx, seqs, batch, n_rows)) != LACACHE_OK) return st;
  int direct = 0;
  const int split = split_keys(ctx, seqs, batch, &direct);
  const int64_t P = partial_rows(split, seqs, batch);
  const size_t need = partial_bytes(ctx, P);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(ctx, LACACHE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes,
                workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const lc::DType dt = dtype_of(ctx);
  const int dh = ctx->cfg.head_dim, H = ctx->cfg.n_heads;
  const Partials part = partial_layout(ctx, workspace, P);

  int row_base = 0, part_base = 0;
  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    const int ns = std::min(kMaxInline, batch - s0);
    lc::SeqArgs sa = slice_args(seqs, s0, ns);
    plan_block_rows(split, sa);
    const int M = sa.pre[0][ns];
    lc::AttnArgs aa;
    std::memset(&aa, 0, sizeof(aa));
    aa.q = q_block;
    aa.k = k;
    aa.v = v;
    aa.out = out_block;
    aa.lse = lse_block;
    aa.part_ml = part.ml;
    aa.part_o = part.o;
    aa.qmode = 1;
    aa.omode = 1;
    aa.row_base = row_base;
    aa.part_base = part_base;
    aa.H = H;
    aa.Hkv = ctx->cfg.n_kv_heads;
    aa.split_keys = split;
    aa.direct = direct;
    aa.scale_log2 = scale_log2(ctx);
    hipError_t e = timed(ctx, LACACHE_KERNEL_BLOCK_ROWS, s, [&](const lc::LaunchEvents &ev) {
      return lc::launch_block_rows(dt, dh, sa, aa, sa.pre[1][ns] * H, s, ev);
    });
    if (e != hipSuccess) return hip_fail(ctx, "dualcache attention launch", e);
    if (!aa.direct) {
      e = timed(ctx, LACACHE_KERNEL_MERGE, s, [&](const lc::LaunchEvents &ev) { return lc::launch_merge(dt, dh, sa, aa, M, s, ev); });
      if (e != hipSuccess) return hip_fail(ctx, "dualcache merge launch", e);
    }
    row_base += M;
    part_base += sa.pre[3][ns];
  }
  return LACACHE_OK;
}

namespace {
bool ffn_capable(const lacache_ctx *ctx, int32_t d_ff) {
  return ctx->cfg.dtype == LACACHE_BF16 && ctx->cfg.d_model % 512 == 0 && d_ff >= 128 && d_ff % 128 == 0;
}
int64_t ffn_rows_padded(int64_t n) { return (n + 255) / 256 * 256; }
struct FfnWs {
  void *xq, *yq, *r;
  float *sx, *sy, *part;
};
// Workspace of one FFN call: x codes [M_pad, D], their scales, y codes
// [M_pad, F], their scales, the residual r when the caller keeps none, and
// the down projection's split partials when it splits.
size_t ffn_ws_layout(const lacache_ctx *ctx, int32_t d_ff, int64_t n_rows, bool own_r, void *base, FfnWs *out) {
  const size_t D = ctx->cfg.d_model, F = d_ff, Mp = (size_t)ffn_rows_padded(n_rows);
  const int M = n_rows > (int64_t)1 << 24 ? 0 : (int)n_rows;
  const size_t sizes[6] = {align256(Mp * D), align256(D / 128 * Mp * 4), align256(Mp * F), align256(F / 128 * Mp * 4),
                           own_r ? align256((size_t)n_rows * D * 2) : 0,
                           align256(lc::fp8_part_bytes(M, (int)Mp, (int)D, (int)F, ctx->fp8_tile))};
  char *p = static_cast<char *>(base);
  size_t off = 0;
  void *ptrs[6];
  for (int i = 0; i < 6; ++i) {
    ptrs[i] = p ? p + off : nullptr;
    off += sizes[i];
  }
  if (out) {
    out->xq = ptrs[0];
    out->sx = static_cast<float *>(ptrs[1]);
    out->yq = ptrs[2];
    out->sy = static_cast<float *>(ptrs[3]);
    out->r = ptrs[4];
    out->part = sizes[5] ? static_cast<float *>(ptrs[5]) : nullptr;
  }
  return off;
}
}  // namespace

lacache_status lacache_ffn_weight_bytes(const lacache_ctx *ctx, int32_t d_ff, size_t *gate_up_bytes,
                                        size_t *gate_up_scale_bytes, size_t *down_bytes, size_t *down_scale_bytes) {
  if (!ctx || !gate_up_bytes || !gate_up_scale_bytes || !down_bytes || !down_scale_bytes) return LACACHE_ERR_INVALID_ARG;
  if (!ffn_capable(ctx, d_ff))
    return fail(ctx, LACACHE_ERR_UNSUPPORTED, "the FP8 FFN needs bf16, d_model a multiple of 512, d_ff a multiple of 128");
  const int D = ctx->cfg.d_model;
  *gate_up_bytes = lc::fp8_packed_bytes(2 * d_ff, D);
  *gate_up_scale_bytes = (size_t)(D / 128) * (2 * d_ff / 128) * sizeof(float);
  *down_bytes = lc::fp8_packed_bytes(D, d_ff);
  *down_scale_bytes = (size_t)(d_ff / 128) * (D / 128) * sizeof(float);
  return LACACHE_OK;
}

lacache_status lacache_ffn_pack_weights(lacache_ctx *ctx, int32_t d_ff, const void *w_gate, const void *w_up,
                                        const void *w_down, void *gate_up, float *s_gate_up, void *down, float *s_down,
                                        void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if (!ffn_capable(ctx, d_ff))
    return fail(ctx, LACACHE_ERR_UNSUPPORTED, "the FP8 FFN needs bf16, d_model a multiple of 512, d_ff a multiple of 128");
  const void *ptrs[7] = {w_gate, w_up, w_down, gate_up, s_gate_up, down, s_down};
  for (const void *p : ptrs)
    if (!p || !aligned16(p)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "a weight pointer is NULL or not 16-byte aligned");
  const int D = ctx->cfg.d_model;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = lc::launch_fp8_pack_weight(w_gate, d_ff, D, 1, gate_up, s_gate_up, 2 * d_ff, s);
  if (e == hipSuccess) e = lc::launch_fp8_pack_weight(w_up, d_ff, D, 2, gate_up, s_gate_up, 2 * d_ff, s);
  if (e == hipSuccess) e = lc::launch_fp8_pack_weight(w_down, D, d_ff, 0, down, s_down, D, s);
  if (e != hipSuccess) return hip_fail(ctx, "FP8 weight packing launch", e);
  return LACACHE_OK;
}

lacache_status lacache_ffn_workspace_size(const lacache_ctx *ctx, int32_t d_ff, int64_t n_rows, int32_t keeps_residual,
                                          size_t *bytes) {
  if (!ctx || !bytes) return LACACHE_ERR_INVALID_ARG;
  *bytes = 0;
  if (!ffn_capable(ctx, d_ff))
    return fail(ctx, LACACHE_ERR_UNSUPPORTED, "the FP8 FFN needs bf16, d_model a multiple of 512, d_ff a multiple of 128");
  if (n_rows < 1 || n_rows > (int64_t)1 << 24)
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "n_rows must be in [1, 2^24] (got %lld)", (long long)n_rows);
  *bytes = ffn_ws_layout(ctx, d_ff, n_rows, !keeps_residual, nullptr, nullptr);
  return LACACHE_OK;
}

lacache_status lacache_ffn_fp8(lacache_ctx *ctx, int32_t d_ff, const lacache_ffn_weights *w, const void *h,
                               const void *attn_out, int64_t n_rows, void *r_out, void *out, void *workspace,
                               size_t workspace_bytes, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if (!ffn_capable(ctx, d_ff))
    return fail(ctx, LACACHE_ERR_UNSUPPORTED, "the FP8 FFN needs bf16, d_model a multiple of 512, d_ff a multiple of 128");
  if (!w || !w->gamma || !w->gate_up || !w->s_gate_up || !w->down || !w->s_down)
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "FFN weights or a weight pointer is NULL");
  const void *ptrs[8] = {w->gamma, w->gate_up, w->s_gate_up, w->down, w->s_down, h, attn_out, out};
  for (const void *p : ptrs)
    if (!p || !aligned16(p)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "a pointer is NULL or not 16-byte aligned");
  if (r_out && !aligned16(r_out)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "r_out is not 16-byte aligned");
  if (n_rows < 1 || n_rows > (int64_t)1 << 24)
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "n_rows must be in [1, 2^24] (got %lld)", (long long)n_rows);
  const size_t need = ffn_ws_layout(ctx, d_ff, n_rows, r_out == nullptr, nullptr, nullptr);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(ctx, LACACHE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes,
                workspace);
  FfnWs ws;
  ffn_ws_layout(ctx, d_ff, n_rows, r_out == nullptr, workspace, &ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = ctx->cfg.d_model, M = (int)n_rows, Mp = (int)ffn_rows_padded(n_rows);
  lc::Fp8NormArgs na;
  na.h = h;
  na.a = attn_out;
  na.gamma = w->gamma;
  na.r = r_out ? r_out : ws.r;
  na.xq = ws.xq;
  na.sx = ws.sx;
  na.M = M;
  na.M_pad = Mp;
  na.D = D;
  na.eps = ctx->cfg.rms_eps;
  hipError_t e = timed(ctx, LACACHE_KERNEL_FFN_NORM, s, [&](const lc::LaunchEvents &ev) { return lc::launch_fp8_addnorm_quant(na, s, ev); });
  if (e != hipSuccess) return hip_fail(ctx, "FFN AddNorm launch", e);
  lc::Fp8GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.A = ws.xq;
  ga.sa = ws.sx;
  ga.B = w->gate_up;
  ga.sw = w->s_gate_up;
  ga.M = M;
  ga.M_pad = Mp;
  ga.N = 2 * d_ff;
  ga.K = D;
  ga.yq = ws.yq;
  ga.sy = ws.sy;
  e = timed(ctx, LACACHE_KERNEL_FFN_GATE_UP, s, [&](const lc::LaunchEvents &ev) { return lc::launch_fp8_gemm_swiglu(ga, s, ev); });
  if (e != hipSuccess) return hip_fail(ctx, "FFN gate-up launch", e);
  lc::Fp8GemmArgs gd;
  std::memset(&gd, 0, sizeof(gd));
  gd.A = ws.yq;
  gd.sa = ws.sy;
  gd.B = w->down;
  gd.sw = w->s_down;
  gd.M = M;
  gd.M_pad = Mp;
  gd.N = D;
  gd.K = d_ff;
  gd.res = na.r;
  gd.out = out;
  gd.part = ws.part;
  e = timed(ctx, LACACHE_KERNEL_FFN_DOWN, s, [&](const lc::LaunchEvents &ev) { return lc::launch_fp8_gemm_resid(gd, ctx->fp8_tile, s, ev); });
  if (e != hipSuccess) return hip_fail(ctx, "FFN down launch", e);
  return LACACHE_OK;
}

namespace {
bool layer_capable(const lacache_ctx *ctx, int32_t d_ff) {
  const int D = ctx->cfg.d_model;
  return ctx->cfg.dtype == LACACHE_BF16 && (D == 512 || D == 1024 || D == 2048 || D == 4096 || D == 8192) &&
         d_ff >= 128 && d_ff % 128 == 0 && (ctx->cfg.n_heads * ctx->cfg.head_dim) % 64 == 0;
}
const char *kLayerNeeds = "the layer finish needs bf16, d_model in {512, 1024, 2048, 4096, 8192}, d_ff a multiple "
                          "of 128 and n_heads * head_dim a multiple of 64";
struct LayerWs {
  void *r, *x, *y;
  float *part;
};
// r [n, D] (when the caller keeps none), x [n, D], y [n, F], all bf16, then
// the split-contraction partials of the three GEMMs (one at a time; none for
// more than 64 rows or where every CU already has an output tile).
size_t layer_ws_layout(const lacache_ctx *ctx, int32_t d_ff, int64_t n, bool own_r, void *base, LayerWs *out) {
  const size_t D = ctx->cfg.d_model, HD = (size_t)ctx->cfg.n_heads * ctx->cfg.head_dim;
  const int M = n > (int64_t)1 << 24 ? 0 : (int)n;
  const size_t part = std::max({lc::bf16_gemm_part_bytes(M, (int)D, (int)HD, lc::kGemmOutBf16),
                                lc::bf16_gemm_part_bytes(M, d_ff, (int)D, lc::kGemmOutSwiglu),
                                lc::bf16_gemm_part_bytes(M, (int)D, d_ff, lc::kGemmOutBf16)});
  const size_t sizes[4] = {own_r ? align256((size_t)n * D * 2) : 0, align256((size_t)n * D * 2),
                           align256((size_t)n * d_ff * 2), align256(part)};
  char *p = static_cast<char *>(base);
  size_t off = 0;
  void *ptrs[4];
  for (int i = 0; i < 4; ++i) {
    ptrs[i] = p && sizes[i] ? p + off : nullptr;
    off += sizes[i];
  }
  if (out) *out = LayerWs{ptrs[0], ptrs[1], ptrs[2], static_cast<float *>(ptrs[3])};
  return off;
}
}  // namespace

lacache_status lacache_layer_finish_workspace_size(const lacache_ctx *ctx, int32_t d_ff, int64_t n_rows,
                                                   int32_t keeps_residual, size_t *bytes) {
  if (!ctx || !bytes) return LACACHE_ERR_INVALID_ARG;
  *bytes = 0;
  if (!layer_capable(ctx, d_ff)) return fail(ctx, LACACHE_ERR_UNSUPPORTED, "%s", kLayerNeeds);
  if (n_rows < 1 || n_rows > (int64_t)1 << 24)
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "n_rows must be in [1, 2^24] (got %lld)", (long long)n_rows);
  *bytes = layer_ws_layout(ctx, d_ff, n_rows, !keeps_residual, nullptr, nullptr);
  return LACACHE_OK;
}

lacache_status lacache_layer_finish(lacache_ctx *ctx, int32_t d_ff, const lacache_layer_weights *w, const void *h,
                                    const void *attn_out, int64_t n_rows, void *r_out, void *out, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if (!layer_capable(ctx, d_ff)) return fail(ctx, LACACHE_ERR_UNSUPPORTED, "%s", kLayerNeeds);
  if (!w) return fail(ctx, LACACHE_ERR_INVALID_ARG, "layer weights are NULL");
  const void *ptrs[8] = {w->w_o, w->gamma, w->w_gate, w->w_up, w->w_down, h, attn_out, out};
  for (const void *p : ptrs)
    if (!p || !aligned16(p)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "a pointer is NULL or not 16-byte aligned");
  if (r_out && !aligned16(r_out)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "r_out is not 16-byte aligned");
  if (n_rows < 1 || n_rows > (int64_t)1 << 24)
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "n_rows must be in [1, 2^24] (got %lld)", (long long)n_rows);
  const size_t need = layer_ws_layout(ctx, d_ff, n_rows, r_out == nullptr, nullptr, nullptr);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(ctx, LACACHE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes,
                workspace);
  LayerWs ws;
  layer_ws_layout(ctx, d_ff, n_rows, r_out == nullptr, workspace, &ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = ctx->cfg.d_model, HD = ctx->cfg.n_heads * ctx->cfg.head_dim, M = (int)n_rows;
  bf16_t *r = static_cast<bf16_t *>(r_out ? r_out : ws.r);
  // r = bf16(h + bf16(O W_o^T))
  lc::Bf16GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.A = static_cast<const bf16_t *>(attn_out);
  g.lda = HD;
  g.B = static_cast<const bf16_t *>(w->w_o);
  g.ldb = HD;
  g.res = static_cast<const bf16_t *>(h);
  g.ldr = D;
  g.out = r;
  g.ldo = D;
  g.M = M;
  g.N = D;
  g.K = HD;
  g.part = ws.part;
  hipError_t e = timed(ctx, LACACHE_KERNEL_LAYER_OPROJ, s, [&](const lc::LaunchEvents &ev) {
    return lc::launch_bf16_gemm(g, lc::kGemmOutBf16, ctx->layer_tile, s, ev);
  });
  if (e != hipSuccess) return hip_fail(ctx, "layer output projection launch", e);
  // x = bf16(RMSNorm(r))
  lc::RowNormArgs na;
  std::memset(&na, 0, sizeof(na));
  na.src = r;
  na.lds = D;
  na.gamma = static_cast<const bf16_t *>(w->gamma);
  na.out = static_cast<bf16_t *>(ws.x);
  na.M = M;
  na.D = D;
  na.eps = ctx->cfg.rms_eps;
  e = timed(ctx, LACACHE_KERNEL_LAYER_NORM, s, [&](const lc::LaunchEvents &ev) { return lc::launch_rmsnorm_rows(na, s, ev); });
  if (e != hipSuccess) return hip_fail(ctx, "layer RMSNorm launch", e);
  // y = bf16(silu(bf16(x W_g^T)) bf16(x W_u^T))
  std::memset(&g, 0, sizeof(g));
  g.A = static_cast<const bf16_t *>(ws.x);
  g.lda = D;
  g.B = static_cast<const bf16_t *>(w->w_gate);
  g.B2 = static_cast<const bf16_t *>(w->w_up);
  g.ldb = D;
  g.out = ws.y;
  g.ldo = d_ff;
  g.M = M;
  g.N = d_ff;
  g.K = D;
  g.part = ws.part;
  e = timed(ctx, LACACHE_KERNEL_LAYER_GATE_UP, s, [&](const lc::LaunchEvents &ev) {
    return lc::launch_bf16_gemm(g, lc::kGemmOutSwiglu, ctx->layer_tile == 2 ? 3 : ctx->layer_tile, s, ev);
  });
  if (e != hipSuccess) return hip_fail(ctx, "layer gate-up launch", e);
  // out = bf16(r + bf16(y W_d^T))
  std::memset(&g, 0, sizeof(g));
  g.A = static_cast<const bf16_t *>(ws.y);
  g.lda = d_ff;
  g.B = static_cast<const bf16_t *>(w->w_down);
  g.ldb = d_ff;
  g.res = r;
  g.ldr = D;
  g.out = out;
  g.ldo = D;
  g.M = M;
  g.N = D;
  g.K = d_ff;
  g.part = ws.part;
  e = timed(ctx, LACACHE_KERNEL_LAYER_DOWN, s, [&](const lc::LaunchEvents &ev) {
    return lc::launch_bf16_gemm(g, lc::kGemmOutBf16, ctx->layer_tile, s, ev);
  });
  if (e != hipSuccess) return hip_fail(ctx, "layer down launch", e);
  return LACACHE_OK;
}

namespace {
bool sampler_capable(const lacache_ctx *ctx, int32_t vocab) {
  const int D = ctx->cfg.d_model;
  return ctx->cfg.dtype == LACACHE_BF16 && (D == 512 || D == 1024 || D == 2048 || D == 4096 || D == 8192) &&
         vocab >= 8 && vocab % 8 == 0;
}
const char *kSamplerNeeds = "the sampler needs bf16, d_model in {512, 1024, 2048, 4096, 8192} and a vocabulary "
                            "that is a multiple of 8";
// z [M, D] bf16 (final norm of the block rows), logits [M, V] fp32, the
// softmax's chunk partials [M, C] float2 and [M, C] int32, and row (max, sum)
// [M] float2, each at a multiple of 256 bytes.
struct SamplerWs {
  void *z;
  float *logits;
  float2 *part;
  int *part_idx;
  float2 *row_stat;
};
size_t sampler_ws(const lacache_ctx *ctx, int64_t M, int32_t vocab, void *base, SamplerWs *out) {
  const size_t C = (size_t)lc::softmax_chunks(vocab);
  const size_t sizes[5] = {align256((size_t)M * ctx->cfg.d_model * 2), align256((size_t)M * vocab * 4),
                           align256((size_t)M * C * 8), align256((size_t)M * C * 4), align256((size_t)M * 8)};
  char *p = static_cast<char *>(base);
  size_t off = 0;
  void *ptrs[5];
  for (int i = 0; i < 5; ++i) {
    ptrs[i] = p ? p + off : nullptr;
    off += sizes[i];
  }
  if (out) {
    out->z = ptrs[0];
    out->logits = static_cast<float *>(ptrs[1]);
    out->part = static_cast<float2 *>(ptrs[2]);
    out->part_idx = static_cast<int *>(ptrs[3]);
    out->row_stat = static_cast<float2 *>(ptrs[4]);
  }
  return off;
}
}  // namespace

lacache_status lacache_sampler_workspace_size(const lacache_ctx *cctx, int32_t vocab, const lacache_seq *seqs,
                                              int32_t batch, size_t *bytes) {
  lacache_ctx *ctx = const_cast<lacache_ctx *>(cctx);
  if (!ctx || !bytes) return LACACHE_ERR_INVALID_ARG;
  *bytes = 0;
  if (!sampler_capable(ctx, vocab)) return fail(ctx, LACACHE_ERR_UNSUPPORTED, "%s", kSamplerNeeds);
  lacache_status st = check_table(ctx, seqs, batch, -1, INT32_MAX);
  if (st != LACACHE_OK) return st;
  *bytes = sampler_ws(ctx, block_tokens(seqs, batch), vocab, nullptr, nullptr);
  return LACACHE_OK;
}

lacache_status lacache_sampler_cut(lacache_ctx *ctx, const void *hidden, int64_t n_rows, const lacache_seq *seqs,
                                   int32_t batch, const void *gamma_final, const void *w_lm, int32_t vocab,
                                   int32_t *token, float *confidence, float *probs, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if (!sampler_capable(ctx, vocab)) return fail(ctx, LACACHE_ERR_UNSUPPORTED, "%s", kSamplerNeeds);
  if ((st = check_table(ctx, seqs, batch, n_rows, INT32_MAX)) != LACACHE_OK) return st;
  const void *ptrs[5] = {hidden, gamma_final, w_lm, token, confidence};
  for (const void *p : ptrs)
    if (!p || !aligned16(p)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "a pointer is NULL or not 16-byte aligned");
  if (probs && !aligned16(probs)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "probs is not 16-byte aligned");
  const int64_t M = block_tokens(seqs, batch);
  if (M > (int64_t)1 << 24) return fail(ctx, LACACHE_ERR_UNSUPPORTED, "%lld block rows (at most 2^24)", (long long)M);
  const size_t need = sampler_ws(ctx, M, vocab, nullptr, nullptr);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(ctx, LACACHE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes,
                workspace);
  SamplerWs sw;
  sampler_ws(ctx, M, vocab, workspace, &sw);
  void *z = sw.z;
  float *logits = sw.logits;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = ctx->cfg.d_model;
  // The cut: the final norm reads only the block rows (block-table order).
  int64_t row_base = 0;
  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    const int ns = std::min(batch - s0, kMaxInline);
    lc::RowNormArgs na;
    std::memset(&na, 0, sizeof(na));
    na.sa = slice_args(seqs, s0, ns);
    na.sa.pre[0][0] = 0;
    for (int i = 0; i < ns; ++i) na.sa.pre[0][i + 1] = na.sa.pre[0][i] + (na.sa.be[i] - na.sa.bs[i]);
    na.gather = 1;
    na.src = static_cast<const bf16_t *>(hidden);
    na.lds = D;
    na.gamma = static_cast<const bf16_t *>(gamma_final);
    na.out = static_cast<bf16_t *>(z) + row_base * D;
    na.M = na.sa.pre[0][ns];
    na.D = D;
    na.eps = ctx->cfg.rms_eps;
    hipError_t e = timed(ctx, LACACHE_KERNEL_SAMPLER_NORM, s, [&](const lc::LaunchEvents &ev) {
      return lc::launch_rmsnorm_rows(na, s, ev);
    });
    if (e != hipSuccess) return hip_fail(ctx, "sampler final norm launch", e);
    row_base += na.M;
  }
  lc::Bf16GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.A = static_cast<const bf16_t *>(z);
  g.lda = D;
  g.B = static_cast<const bf16_t *>(w_lm);
  g.ldb = D;
  g.out = logits;
  g.ldo = vocab;
  g.M = (int)M;
  g.N = vocab;
  g.K = D;
  hipError_t e = timed(ctx, LACACHE_KERNEL_SAMPLER_LMHEAD, s, [&](const lc::LaunchEvents &ev) {
    return lc::launch_bf16_gemm(g, lc::kGemmOutF32, ctx->layer_tile, s, ev);
  });
  if (e != hipSuccess) return hip_fail(ctx, "sampler lm-head launch", e);
  lc::SoftmaxArgs sm;
  sm.logits = logits;
  sm.ld = vocab;
  sm.token = token;
  sm.conf = confidence;
  sm.probs = probs;
  sm.ldp = vocab;
  sm.part = sw.part;
  sm.part_idx = sw.part_idx;
  sm.row_stat = sw.row_stat;
  sm.M = (int)M;
  sm.V = vocab;
  e = timed(ctx, LACACHE_KERNEL_SAMPLER_SOFTMAX, s, [&](const lc::LaunchEvents &ev) {
    return lc::launch_softmax_argmax(sm, s, ev);
  });
  if (e != hipSuccess) return hip_fail(ctx, "sampler softmax launch", e);
  return LACACHE_OK;
}

namespace {
bool flashdllm_capable(const lacache_ctx *ctx) {
  return ctx->cfg.dtype == LACACHE_BF16 && (ctx->cfg.head_dim == 64 || ctx->cfg.head_dim == 128);
}
const char *kFlashNeeds = "the selective update and verify need bf16 (fp16 RoPECache) and head_dim 64 or 128";
int max_seq_len_of(const lacache_seq *seqs, int32_t batch) {
  int m = 0;
  for (int i = 0; i < batch; ++i) m = std::max(m, seqs[i].seq_len);
  return m;
}
// Host prefix sums over samples (verify tokens or search positions): non-decreasing, from >= 0.
lacache_status check_prefix(lacache_ctx *ctx, const int32_t *start, int32_t batch, int max_per_sample, const char *what) {
  if (!start) return fail(ctx, LACACHE_ERR_INVALID_ARG, "%s is NULL", what);
  if (start[0] < 0) return fail(ctx, LACACHE_ERR_INVALID_ARG, "%s[0] < 0", what);
  for (int i = 0; i < batch; ++i) {
    const int n = start[i + 1] - start[i];
    if (n < 0) return fail(ctx, LACACHE_ERR_INVALID_ARG, "%s decreases at sample %d", what, i);
    if (max_per_sample > 0 && n > max_per_sample)
      return fail(ctx, LACACHE_ERR_UNSUPPORTED, "%s: %d entries for sample %d (at most %d)", what, n, i, max_per_sample);
  }
  return LACACHE_OK;
}
}  // namespace

lacache_status lacache_track_workspace_size(const lacache_ctx *ctx, int64_t n_rows, size_t *bytes) {
  if (!ctx || !bytes || n_rows < 1) return LACACHE_ERR_INVALID_ARG;
  *bytes = align256((size_t)ctx->cfg.n_heads * n_rows * sizeof(float));
  return LACACHE_OK;
}

lacache_status lacache_track_select(lacache_ctx *ctx, const lacache_cache *cache, const float *lse,
                                    const lacache_seq *seqs, int32_t batch, int32_t budget, float *importance,
                                    int32_t *tracked, void *workspace, size_t workspace_bytes, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if (!flashdllm_capable(ctx)) return fail(ctx, LACACHE_ERR_UNSUPPORTED, "%s", kFlashNeeds);
  if ((st = check_cache(ctx, cache, false)) != LACACHE_OK) return st;
  if ((st = check_table(ctx, seqs, batch, cache->n_rows)) != LACACHE_OK) return st;
  if (budget < 1 || budget > 64) return fail(ctx, LACACHE_ERR_UNSUPPORTED, "budget %d (1 .. 64 supported)", budget);
  if (max_seq_len_of(seqs, batch) > lc::kTrackMaxKeys)
    return fail(ctx, LACACHE_ERR_UNSUPPORTED, "sequences of more than %d rows", lc::kTrackMaxKeys);
  if (!lse || !importance || !tracked) return fail(ctx, LACACHE_ERR_INVALID_ARG, "lse, importance or tracked is NULL");
  const size_t need = (size_t)ctx->cfg.n_heads * cache->n_rows * sizeof(float);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(ctx, LACACHE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes,
                workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  lc::TrackArgs ta;
  ta.q = cache->q;
  ta.lse = lse;
  ta.k = cache->k;
  ta.partial = static_cast<float *>(workspace);
  ta.importance = importance;
  ta.tracked = tracked;
  ta.n_rows = cache->n_rows;
  ta.H = ctx->cfg.n_heads;
  ta.Hkv = ctx->cfg.n_kv_heads;
  ta.budget = budget;
  ta.scale_log2 = scale_log2(ctx);
  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    const int ns = std::min(kMaxInline, batch - s0);
    lc::SeqArgs sa = slice_args(seqs, s0, ns);
    for (int i = 0; i < ns; ++i) sa.pre[1][i + 1] = sa.pre[1][i] + (sa.len[i] + 63) / 64;
    ta.sample_base = s0;
    hipError_t e = timed(ctx, LACACHE_KERNEL_TRACK_IMPORTANCE, s, [&](const lc::LaunchEvents &ev) {
      return lc::launch_importance(ctx->cfg.head_dim, sa, ta, s, ev);
    });
    if (e != hipSuccess) return hip_fail(ctx, "importance launch", e);
    e = timed(ctx, LACACHE_KERNEL_TRACK_SELECT, s, [&](const lc::LaunchEvents &ev) {
      return lc::launch_track_select(sa, ta, max_seq_len_of(seqs + s0, ns), s, ev);
    });
    if (e != hipSuccess) return hip_fail(ctx, "tracking selection launch", e);
  }
  return LACACHE_OK;
}

lacache_status lacache_verify_attn(lacache_ctx *ctx, const void *q_ver, const void *k_ver, const void *v_ver,
                                   const int32_t *view, const int32_t *pos, const int32_t *ver_start,
                                   const lacache_cache *cache, const lacache_seq *seqs, int32_t batch, void *out,
                                   float *lse, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if (!flashdllm_capable(ctx)) return fail(ctx, LACACHE_ERR_UNSUPPORTED, "%s", kFlashNeeds);
  if ((st = check_cache(ctx, cache, false)) != LACACHE_OK) return st;
  if ((st = check_table(ctx, seqs, batch, cache->n_rows, INT32_MAX)) != LACACHE_OK) return st;
  if (max_seq_len_of(seqs, batch) > lc::kVerifyMaxKeys)
    return fail(ctx, LACACHE_ERR_UNSUPPORTED, "sequences of more than %d rows", lc::kVerifyMaxKeys);
  if ((st = check_prefix(ctx, ver_start, batch, 0, "ver_start")) != LACACHE_OK) return st;
  const void *ptrs[6] = {q_ver, k_ver, v_ver, view, pos, out};
  for (const void *p : ptrs)
    if (!p || !aligned16(p)) return fail(ctx, LACACHE_ERR_INVALID_ARG, "a pointer is NULL or not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  lc::VerifyArgs va;
  va.q = q_ver;
  va.k_ver = k_ver;
  va.v_ver = v_ver;
  va.view = view;
  va.pos = pos;
  va.k = cache->k;
  va.v = cache->v;
  va.out = out;
  va.lse = lse;
  va.H = ctx->cfg.n_heads;
  va.Hkv = ctx->cfg.n_kv_heads;
  va.scale_log2 = scale_log2(ctx);
  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    const int ns = std::min(kMaxInline, batch - s0);
    lc::SeqArgs sa = slice_args(seqs, s0, ns);
    for (int i = 0; i <= ns; ++i) sa.pre[0][i] = ver_start[s0 + i];
    for (int i = 0; i < ns; ++i) sa.pre[1][i + 1] = sa.pre[1][i] + (ver_start[s0 + i + 1] - ver_start[s0 + i] + 15) / 16;
    hipError_t e = timed(ctx, LACACHE_KERNEL_VERIFY_ATTN, s, [&](const lc::LaunchEvents &ev) {
      return lc::launch_verify_attn(ctx->cfg.head_dim, sa, va, s, ev);
    });
    if (e != hipSuccess) return hip_fail(ctx, "verify attention launch", e);
  }
  return LACACHE_OK;
}

lacache_status lacache_verify_accept(lacache_ctx *ctx, const int32_t *draft, const int32_t *mask_tok,
                                     const float *mask_conf, const int32_t *pos, const int32_t *search_start,
                                     const lacache_seq *seqs, int32_t batch, float gamma, int32_t *ids,
                                     int32_t *n_accepted, void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if ((st = check_table(ctx, seqs, batch, -1, INT32_MAX)) != LACACHE_OK) return st;
  if ((st = check_prefix(ctx, search_start, batch, 64, "search_start")) != LACACHE_OK) return st;
  const void *ptrs[6] = {draft, mask_tok, mask_conf, pos, ids, n_accepted};
  for (const void *p : ptrs)
    if (!p) return fail(ctx, LACACHE_ERR_INVALID_ARG, "a pointer is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  lc::AcceptArgs aa;
  aa.draft = draft;
  aa.mask_tok = mask_tok;
  aa.mask_conf = mask_conf;
  aa.pos = pos;
  aa.ids = ids;
  aa.flags = ctx->flags;
  aa.gamma = gamma;
  for (int s0 = 0; s0 < batch; s0 += kMaxInline) {
    const int ns = std::min(kMaxInline, batch - s0);
    lc::SeqArgs sa = slice_args(seqs, s0, ns);
    for (int i = 0; i <= ns; ++i) sa.pre[0][i] = search_start[s0 + i];
    aa.n_accepted = n_accepted + s0;
    hipError_t e = timed(ctx, LACACHE_KERNEL_VERIFY_ACCEPT, s, [&](const lc::LaunchEvents &ev) {
      return lc::launch_verify_accept(sa, aa, s, ev);
    });
    if (e != hipSuccess) return hip_fail(ctx, "verify acceptance launch", e);
  }
  return LACACHE_OK;
}

lacache_status lacache_packed_weight_size(const lacache_ctx *ctx, size_t *bytes) {
  if (!ctx || !bytes) return LACACHE_ERR_INVALID_ARG;
  *bytes = gemm_capable(ctx) ? lc::packed_qkv_weight_bytes(ctx->cfg.d_model, features(ctx)) : 0;
  return LACACHE_OK;
}

lacache_status lacache_pack_qkv_weight(lacache_ctx *ctx, const void *w_qkv, void *w_packed, size_t packed_bytes,
                                       void *stream) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  if (!gemm_capable(ctx))
    return fail(ctx, LACACHE_ERR_UNSUPPORTED, "packed weights need bf16 and d_model a multiple of 512");
  if (!w_qkv || !w_packed || !aligned16(w_qkv) || !aligned16(w_packed))
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "w_qkv or w_packed is NULL or not 16-byte aligned");
  const size_t need = lc::packed_qkv_weight_bytes(ctx->cfg.d_model, features(ctx));
  if (packed_bytes < need)
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "w_packed holds %zu bytes, %zu needed", packed_bytes, need);
  const hipError_t e = lc::launch_pack_qkv_weight(w_qkv, w_packed, ctx->cfg.d_model, features(ctx),
                                                  ctx->cfg.head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(ctx, "pack launch", e);
  return LACACHE_OK;
}

lacache_status lacache_read_device_status(lacache_ctx *ctx, void *stream, uint32_t *flags) {
  if (!ctx || !flags) return LACACHE_ERR_INVALID_ARG;
  lacache_status st;
  if ((st = check_device(ctx)) != LACACHE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(flags, ctx->flags, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(ctx->flags, 0, sizeof(uint32_t));
  if (e != hipSuccess) return hip_fail(ctx, "read device status", e);
  return LACACHE_OK;
}

lacache_status lacache_profile_enable(lacache_ctx *ctx, int enable) {
  if (!ctx) return LACACHE_ERR_INVALID_ARG;
  ctx->profiling = enable != 0;
  return LACACHE_OK;
}

lacache_status lacache_profile_read(lacache_ctx *ctx, int32_t kernel, double *total_ms, int64_t *launches) {
  if (!ctx || !total_ms || !launches) return LACACHE_ERR_INVALID_ARG;
  if (kernel < 0 || kernel >= LACACHE_KERNEL_COUNT)
    return fail(ctx, LACACHE_ERR_INVALID_ARG, "unknown kernel class %d", kernel);
  for (auto &mk : ctx->marks) {
    hipError_t e = hipEventSynchronize(mk.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, mk.start, mk.stop);
    if (e != hipSuccess) return hip_fail(ctx, "profile events", e);
    ctx->prof_ms[mk.kernel] += ms;
    ctx->prof_n[mk.kernel] += 1;
    ctx->free_events.push_back(mk.start);
    ctx->free_events.push_back(mk.stop);
  }
  ctx->marks.clear();
  *total_ms = ctx->prof_ms[kernel];
  *launches = ctx->prof_n[kernel];
  ctx->prof_ms[kernel] = 0;
  ctx->prof_n[kernel] = 0;
  return LACACHE_OK;
}

}  // extern "C"
