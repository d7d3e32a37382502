// Flash-dLLM's selective cache update and two-view verify (the Flash-dLLM
// article: the third element of "Flash-Cache", and "Flash-Verify"), on the
// RoPECache (fp16 q, k, v rows [rows, heads, d_h]).
//
// * Attention importance: importance_j = sum_h sum_i exp(scale q_ih . k_jh -
//   lse_ih) over the current block's queries i of the sample (lse: the block
//   rows' log-sum-exp from their attention), i.e. the softmax weight key row j
//   receives.  One wave per 16 keys and head: MFMA 16x16x32 f16 of the key
//   rows against the query rows, per-head partial sums [rows][heads] (no
//   atomics; the heads are added in order by the selection kernel).
// * Tracking set: per sample, the `budget` rows outside the block of largest
//   importance (the lower row on ties), in row order.
// * Verify attention: verify queries (tracking, draft view, mask view) over
//   the sample's cached rows other than the positions they carry, then their
//   own keys: a key of view 0 (tracking) is seen by every query, a key of view
//   1 or 2 only by queries of the same view.  Flash attention per 16 queries
//   and head, 32 keys per step, fp32 online softmax, the key tiles split over
//   4 waves and merged.
// * Acceptance: per sample, the longest prefix of the search positions whose
//   draft and mask-view tokens agree with mask-view confidence above gamma;
//   the accepted draft tokens are written into the ids.

#include "internal.h"

namespace lc {

namespace {
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ h8_t ld_h8(const f16_t *p) { return *reinterpret_cast<const h8_t *>(p); }
__device__ __forceinline__ f32x4_t mfma_h(const h8_t &a, const h8_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float sum16(float x) {                 // over the 16 lanes of a lane group
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x + __shfl_xor(x, 8);
}
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 4));
  return fmaxf(x, __shfl_xor(x, 8));
}
}  // namespace

// ---------------------------------------------------------------------------
// Importance partials: grid (key-tile items, heads); item t of sample b covers
// keys 64 (t - pre[1][b]) .. +63 of the sample, 16 per wave.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void importance_kernel(const SeqArgs sa, const TrackArgs a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int item = blockIdx.x, h = blockIdx.y;
  const int b = find_sample(sa.pre[1], sa.n, item);
  const int N = sa.len[b], off = sa.off[b], bs = sa.bs[b], B = sa.be[b] - sa.bs[b];
  const int key0 = (item - sa.pre[1][b]) * 64 + w * 16;
  if (key0 >= N) return;                                           // whole wave
  const int kvh = h * a.Hkv / a.H, r16 = lane & 15, g = lane >> 4;
  const f16_t *k = static_cast<const f16_t *>(a.k);
  const f16_t *q = static_cast<const f16_t *>(a.q);
  h8_t kf[DH / 32];
  const int kr = min(key0 + r16, N - 1);
#pragma unroll
  for (int ks = 0; ks < DH / 32; ++ks) kf[ks] = ld_h8(k + ((size_t)(off + kr) * a.Hkv + kvh) * DH + ks * 32 + g * 8);
  float imp[4] = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < B; q0 += 16) {
    const int qi = min(q0 + r16, B - 1);                           // the lane's query column (clamped)
    const size_t qrow = (size_t)(off + bs + qi);
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) s = mfma_h(kf[ks], ld_h8(q + (qrow * a.H + h) * DH + ks * 32 + g * 8), s);
    // C layout: lane l holds keys 4 (l / 16) + v against query l % 16.
    const int qc = q0 + r16;
    const float l2 = qc < B ? a.lse[(size_t)(off + bs + qc) * a.H + h] * kLog2e : 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) imp[v] += qc < B ? fast_exp2(s[v] * a.scale_log2 - l2) : 0.f;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) imp[v] = sum16(imp[v]);
  if (r16 == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int key = key0 + 4 * g + v;
      if (key < N) a.partial[(size_t)(off + key) * a.H + h] = imp[v];
    }
  }
}

// ---------------------------------------------------------------------------
// Tracking set: one workgroup per sample (N <= kTrackMaxKeys).  Each row's
// importance is the sum of its heads' partials (in head order); rows outside
// the block are ranked by d = ~bits(max(importance, 0)), which orders larger
// importance first (the bits of a non-negative float order like its value).
// A radix select finds T, the K-th smallest d over those rows (K = budget,
// or fewer rows), in three passes over 11, 11 and 10 bits: each pass counts
// the rows that match the bits found so far into buckets of the next bits
// (LDS atomics) and picks the bucket where the count crosses what remains.
// Rows with d < T are all in the set; of the rows with d = T, the lowest
// rows fill it (a pass in row order, only when they are more than needed).
// One wave then writes the set in row order (-1 where fewer than budget).
// ---------------------------------------------------------------------------
constexpr int kSelBuckets = 2048;

// Exclusive prefix over the 256 threads of v; the total in *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *s_w, uint32_t *total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    before += k < w ? s_w[k] : 0u;
    all += s_w[k];
  }
  __syncthreads();                                            // s_w is reused by the next scan
  *total = all;
  return before + x - v;
}

__global__ __launch_bounds__(256) void track_select_kernel(const SeqArgs sa, const TrackArgs a) {
  extern __shared__ __align__(16) char smem[];
  uint32_t *s_d = reinterpret_cast<uint32_t *>(smem);          // [N] d of every row
  __shared__ uint32_t s_hist[kSelBuckets];
  __shared__ uint32_t s_w[4];
  __shared__ uint32_t s_pick[2];                               // bucket, rows before it
  __shared__ uint32_t s_n, s_eq;
  __shared__ int s_sel[64];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int N = sa.len[b], off = sa.off[b], bs = sa.bs[b], be = sa.be[b];
  const int K = min(a.budget, N - (be - bs));                  // rows the set holds
  for (int j = tid; j < N; j += 256) {
    // The row's heads are contiguous: all loaded at once (up to 64 heads, a
    // multiple of 4), then added in head order.
    const float *pr = a.partial + (size_t)(off + j) * a.H;
    float v = 0.f;
    if ((a.H & 3) == 0 && a.H <= 64) {
      float4 x[16];
#pragma unroll
      for (int c = 0; c < 16; ++c)
        if (4 * c < a.H) x[c] = *reinterpret_cast<const float4 *>(pr + 4 * c);
#pragma unroll
      for (int c = 0; c < 16; ++c)
        if (4 * c < a.H) v = (((v + x[c].x) + x[c].y) + x[c].z) + x[c].w;
    } else {
      for (int h = 0; h < a.H; ++h) v += pr[h];
    }
    a.importance[off + j] = v;
    s_d[j] = ~__float_as_uint(fmaxf(v, 0.f));
  }
  uint32_t prefix = 0, mask = 0, need = (uint32_t)max(K, 0);
  if (K > 0) {
    // Three passes: bits 31..21, 20..10, 9..0 of d.
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t nb = pass == 2 ? 1024u : 2048u;
      for (int k = tid; k < kSelBuckets; k += 256) s_hist[k] = 0u;
      __syncthreads();                                         // also publishes s_d (first pass)
      for (int j = tid; j < N; j += 256) {
        if (j >= bs && j < be) continue;
        const uint32_t d = s_d[j];
        if ((d & mask) == prefix) atomicAdd(&s_hist[(d >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      // Thread t owns buckets 8t .. 8t + 7; the bucket where the ascending
      // count reaches `need` is found by the thread whose range holds it.
      uint32_t c[8], sum = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        c[q] = s_hist[8 * tid + q];
        sum += c[q];
      }
      uint32_t total;
      uint32_t before = block_exclusive_scan(sum, s_w, &total);
      if (before < need && need <= before + sum) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (need <= before + c[q]) {
            s_pick[0] = 8 * tid + q;
            s_pick[1] = before;
            break;
          }
          before += c[q];
        }
      }
      __syncthreads();
      prefix |= s_pick[0] << sh;
      mask |= (nb - 1) << sh;
      need -= s_pick[1];
      __syncthreads();                                         // s_pick is rewritten by the next pass
    }
    // prefix = T; `need` rows with d = T complete the set.
    if (tid == 0) {
      s_n = 0u;
      s_eq = 0u;
    }
    __syncthreads();
    for (int j = tid; j < N; j += 256) {
      if (j >= bs && j < be) continue;
      const uint32_t d = s_d[j];
      if (d < prefix) s_sel[atomicAdd(&s_n, 1u)] = j;
      else if (d == prefix) atomicAdd(&s_eq, 1u);
    }
    __syncthreads();
    const uint32_t n_less = s_n, n_eq = s_eq;
    if (n_eq == need) {                                        // every tie is in the set
      for (int j = tid; j < N; j += 256)
        if (!(j >= bs && j < be) && s_d[j] == prefix) s_sel[atomicAdd(&s_n, 1u)] = j;
    } else {
      // The lowest `need` rows with d = T: 256 rows at a time in row order.
      uint32_t taken = 0;
      for (int j0 = 0; j0 < N && taken < need; j0 += 256) {
        const int j = j0 + tid;
        const uint32_t f = j < N && !(j >= bs && j < be) && s_d[j] == prefix ? 1u : 0u;
        uint32_t cnt;
        const uint32_t pos = block_exclusive_scan(f, s_w, &cnt);
        if (f && taken + pos < need) s_sel[n_less + taken + pos] = j;
        taken += cnt;
      }
    }
    __syncthreads();
  }
  // The set in row order (-1 where fewer rows than budget).
  if (tid < 64) {
    const int me = tid < K ? s_sel[tid] : 0x7fffffff;
    int rank = 0;
    for (int q = 0; q < K; ++q) {
      const int o = __shfl(me, q);
      rank += o < me;
    }
    if (tid < a.budget) {
      const size_t base = (size_t)(a.sample_base + b) * a.budget;
      if (tid < K) a.tracked[base + rank] = me;
      else a.tracked[base + tid] = -1;
    }
  }
}

// ---------------------------------------------------------------------------
// Verify attention: one workgroup of NW waves per (16 verify queries, head);
// grid (query-tile items, heads).  Keys in tiles of 32 (the sample's context
// rows, then the verify tokens' own), wave w taking tiles w, w + NW, ..., the
// next one loaded while the current one is used; the waves' states (max,
// normaliser, unnormalised O) are merged in LDS at the end by every thread.
// Eight waves (each with three or four of llada8b's 27 tiles): 23.3 us,
// against 28.5 us with four and 40.7 us with sixteen (LDS for one
// workgroup per CU).
// ---------------------------------------------------------------------------
template <int DH, int NW>
__global__ __launch_bounds__(64 * NW) void verify_attn_kernel(const SeqArgs sa, const VerifyArgs a) {
  __shared__ uint32_t s_carried[kVerifyMaxKeys / 32];
  __shared__ __align__(16) f16_t s_p[NW][16 * 32];               // per wave: P [16 queries][32 keys]
  constexpr int VS = DH + 8;                                     // staged V row (halves): conflict-free 16-byte writes
  __shared__ __align__(16) f16_t s_vt[NW][32 * VS];              // per wave: V [32 keys][DH (+8)]
  static_assert(sizeof(f16_t) * 32 * VS >= sizeof(float) * 16 * DH, "a wave's V area holds its O for the merge");
  __shared__ float s_m[NW][16], s_l[NW][16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int item = blockIdx.x, h = blockIdx.y;
  const int b = find_sample(sa.pre[1], sa.n, item);
  const int N = sa.len[b], off = sa.off[b];
  const int v0 = sa.pre[0][b], Q = sa.pre[0][b + 1] - v0;        // this sample's verify tokens
  const int kvh = h * a.Hkv / a.H, r16 = lane & 15, g = lane >> 4;
  // Positions the verify tokens carry are not context.
  for (int j = tid; j < (N + 31) / 32; j += 64 * NW) s_carried[j] = 0u;
  __syncthreads();
  for (int j = tid; j < Q; j += 64 * NW) {
    const int p = a.pos[v0 + j];
    if (p >= 0 && p < N) atomicOr(&s_carried[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  f16_t *P = s_p[w];
  f16_t *VT = s_vt[w];
  const int qt0 = (item - sa.pre[1][b]) * 16;                    // the wave's first query (within the sample)
  const f16_t *qv = static_cast<const f16_t *>(a.q);
  const f16_t *kc = static_cast<const f16_t *>(a.k), *vc = static_cast<const f16_t *>(a.v);
  const f16_t *kv = static_cast<const f16_t *>(a.k_ver), *vv = static_cast<const f16_t *>(a.v_ver);
  h8_t qf[DH / 32];
  const int qa = min(qt0 + r16, Q - 1);                          // A operand: query row l % 16
#pragma unroll
  for (int ks = 0; ks < DH / 32; ++ks) qf[ks] = ld_h8(qv + ((size_t)(v0 + qa) * a.H + h) * DH + ks * 32 + g * 8);
  // C layout rows: queries qt0 + 4 g + v; their views.
  int qview[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) qview[v] = a.view[v0 + min(qt0 + 4 * g + v, Q - 1)];
  float m[4], l[4];
  f32x4_t o[DH / 16];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    m[v] = -INFINITY;
    l[v] = 0.f;
  }
#pragma unroll
  for (int f = 0; f < DH / 16; ++f) o[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nctx = (N + 31) / 32, nkt = nctx + (Q + 31) / 32;   // context tiles, then the verify keys
  // Tile t's K operands (key l % 16 of each 16-key half) and V pieces (piece
  // c * 64 + l: key e / (DH / 8), features 8 (e % (DH / 8)) ..).
  h8_t kf[2][DH / 32], vp[DH / 16];
  auto load = [&](int t) {
    const bool ctx = t < nctx;
    const int j0 = (ctx ? t : t - nctx) * 32, lim = ctx ? N : Q;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int j = min(j0 + 16 * half + r16, lim - 1);
      const f16_t *kp = ctx ? kc + ((size_t)(off + j) * a.Hkv + kvh) * DH : kv + ((size_t)(v0 + j) * a.Hkv + kvh) * DH;
#pragma unroll
      for (int ks = 0; ks < DH / 32; ++ks) kf[half][ks] = ld_h8(kp + ks * 32 + g * 8);
    }
#pragma unroll
    for (int c = 0; c < DH / 16; ++c) {
      const int e = c * 64 + lane, key = e / (DH / 8), f0 = 8 * (e % (DH / 8));
      const int j = min(j0 + key, lim - 1);
      const f16_t *vpp = ctx ? vc + ((size_t)(off + j) * a.Hkv + kvh) * DH : vv + ((size_t)(v0 + j) * a.Hkv + kvh) * DH;
      vp[c] = ld_h8(vpp + f0);
    }
  };
  if (w < nkt) load(w);
  for (int t = w; t < nkt; t += NW) {
    const bool ctx = t < nctx;
    const int j0 = (ctx ? t : t - nctx) * 32, lim = ctx ? N : Q;
    // Scores of the 16 queries against keys j0 .. j0 + 31 (two 16-key halves).
    f32x4_t s[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      s[half] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DH / 32; ++ks) s[half] = mfma_h(qf[ks], kf[half][ks], s[half]);
    }
    // V of the tile into LDS, then the next tile's loads go out.
#pragma unroll
    for (int c = 0; c < DH / 16; ++c) {
      const int e = c * 64 + lane, key = e / (DH / 8), f0 = 8 * (e % (DH / 8));
      *reinterpret_cast<h8_t *>(VT + key * VS + f0) = vp[c];
    }
    if (t + NW < nkt) load(t + NW);
    // Visibility of key column l % 16 (+16) for the lane's 4 query rows.
    float tmax[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) tmax[v] = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int j = j0 + 16 * half + r16;
      bool base_ok = j < lim;
      int kview = 0;
      if (ctx) base_ok = base_ok && !((s_carried[min(j, N - 1) >> 5] >> (j & 31)) & 1u);
      else if (base_ok) kview = a.view[v0 + j];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool ok = base_ok && (ctx || kview == 0 || kview == qview[v]);
        s[half][v] = ok ? s[half][v] * a.scale_log2 : -INFINITY;
        tmax[v] = fmaxf(tmax[v], s[half][v]);
      }
    }
    float alpha[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float mn = fmaxf(m[v], max16(tmax[v]));
      alpha[v] = mn == -INFINITY ? 1.f : fast_exp2(m[v] - mn);
      m[v] = mn;
      float ps = 0.f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float p = s[half][v] == -INFINITY ? 0.f : fast_exp2(s[half][v] - mn);
        ps += p;
        P[(4 * g + v) * 32 + 16 * half + r16] = (f16_t)p;
      }
      l[v] = l[v] * alpha[v] + sum16(ps);
    }
    wave_lds_sync();
    // O = O alpha + P V: A = P rows (query l % 16, keys 8 (l / 16) ..), B =
    // column 16 f + l % 16 of V over the same 8 keys.
    const h8_t pa = *reinterpret_cast<const h8_t *>(P + r16 * 32 + 8 * g);
#pragma unroll
    for (int f = 0; f < DH / 16; ++f) {
      h8_t vb;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) vb[kk] = VT[(8 * g + kk) * VS + 16 * f + r16];
#pragma unroll
      for (int v = 0; v < 4; ++v) o[f][v] *= alpha[v];
      o[f] = mfma_h(pa, vb, o[f]);
    }
    wave_lds_sync();
  }
  // Merge of the NW waves' states (the V areas reused for the unnormalised O).
  __syncthreads();
  float *so = reinterpret_cast<float *>(&s_vt[0][0]);            // [NW waves][16 rows][DH]
#pragma unroll
  for (int f = 0; f < DH / 16; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) so[(w * 16 + 4 * g + v) * DH + 16 * f + r16] = o[f][v];
  if (r16 == 0)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      s_m[w][4 * g + v] = m[v];
      s_l[w][4 * g + v] = l[v];
    }
  __syncthreads();
  for (int e = tid; e < 16 * DH; e += 64 * NW) {
    const int row = e / DH, qi = qt0 + row;
    if (qi >= Q) continue;
    float M = s_m[0][row];
#pragma unroll
    for (int k = 1; k < NW; ++k) M = fmaxf(M, s_m[k][row]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float c = s_m[k][row] == -INFINITY ? 0.f : fast_exp2(s_m[k][row] - M);
      num += c * so[(k * 16 + row) * DH + (e % DH)];
      den += c * s_l[k][row];
    }
    static_cast<bf16_t *>(a.out)[((size_t)(v0 + qi) * a.H + h) * DH + (e % DH)] = f2bf(num / den);
    if (a.lse && e % DH == 0) a.lse[(size_t)(v0 + qi) * a.H + h] = (M + __log2f(den)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Acceptance: one wave per sample (at most 64 search positions).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void verify_accept_kernel(const SeqArgs sa, const AcceptArgs a) {
  const int lane = threadIdx.x, b = blockIdx.x;
  const int s0 = sa.pre[0][b], S = sa.pre[0][b + 1] - s0;
  bool ok = false, order_ok = true;
  int p = 0;
  if (lane < S) {
    p = a.pos[s0 + lane];
    ok = a.draft[s0 + lane] == a.mask_tok[s0 + lane] && a.mask_conf[s0 + lane] > a.gamma;
    order_ok = p >= 0 && p < sa.len[b] && (lane == 0 || a.pos[s0 + lane - 1] < p);
  }
  const unsigned long long good = __ballot(ok), bad_order = __ballot(!order_ok);
  const unsigned long long inside = S >= 64 ? ~0ull : ((1ull << S) - 1ull), gi = good & inside;
  const int n = gi == inside ? S : (int)__builtin_ctzll(~gi);        // first failing lane, or S
  if (bad_order) {
    if (lane == 0) {
      atomicOr(a.flags, 4u);
      a.n_accepted[b] = 0;
    }
    return;
  }
  if (lane == 0) a.n_accepted[b] = n;
  if (lane < n) a.ids[sa.off[b] + p] = a.draft[s0 + lane];
}

// ---------------------------------------------------------------------------
hipError_t launch_importance(int dh, const SeqArgs &sa, const TrackArgs &a, hipStream_t s, const LaunchEvents &ev) {
  const int items = sa.pre[1][sa.n];
  if (items <= 0) return hipSuccess;
  const dim3 grid(items, a.H);
  if (dh == 128) lc_launch<importance_kernel<128>>(grid, dim3(256), 0, s, ev, sa, a);
  else if (dh == 64) lc_launch<importance_kernel<64>>(grid, dim3(256), 0, s, ev, sa, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_track_select(const SeqArgs &sa, const TrackArgs &a, int max_len, hipStream_t s,
                               const LaunchEvents &ev) {
  if (sa.n <= 0) return hipSuccess;
  if (max_len > kTrackMaxKeys || a.budget > 64 || a.budget < 1) return hipErrorInvalidValue;
  lc_launch<track_select_kernel>(dim3(sa.n), dim3(256), (unsigned)(max_len * sizeof(uint32_t)), s, ev, sa, a);
  return hipGetLastError();
}

hipError_t launch_verify_attn(int dh, const SeqArgs &sa, const VerifyArgs &a, hipStream_t s, const LaunchEvents &ev) {
  const int items = sa.pre[1][sa.n];
  if (items <= 0) return hipSuccess;
  const dim3 grid(items, a.H);
  constexpr int nw = 8;
  if (dh == 128) lc_launch<verify_attn_kernel<128, nw>>(grid, dim3(64 * nw), 0, s, ev, sa, a);
  else if (dh == 64) lc_launch<verify_attn_kernel<64, nw>>(grid, dim3(64 * nw), 0, s, ev, sa, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_verify_accept(const SeqArgs &sa, const AcceptArgs &a, hipStream_t s, const LaunchEvents &ev) {
  if (sa.n <= 0) return hipSuccess;
  lc_launch<verify_accept_kernel>(dim3(sa.n), dim3(64), 0, s, ev, sa, a);
  return hipGetLastError();
}

hipError_t setup_flashdllm_attributes() {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(track_select_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kTrackMaxKeys * (int)sizeof(uint32_t));
}

}  // namespace lc
