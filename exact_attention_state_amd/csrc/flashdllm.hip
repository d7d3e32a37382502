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
// Tracking set: one workgroup per sample (N <= kTrackMaxKeys).  Every row
// gets a 64-bit key that orders block rows last, then larger importance
// first, then the lower row; a bitonic sort in LDS orders the keys and the
// first `budget` name the tracking set, which one wave puts in row order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void track_select_kernel(const SeqArgs sa, const TrackArgs a) {
  extern __shared__ __align__(16) char smem[];
  unsigned long long *key = reinterpret_cast<unsigned long long *>(smem);   // [NP]
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int N = sa.len[b], off = sa.off[b], bs = sa.bs[b], be = sa.be[b];
  int NP = 1;
  while (NP < N) NP <<= 1;
  for (int j = tid; j < NP; j += 256) {
    unsigned long long k = ~0ull;                                // padding: after every row
    if (j < N) {
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
      // Bit 63: a block row (last); bits 62..31: the complement of the
      // importance's bits (importance >= 0 orders like its bits, so larger
      // first); bits 30..0: the row.
      const bool excl = j >= bs && j < be;
      const uint32_t desc = ~__float_as_uint(fmaxf(v, 0.f));
      k = ((unsigned long long)excl << 63) | ((unsigned long long)desc << 31) | (uint32_t)j;
    }
    key[j] = k;
  }
  __syncthreads();
  // Pair i of a stage is (lo, lo + stride), lo = 2 i - i % stride; thread t
  // takes pairs t, t + 256, ...  At strides up to 64 the 64 pairs of a wave lie
  // in 128 elements no other wave touches, so the wave's own ordering suffices
  // there; a workgroup barrier separates the stages at larger strides.
  for (int size = 2; size <= NP; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < NP / 2; i += 256) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned long long x = key[lo], y = key[hi];
        if ((x > y) == up) {
          key[lo] = y;
          key[hi] = x;
        }
      }
      const int next = stride > 1 ? stride >> 1 : size;            // the next stage's stride
      if (stride > 64 || (next > 64 && 2 * size <= NP)) __syncthreads();
      else wave_lds_sync();
    }
  __syncthreads();
  // The first `budget` keys, put in row order (block rows and padding: -1, last).
  if (tid < 64) {
    int me = 0x7fffffff;
    if (tid < a.budget && tid < N) {
      const unsigned long long k = key[tid];
      if (!(k >> 63)) me = (int)(uint32_t)(k & 0x7fffffffu);
    }
    int rank = 0;
    for (int j = 0; j < a.budget; ++j) {
      const int o = __shfl(me, j);
      rank += (o < me) || (o == me && j < tid);
    }
    if (tid < a.budget) a.tracked[(size_t)(a.sample_base + b) * a.budget + rank] = me == 0x7fffffff ? -1 : me;
  }
}

// ---------------------------------------------------------------------------
// Verify attention: one workgroup of 4 waves per (16 verify queries, head);
// grid (query-tile items, heads).  Keys in tiles of 32 (the sample's context
// rows, then the verify tokens' own), wave w taking tiles w, w + 4, ..., the
// next one loaded while the current one is used; the 4 waves' states
// (max, normaliser, unnormalised O) are merged in LDS at the end.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void verify_attn_kernel(const SeqArgs sa, const VerifyArgs a) {
  __shared__ uint32_t s_carried[kVerifyMaxKeys / 32];
  __shared__ __align__(16) f16_t s_p[4][16 * 32];                // per wave: P [16 queries][32 keys]
  constexpr int VS = DH + 8;                                     // staged V row (halves): conflict-free 16-byte writes
  __shared__ __align__(16) f16_t s_vt[4][32 * VS];               // per wave: V [32 keys][DH (+8)]
  __shared__ float s_m[4][16], s_l[4][16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int item = blockIdx.x, h = blockIdx.y;
  const int b = find_sample(sa.pre[1], sa.n, item);
  const int N = sa.len[b], off = sa.off[b];
  const int v0 = sa.pre[0][b], Q = sa.pre[0][b + 1] - v0;        // this sample's verify tokens
  const int kvh = h * a.Hkv / a.H, r16 = lane & 15, g = lane >> 4;
  // Positions the verify tokens carry are not context.
  for (int j = tid; j < (N + 31) / 32; j += 256) s_carried[j] = 0u;
  __syncthreads();
  for (int j = tid; j < Q; j += 256) {
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
  for (int t = w; t < nkt; t += 4) {
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
    if (t + 4 < nkt) load(t + 4);
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
  // Merge of the 4 waves' states (the V areas reused for the unnormalised O).
  __syncthreads();
  float *so = reinterpret_cast<float *>(&s_vt[0][0]);            // [4 waves][16 rows][DH]
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
  if (w != 0) return;
  for (int e = lane; e < 16 * DH; e += 64) {
    const int row = e / DH, qi = qt0 + row;
    if (qi >= Q) continue;
    float M = s_m[0][row];
#pragma unroll
    for (int k = 1; k < 4; ++k) M = fmaxf(M, s_m[k][row]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
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
  int np = 1;
  while (np < max_len) np <<= 1;
  lc_launch<track_select_kernel>(dim3(sa.n), dim3(256), (unsigned)(np * sizeof(unsigned long long)), s, ev, sa, a);
  return hipGetLastError();
}

hipError_t launch_verify_attn(int dh, const SeqArgs &sa, const VerifyArgs &a, hipStream_t s, const LaunchEvents &ev) {
  const int items = sa.pre[1][sa.n];
  if (items <= 0) return hipSuccess;
  const dim3 grid(items, a.H);
  if (dh == 128) lc_launch<verify_attn_kernel<128>>(grid, dim3(256), 0, s, ev, sa, a);
  else if (dh == 64) lc_launch<verify_attn_kernel<64>>(grid, dim3(256), 0, s, ev, sa, a);
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
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             kTrackMaxKeys * (int)sizeof(unsigned long long));
}

}  // namespace lc
