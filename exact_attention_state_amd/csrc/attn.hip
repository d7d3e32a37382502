// First-layer attention kernels of the cached block step (LaCache Section
// 3.3.3, Eqs. (2)-(6); Algorithm 1) and of the block-boundary refresh.
//
// All of them share one 32-key step on MFMA (attend_step):
//   S^T = K Q^T       A = 16 keys x 32 head-dim slots, B = Q^T; the key rows
//                     of a block are loaded in an order that leaves lane group
//                     g holding keys 8g..8g+7 of the step in the result.
//   online softmax    per query row (lane%16), max shared by the 4 lane
//                     groups, scores in log2 units so exp is v_exp_f32.
//   O^T += V^T P^T    A = V^T read from LDS (V is transposed while staged),
//                     B = P^T straight from the softmax registers; the result
//                     keeps each query row in one lane, so the per-row rescale
//                     is lane-local.
// K fragments are read straight from HBM (16 or 32 contiguous bytes per lane,
// full 128-byte lines per instruction); only V goes through LDS.
//
// Work items (one workgroup of 4 waves each, times the head count):
//   type A  block rows (<= 32) of one sample against one chunk of its keys
//           [prefix | fresh block | suffix]; the 4 waves take alternate 32-key
//           steps and merge their states in LDS; the chunk's (m, l, O~) goes to
//           the workspace (split-KV).  This is also the DualCache step.
//   type B  64 invariant rows of one sample: the state starts from FACache and
//           streams only the block's keys, then O = O~/l and LSE = m + ln l.
//   merge   combines the type-A chunks of every block row into O and LSE.
//   refresh 64 rows of one sample against every key: invariant keys first,
//           a snapshot of (m, l, O~) into FACache for invariant rows, then the
//           block's keys, then O and LSE.

#include "internal.h"

namespace lc {

template <typename T> struct VtPad { static constexpr int v = 8; };
template <> struct VtPad<float> { static constexpr int v = 4; };

template <int MB, int DH> struct AttnState {
  float m[MB];                 // running max, log2 units (same in the 4 lane groups)
  float l[MB];                 // this lane's share of the normaliser
  f32x4_t o[MB][DH / 16];      // O~ of row lane%16, features 16*db + 4*g + i
};

template <int MB, int DH> __device__ __forceinline__ void state_init_empty(AttnState<MB, DH> &st) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    st.m[mb] = -INFINITY;
    st.l[mb] = 0.f;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) st.o[mb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Load 16 consecutive elements as two fragments (32 or 64 contiguous bytes).
template <typename T>
__device__ __forceinline__ void frag_load2(Frag<T> &f0, Frag<T> &f1, const T *p) {
  frag_load(f0, p);
  frag_load(f1, p + 8);
}

// Query fragments of one row (lane%16 of each row block): head-dim slot
// mapping shared with the key fragments: step kd = 2p + half covers features
// 64p + 16g + 8*half + (0..7).
template <typename T, int MB, int DH>
__device__ __forceinline__ void load_q(Frag<T> (&qf)[MB][DH / 32], const T *const (&qrow)[MB],
                                       const bool (&qvalid)[MB], int g) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int p = 0; p < DH / 64; ++p) {
      if (qvalid[mb]) {
        frag_load2(qf[mb][2 * p], qf[mb][2 * p + 1], qrow[mb] + 64 * p + 16 * g);
      } else {
        frag_zero(qf[mb][2 * p]);
        frag_zero(qf[mb][2 * p + 1]);
      }
    }
}

// One step of up to 32 keys.  kbase points at key 0 of the step (head offset
// applied), kstride = elements between consecutive keys.  vt = LDS V^T of the
// step: vt[d * vts + c] for key c.  Keys c >= nvalid are masked; their V^T
// entries must be finite (the stager writes zeros).
template <typename T, int MB, int DH>
__device__ __forceinline__ void attend_step(AttnState<MB, DH> &st, const Frag<T> (&qf)[MB][DH / 32],
                                            const T *kbase, size_t kstride, int nvalid, const T *vt,
                                            int vts, float scale_log2, int lane) {
  const int g = lane >> 4, r16 = lane & 15;
  f32x4_t s[2][MB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = 8 * (r16 >> 2) + 4 * kb + (r16 & 3);
    const bool kv = key < nvalid;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) s[kb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < DH / 64; ++p) {
      Frag<T> k0, k1;
      if (kv) {
        frag_load2(k0, k1, kbase + (size_t)key * kstride + 64 * p + 16 * g);
      } else {
        frag_zero(k0);
        frag_zero(k1);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        mma16(s[kb][mb], k0, qf[mb][2 * p]);
        mma16(s[kb][mb], k1, qf[mb][2 * p + 1]);
      }
    }
  }
  Frag<T> pf[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = (8 * g + j < nvalid) ? s[j >> 2][mb][j & 3] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[j]);
    }
    mx = group_max(mx);
    const float mnew = fmaxf(st.m[mb], mx);
    const float alpha = fast_exp2(st.m[mb] - mnew);
    st.m[mb] = mnew;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = fast_exp2(x[j] - mnew);
      ps += p;
      frag_set(pf[mb], j, p);
    }
    st.l[mb] = fmaf(st.l[mb], alpha, ps);
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) st.o[mb][db] *= alpha;
  }
#pragma unroll
  for (int db = 0; db < DH / 16; ++db) {
    Frag<T> vf;
    frag_load(vf, vt + (16 * db + r16) * vts + 8 * g);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) mma16(st.o[mb][db], vf, pf[mb]);
  }
}

// Stage V^T for `ncols` keys starting at vbase (zeros for keys >= nvalid):
// vt[d * vts + c].  Threads [tid0, tid0 + nthr) cooperate; consecutive threads
// read consecutive 16/32-byte chunks of one key row.
template <typename T, int DH>
__device__ __forceinline__ void stage_vt(T *vt, int vts, const T *vbase, size_t vstride, int nvalid,
                                         int ncols, int t, int nthr) {
  constexpr int CH = DH / 8;
  for (int idx = t; idx < ncols * CH; idx += nthr) {
    const int c = idx / CH, ch = idx % CH;
    if constexpr (sizeof(T) == 2) {
      // Raw 16-bit halves of one 16-byte load (8 features of key c).
      uint4 u = make_uint4(0, 0, 0, 0);
      if (c < nvalid) u = *reinterpret_cast<const uint4 *>(vbase + (size_t)c * vstride + ch * 8);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        reinterpret_cast<uint16_t *>(vt)[(ch * 8 + j) * vts + c] = (uint16_t)((wd[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
    } else {
      Frag<T> f;
      if (c < nvalid) frag_load(f, vbase + (size_t)c * vstride + ch * 8); else frag_zero(f);
#pragma unroll
      for (int j = 0; j < 8; ++j) vt[(ch * 8 + j) * vts + c] = frag_get(f, j);
    }
  }
}

// ---------------------------------------------------------------------------
// Type A: block rows x key chunk -> partial state in the workspace.
// ---------------------------------------------------------------------------
template <typename T, typename TO, int DH>
__device__ void block_rows_partial(const SeqArgs &sa, const AttnArgs &a, int item, int h, char *smem) {
  constexpr int MB = kRowsA / 16;
  constexpr int VTS = 32 + VtPad<T>::v;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  const int b = find_sample(sa.pre[1], sa.n, item);
  const int t = item - sa.pre[1][b];
  const int B = sa.be[b] - sa.bs[b], N = sa.len[b];
  const int nrg = (B + kRowsA - 1) / kRowsA;
  const int chunk = t / nrg, rg = t % nrg;
  const int key0 = chunk * a.split_keys;
  const int nkeys = min(a.split_keys, N - key0);
  const int nsteps = (nkeys + 31) / 32;
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;

  const T *q = static_cast<const T *>(a.q);
  const T *qrow[MB];
  bool qvalid[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = rg * kRowsA + mb * 16 + r16;
    qvalid[mb] = r < B;
    const int row = a.qmode == 0 ? sa.off[b] + sa.bs[b] + r : a.row_base + sa.pre[0][b] + r;
    qrow[mb] = q + ((size_t)(qvalid[mb] ? row : 0) * a.H + h) * DH;
  }
  Frag<T> qf[MB][DH / 32];
  load_q<T, MB, DH>(qf, qrow, qvalid, g);

  AttnState<MB, DH> st;
  state_init_empty(st);
  T *vt = reinterpret_cast<T *>(smem) + w * (DH * VTS);
  const T *kbase0 = static_cast<const T *>(a.k) + ((size_t)(sa.off[b] + key0)) * kvstride + hk * DH;
  const T *vbase0 = static_cast<const T *>(a.v) + ((size_t)(sa.off[b] + key0)) * kvstride + hk * DH;
  const int niter = (nsteps + 3) / 4;
  for (int it = 0; it < niter; ++it) {
    const int step = it * 4 + w;
    const bool valid = step < nsteps;
    const int nvalid = valid ? min(32, nkeys - step * 32) : 0;
    __syncthreads();
    if (valid) stage_vt<T, DH>(vt, VTS, vbase0 + (size_t)step * 32 * kvstride, kvstride, nvalid, 32, lane, 64);
    __syncthreads();
    if (valid)
      attend_step<T, MB, DH>(st, qf, kbase0 + (size_t)step * 32 * kvstride, kvstride, nvalid, vt, VTS,
                             a.scale_log2, lane);
  }
  __syncthreads();

  // Merge the 4 waves' states of each row in LDS.
  float *s_m = reinterpret_cast<float *>(smem);              // [4][kRowsA]
  float *s_l = s_m + 4 * kRowsA;                             // [4][kRowsA]
  float *s_o = s_l + 4 * kRowsA;                             // [4][kRowsA][DH]
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rr = mb * 16 + r16;
    const float lt = group_sum(st.l[mb]);
    if (g == 0) {
      s_m[w * kRowsA + rr] = st.m[mb];
      s_l[w * kRowsA + rr] = lt;
    }
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[(w * kRowsA + rr) * DH + 16 * db + 4 * g + i] = st.o[mb][db][i];
  }
  __syncthreads();
  const int pbase = a.part_base + sa.pre[3][b] + chunk * B;
  for (int idx = tid; idx < kRowsA * DH; idx += blockDim.x) {
    const int rr = idx / DH, d = idx % DH;
    const int r = rg * kRowsA + rr;
    if (r >= B) continue;
    float mx = s_m[rr];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) mx = fmaxf(mx, s_m[ww * kRowsA + rr]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float e = fast_exp2(s_m[ww * kRowsA + rr] - mx);
      lsum = fmaf(e, s_l[ww * kRowsA + rr], lsum);
      osum = fmaf(e, s_o[(ww * kRowsA + rr) * DH + d], osum);
    }
    const size_t prow = (size_t)(pbase + r) * a.H + h;
    a.part_o[prow * DH + d] = osum;
    if (d == 0) a.part_ml[prow] = make_float2(mx, lsum);
  }
}

// ---------------------------------------------------------------------------
// Type B: 64 invariant rows, state from FACache, stream the block's keys.
// ---------------------------------------------------------------------------
template <typename T, typename TO, int DH>
__device__ void invariant_rows(const SeqArgs &sa, const AttnArgs &a, int item, int h, char *smem) {
  constexpr int MB = 1;
  constexpr int VTS = 128 + VtPad<T>::v;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  const int b = find_sample(sa.pre[2], sa.n, item);
  const int tile = item - sa.pre[2][b];
  const int bs = sa.bs[b], be = sa.be[b], B = be - bs, N = sa.len[b];
  const int nU = N - B;
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;
  const int off = sa.off[b];

  T *vt = reinterpret_cast<T *>(smem);
  stage_vt<T, DH>(vt, VTS, static_cast<const T *>(a.v) + (size_t)(off + bs) * kvstride + hk * DH, kvstride, B,
                  (B + 31) & ~31, tid, blockDim.x);

  const int u = tile * kRowsB + w * 16 + r16;
  const bool uvalid = u < nU;
  const int row = off + (u < bs ? u : u + B);
  const T *q = static_cast<const T *>(a.q);
  const T *qrow[MB] = {q + ((size_t)(uvalid ? row : off) * a.H + h) * DH};
  const bool qvalid[MB] = {uvalid};
  Frag<T> qf[MB][DH / 32];
  load_q<T, MB, DH>(qf, qrow, qvalid, g);

  // FACache state of this row (Algorithm 1: initialise with the cache).
  AttnState<MB, DH> st;
  const size_t crow = (size_t)(uvalid ? row : off) * a.H + h;
  if (uvalid) {
    st.m[0] = a.m_c[crow] * kLog2e;
    st.l[0] = g == 0 ? a.l_c[crow] : 0.f;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
      st.o[0][db] = *reinterpret_cast<const f32x4_t *>(a.o_c + crow * DH + 16 * db + 4 * g);
  } else {
    state_init_empty(st);
  }
  __syncthreads();

  const T *kbase = static_cast<const T *>(a.k) + (size_t)(off + bs) * kvstride + hk * DH;
  for (int c0 = 0; c0 < B; c0 += 32)
    attend_step<T, MB, DH>(st, qf, kbase + (size_t)c0 * kvstride, kvstride, min(32, B - c0), vt + c0, VTS,
                           a.scale_log2, lane);

  const float lt = group_sum(st.l[0]);
  if (uvalid) {
    const float inv = 1.0f / lt;
    TO *out = static_cast<TO *>(a.out) + crow * DH;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[16 * db + 4 * g + i] = from_f32<TO>(st.o[0][db][i] * inv);
    if (a.lse && g == 0) a.lse[crow] = (st.m[0] + __log2f(lt)) * kLn2;
  }
}

template <typename T, typename TO, int DH>
__global__ __launch_bounds__(256) void step_attn_kernel(const SeqArgs sa, const AttnArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int gid = blockIdx.x;
  if (gid < a.nA) {
    block_rows_partial<T, TO, DH>(sa, a, gid / a.H, gid % a.H, smem);
  } else {
    const int j = gid - a.nA;
    invariant_rows<T, TO, DH>(sa, a, j / a.H, j % a.H, smem);
  }
}

// Only type-A items: the DualCache block-query attention.
template <typename T, typename TO, int DH>
__global__ __launch_bounds__(256) void block_attn_kernel(const SeqArgs sa, const AttnArgs a) {
  extern __shared__ __align__(16) char smem[];
  block_rows_partial<T, TO, DH>(sa, a, blockIdx.x / a.H, blockIdx.x % a.H, smem);
}

// ---------------------------------------------------------------------------
// Merge of the type-A partial states: one wave per (block row, head).
// ---------------------------------------------------------------------------
template <typename T, typename TO, int DH>
__global__ __launch_bounds__(256) void merge_kernel(const SeqArgs sa, const AttnArgs a, int M) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= M * a.H) return;
  const int m = wid / a.H, h = wid % a.H;
  const int b = find_sample(sa.pre[0], sa.n, m);
  const int r = m - sa.pre[0][b];
  const int B = sa.be[b] - sa.bs[b];
  const int nch = (sa.len[b] + a.split_keys - 1) / a.split_keys;
  const int pbase = a.part_base + sa.pre[3][b];

  float mx = -INFINITY;
  for (int c = lane; c < nch; c += 64) mx = fmaxf(mx, a.part_ml[(size_t)(pbase + c * B + r) * a.H + h].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float lsum = 0.f;
  float acc[DH / 64] = {};
  for (int c = 0; c < nch; ++c) {
    const size_t prow = (size_t)(pbase + c * B + r) * a.H + h;
    const float2 ml = a.part_ml[prow];
    const float e = fast_exp2(ml.x - mx);
    lsum = fmaf(e, ml.y, lsum);
#pragma unroll
    for (int j = 0; j < DH / 64; ++j) acc[j] = fmaf(e, a.part_o[prow * DH + lane + 64 * j], acc[j]);
  }
  const int orow = a.omode == 0 ? sa.off[b] + sa.bs[b] + r : a.row_base + m;
  const float inv = 1.0f / lsum;
  TO *out = static_cast<TO *>(a.out) + ((size_t)orow * a.H + h) * DH;
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) out[lane + 64 * j] = from_f32<TO>(acc[j] * inv);
  if (a.lse && lane == 0) a.lse[(size_t)orow * a.H + h] = (mx + __log2f(lsum)) * kLn2;
}

// ---------------------------------------------------------------------------
// Refresh: 64 rows of one sample over all keys, invariant keys first, with a
// snapshot of the invariant rows' state into FACache before the block keys.
// ---------------------------------------------------------------------------
template <typename T, typename TO, int DH>
__global__ __launch_bounds__(256) void refresh_attn_kernel(const SeqArgs sa, const AttnArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int MB = 1;
  constexpr int TK = 128;                     // keys staged per tile
  constexpr int VTS = TK + VtPad<T>::v;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int item = blockIdx.x / a.H, h = blockIdx.x % a.H;

  const int b = find_sample(sa.pre[1], sa.n, item);
  const int tile = item - sa.pre[1][b];
  const int bs = sa.bs[b], be = sa.be[b], N = sa.len[b];
  const int off = sa.off[b];
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;

  const int t = tile * kRowsR + w * 16 + r16;
  const bool tvalid = t < N;
  const bool in_u = tvalid && (t < bs || t >= be);
  const T *q = static_cast<const T *>(a.q);
  const T *qrow[MB] = {q + ((size_t)(off + (tvalid ? t : 0)) * a.H + h) * DH};
  const bool qvalid[MB] = {tvalid};
  Frag<T> qf[MB][DH / 32];
  load_q<T, MB, DH>(qf, qrow, qvalid, g);

  AttnState<MB, DH> st;
  state_init_empty(st);
  T *vt = reinterpret_cast<T *>(smem);
  const T *kb = static_cast<const T *>(a.k) + (size_t)off * kvstride + hk * DH;
  const T *vb = static_cast<const T *>(a.v) + (size_t)off * kvstride + hk * DH;
  const size_t crow = (size_t)(off + (tvalid ? t : 0)) * a.H + h;

  // Key segments: [0, bs) and [be, N) (invariant), then [bs, be) (block).
  const int seg_lo[3] = {0, be, bs};
  const int seg_hi[3] = {bs, N, be};
#pragma unroll 1
  for (int sgi = 0; sgi < 3; ++sgi) {
    if (sgi == 2) {
      // Snapshot of the state over the invariant keys (FACache store).
      const float lt = group_sum(st.l[0]);
      if (in_u) {
        if (g == 0) {
          a.m_w[crow] = st.m[0] * kLn2;
          a.l_w[crow] = lt;
        }
#pragma unroll
        for (int db = 0; db < DH / 16; ++db)
          *reinterpret_cast<f32x4_t *>(a.o_w + crow * DH + 16 * db + 4 * g) = st.o[0][db];
      }
    }
    for (int k0 = seg_lo[sgi]; k0 < seg_hi[sgi]; k0 += TK) {
      const int nk = min(TK, seg_hi[sgi] - k0);
      __syncthreads();
      stage_vt<T, DH>(vt, VTS, vb + (size_t)k0 * kvstride, kvstride, nk, (nk + 31) & ~31, tid, blockDim.x);
      __syncthreads();
      for (int c0 = 0; c0 < nk; c0 += 32)
        attend_step<T, MB, DH>(st, qf, kb + (size_t)(k0 + c0) * kvstride, kvstride, min(32, nk - c0), vt + c0,
                               VTS, a.scale_log2, lane);
    }
  }
  const float lt = group_sum(st.l[0]);
  if (tvalid) {
    const float inv = 1.0f / lt;
    TO *out = static_cast<TO *>(a.out) + crow * DH;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[16 * db + 4 * g + i] = from_f32<TO>(st.o[0][db][i] * inv);
    if (a.lse && g == 0) a.lse[crow] = (st.m[0] + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T, int DH> constexpr size_t step_smem() {
  constexpr size_t vt_a = 4 * DH * (32 + VtPad<T>::v) * sizeof(T);
  constexpr size_t merge_a = (2 * 4 * kRowsA + 4 * kRowsA * DH) * sizeof(float);
  constexpr size_t vt_b = DH * (128 + VtPad<T>::v) * sizeof(T);
  constexpr size_t m1 = vt_a > merge_a ? vt_a : merge_a;
  return m1 > vt_b ? m1 : vt_b;
}
template <typename T, int DH> constexpr size_t refresh_smem() {
  return DH * (128 + VtPad<T>::v) * sizeof(T);
}

// Cache type T and output type TO: fp16 / bf16 for bf16 parameters, fp32 / fp32.
#define LC_DISPATCH(dt, dh, CALL)                                                        \
  do {                                                                                   \
    if (dt == kBF16) {                                                                   \
      if (dh == 128) { using T = f16_t; using TO = bf16_t; constexpr int DH = 128; CALL; } \
      else { using T = f16_t; using TO = bf16_t; constexpr int DH = 64; CALL; }          \
    } else {                                                                             \
      if (dh == 128) { using T = float; using TO = float; constexpr int DH = 128; CALL; }  \
      else { using T = float; using TO = float; constexpr int DH = 64; CALL; }           \
    }                                                                                    \
  } while (0)

hipError_t launch_step_attn(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  LC_DISPATCH(dt, dh, (step_attn_kernel<T, TO, DH><<<n_blocks, 256, step_smem<T, DH>(), s>>>(sa, a)));
  return hipGetLastError();
}

hipError_t launch_block_attn(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  LC_DISPATCH(dt, dh, (block_attn_kernel<T, TO, DH><<<n_blocks, 256, step_smem<T, DH>(), s>>>(sa, a)));
  return hipGetLastError();
}

hipError_t launch_merge(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int M, hipStream_t s) {
  const int waves = M * a.H;
  if (waves <= 0) return hipSuccess;
  LC_DISPATCH(dt, dh, (merge_kernel<T, TO, DH><<<(waves + 3) / 4, 256, 0, s>>>(sa, a, M)));
  return hipGetLastError();
}

hipError_t launch_refresh_attn(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks,
                               hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  LC_DISPATCH(dt, dh, (refresh_attn_kernel<T, TO, DH><<<n_blocks, 256, refresh_smem<T, DH>(), s>>>(sa, a)));
  return hipGetLastError();
}

hipError_t setup_kernel_attributes() {
  hipError_t e = hipSuccess;
#define LC_ATTR(K, BYTES)                                                                        \
  if (e == hipSuccess)                                                                           \
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(K), hipFuncAttributeMaxDynamicSharedMemorySize, \
                            (int)(BYTES));
  LC_ATTR((step_attn_kernel<f16_t, bf16_t, 128>), (step_smem<f16_t, 128>()));
  LC_ATTR((step_attn_kernel<f16_t, bf16_t, 64>), (step_smem<f16_t, 64>()));
  LC_ATTR((step_attn_kernel<float, float, 128>), (step_smem<float, 128>()));
  LC_ATTR((step_attn_kernel<float, float, 64>), (step_smem<float, 64>()));
  LC_ATTR((block_attn_kernel<f16_t, bf16_t, 128>), (step_smem<f16_t, 128>()));
  LC_ATTR((block_attn_kernel<f16_t, bf16_t, 64>), (step_smem<f16_t, 64>()));
  LC_ATTR((block_attn_kernel<float, float, 128>), (step_smem<float, 128>()));
  LC_ATTR((block_attn_kernel<float, float, 64>), (step_smem<float, 64>()));
  LC_ATTR((refresh_attn_kernel<f16_t, bf16_t, 128>), (refresh_smem<f16_t, 128>()));
  LC_ATTR((refresh_attn_kernel<f16_t, bf16_t, 64>), (refresh_smem<f16_t, 64>()));
  LC_ATTR((refresh_attn_kernel<float, float, 128>), (refresh_smem<float, 128>()));
  LC_ATTR((refresh_attn_kernel<float, float, 64>), (refresh_smem<float, 64>()));
#undef LC_ATTR
  return e;
}

}  // namespace lc
