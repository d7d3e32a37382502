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

// ---------------------------------------------------------------------------
// V of up to MAXC keys staged in LDS, read back as the A operand of P*V (one
// head-dim row, 8 consecutive keys per lane).
//   16-bit types: V is kept row-major (key rows of DH + 16 elements; the pad
//   puts 8 consecutive rows on disjoint bank groups) and written with 16-byte
//   stores; the operand is read with ds_read_b64_tr_b16, which hands lane i
//   of a 16-lane group element i%4 of the 8-byte chunks addressed by lanes
//   4j + i/4 (j = 0..3).  Lane t of group g points at key 8g + t/4 (+4 for the
//   second read), features 16*db + 4*(t%4): lane i then holds keys 8g..8g+7
//   of feature 16*db + i.
//   fp32: V is stored transposed, V^T[d][c], and read with plain loads.
// ---------------------------------------------------------------------------
template <typename T, int DH, int MAXC> struct VTile {
  static constexpr bool kTr = sizeof(T) == 2;
  static constexpr int kStride = kTr ? DH + 16 : MAXC + 4;     // elements per LDS row
  static constexpr size_t kBytes = (size_t)(kTr ? MAXC : DH) * kStride * sizeof(T);
};

typedef __fp16 h4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) h4_t lds_h4_t;

template <typename T, int DH, int MAXC>
__device__ __forceinline__ void vtile_frag(Frag<T> &f, const T *buf, int c0, int db, int lane) {
  using VT = VTile<T, DH, MAXC>;
  const int g = lane >> 4, r16 = lane & 15;
  if constexpr (VT::kTr) {
    const T *p = buf + (size_t)(c0 + 8 * g + (r16 >> 2)) * VT::kStride + 16 * db + 4 * (r16 & 3);
    const h4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4_t *)(p));
    const h4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4_t *)(p + 4 * VT::kStride));
    typedef short s4_t __attribute__((ext_vector_type(4)));
    typedef short s8_t __attribute__((ext_vector_type(8)));
    const s4_t a = __builtin_bit_cast(s4_t, lo), b = __builtin_bit_cast(s4_t, hi);
    const s8_t v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    f.v = __builtin_bit_cast(decltype(f.v), v);
  } else {
    frag_load(f, buf + (16 * db + r16) * VT::kStride + c0 + 8 * g);
  }
}

// Stage MAXC keys starting at vbase; keys >= nvalid (>= 1) get a copy of key
// nvalid-1 (finite values; their probabilities are zero).  NTHR threads
// cooperate; consecutive threads take consecutive 16-byte pieces of one key
// row.  Loads and stores are unconditional: any guard lets the compiler sink
// each load next to its store and serialise the round trips.
template <typename T, int DH, int MAXC, int NTHR>
__device__ __forceinline__ void vtile_stage(T *buf, const T *vbase, size_t vstride, int nvalid, int t) {
  using VT = VTile<T, DH, MAXC>;
  constexpr int EPC = 16 / sizeof(T);            // elements per 16-byte piece
  constexpr int CPK = DH / EPC;                  // pieces per key row
  static_assert((MAXC * CPK) % NTHR == 0, "staging threads must tile the buffer");
  constexpr int ITER = MAXC * CPK / NTHR;
  uint4 u[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = t + it * NTHR;
    const int c = min(idx / CPK, nvalid - 1), ch = idx % CPK;
    u[it] = *reinterpret_cast<const uint4 *>(vbase + (size_t)c * vstride + ch * EPC);
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = t + it * NTHR;
    const int c = idx / CPK, ch = idx % CPK;
    if constexpr (VT::kTr) {
      *reinterpret_cast<uint4 *>(buf + (size_t)c * VT::kStride + ch * EPC) = u[it];
    } else {
      const uint32_t wd[4] = {u[it].x, u[it].y, u[it].z, u[it].w};
      uint32_t *v32 = reinterpret_cast<uint32_t *>(buf);
#pragma unroll
      for (int j = 0; j < 4; ++j) v32[(ch * 4 + j) * VT::kStride + c] = wd[j];
    }
  }
}

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
// 64p + 16g + 8*half + (0..7).  Loads are unconditional (callers point rows
// without a query at some valid row and drop their results): a guarded load
// would make the compiler wait for it at the branch join.
template <typename T, int MB, int DH>
__device__ __forceinline__ void load_q(Frag<T> (&qf)[MB][DH / 32], const T *const (&qrow)[MB], int g) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int p = 0; p < DH / 64; ++p) frag_load2(qf[mb][2 * p], qf[mb][2 * p + 1], qrow[mb] + 64 * p + 16 * g);
}

// Key fragments of one step of 32 keys (1 <= nvalid): key block kb (16 keys)
// x head-dim steps.  The A-operand row r16 of key block kb holds key
// 8*(r16/4) + 4*kb + r16%4, so that in the S^T result lane group g holds keys
// 8g..8g+7 of the step (the B-operand slots of P^T in the P*V product).
template <typename T, int DH> struct KStep {
  Frag<T> f[2][DH / 32];
};

template <typename T, int DH>
__device__ __forceinline__ void load_k_step(KStep<T, DH> &kf, const T *kbase, size_t kstride, int nvalid,
                                            int lane) {
  const int g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // Keys past nvalid read key nvalid-1 (their scores are masked later).
    const int key = min(8 * (r16 >> 2) + 4 * kb + (r16 & 3), nvalid - 1);
#pragma unroll
    for (int p = 0; p < DH / 64; ++p)
      frag_load2(kf.f[kb][2 * p], kf.f[kb][2 * p + 1], kbase + (size_t)key * kstride + 64 * p + 16 * g);
  }
}

// One step of up to 32 keys with its key fragments already loaded; V of the
// step is keys c0 .. c0+31 of the staged tile `vbuf`.  Keys >= nvalid are
// masked; their staged V must be finite (the stager copies a valid key).
template <typename T, int MB, int DH, int MAXC>
__device__ __forceinline__ void attend_step_pre(AttnState<MB, DH> &st, const Frag<T> (&qf)[MB][DH / 32],
                                                const KStep<T, DH> &kf, int nvalid, const T *vbuf, int c0,
                                                float scale_log2, int lane) {
  const int g = lane >> 4;
  f32x4_t s[2][MB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s[kb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kd = 0; kd < DH / 32; ++kd) mma16(s[kb][mb], kf.f[kb][kd], qf[mb][kd]);
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
    vtile_frag<T, DH, MAXC>(vf, vbuf, c0, db, lane);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) mma16(st.o[mb][db], vf, pf[mb]);
  }
}

template <typename T, int MB, int DH, int MAXC>
__device__ __forceinline__ void attend_step(AttnState<MB, DH> &st, const Frag<T> (&qf)[MB][DH / 32],
                                            const T *kbase, size_t kstride, int nvalid, const T *vbuf, int c0,
                                            float scale_log2, int lane) {
  KStep<T, DH> kf;
  load_k_step<T, DH>(kf, kbase, kstride, nvalid, lane);
  attend_step_pre<T, MB, DH, MAXC>(st, qf, kf, nvalid, vbuf, c0, scale_log2, lane);
}

// ---------------------------------------------------------------------------
// Type A: 32 block rows x one key chunk -> partial state in the workspace.
// Wave w takes row block w%2 and key half w/2 of every staged 128-key tile.
// ---------------------------------------------------------------------------
constexpr int kTileA = 128;     // keys staged in LDS per tile (type A, refresh)

template <typename T, typename TO, int DH>
__device__ void block_rows_partial(const SeqArgs &sa, const AttnArgs &a, int item, int h, char *smem) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int rb = w & 1, kh = w >> 1;

  const int b = find_sample(sa.pre[1], sa.n, item);
  const int t = item - sa.pre[1][b];
  const int B = sa.be[b] - sa.bs[b], N = sa.len[b];
  const int nrg = (B + kRowsA - 1) / kRowsA;
  const int chunk = t / nrg, rg = t % nrg;
  const int key0 = chunk * a.split_keys;
  const int nkeys = min(a.split_keys, N - key0);
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;

  const int r = rg * kRowsA + rb * 16 + r16;
  const bool qvalid1 = r < B;
  const int rq = min(r, B - 1);
  const int qrow_i = a.qmode == 0 ? sa.off[b] + sa.bs[b] + rq : a.row_base + sa.pre[0][b] + rq;
  const T *qrow[1] = {static_cast<const T *>(a.q) + ((size_t)qrow_i * a.H + h) * DH};
  Frag<T> qf[1][DH / 32];
  load_q<T, 1, DH>(qf, qrow, g);

  AttnState<1, DH> st;
  state_init_empty(st);
  T *vbuf = reinterpret_cast<T *>(smem);
  const T *kbase0 = static_cast<const T *>(a.k) + ((size_t)(sa.off[b] + key0)) * kvstride + hk * DH;
  const T *vbase0 = static_cast<const T *>(a.v) + ((size_t)(sa.off[b] + key0)) * kvstride + hk * DH;
  for (int t0 = 0; t0 < nkeys; t0 += kTileA) {
    const int nk = min(kTileA, nkeys - t0);
    // This wave's two steps of the tile: keys [64*kh, 64*kh + 64).
    KStep<T, DH> kf[2];
    int nv[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int c0 = 64 * kh + 32 * s2;
      nv[s2] = max(0, min(32, nk - c0));
      // A step past the tile's end reads the tile's first keys (and is skipped).
      load_k_step<T, DH>(kf[s2], kbase0 + (size_t)(t0 + (nv[s2] > 0 ? c0 : 0)) * kvstride, kvstride, max(nv[s2], 1),
                         lane);
    }
    __syncthreads();
    vtile_stage<T, DH, kTileA, 256>(vbuf, vbase0 + (size_t)t0 * kvstride, kvstride, nk, tid);
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      if (nv[s2] > 0)
        attend_step_pre<T, 1, DH, kTileA>(st, qf, kf[s2], nv[s2], vbuf, 64 * kh + 32 * s2, a.scale_log2, lane);
  }
  __syncthreads();

  // Merge the two key halves of each row block in LDS, then write the partial.
  float *s_m = reinterpret_cast<float *>(smem);     // [2 row blocks][16]
  float *s_l = s_m + 32;
  float *s_o = s_l + 32;                            // [2][16][DH]
  const float lt = group_sum(st.l[0]);
  if (kh == 1) {
    if (g == 0) {
      s_m[rb * 16 + r16] = st.m[0];
      s_l[rb * 16 + r16] = lt;
    }
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
      *reinterpret_cast<f32x4_t *>(s_o + (rb * 16 + r16) * DH + 16 * db + 4 * g) = st.o[0][db];
  }
  __syncthreads();
  const size_t pbase = (size_t)(a.part_base + sa.pre[3][b]) + r;      // chunk c: pbase + c*B
  if (kh == 0 && qvalid1) {
    const float m1 = s_m[rb * 16 + r16], l1 = s_l[rb * 16 + r16];
    const float mx = fmaxf(st.m[0], m1);
    const float e0 = fast_exp2(st.m[0] - mx), e1 = fast_exp2(m1 - mx);
    const size_t prow = (pbase + (size_t)chunk * B) * a.H + h;
    float *po = a.part_o + prow * DH;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) {
      const f32x4_t o1 = *reinterpret_cast<const f32x4_t *>(s_o + (rb * 16 + r16) * DH + 16 * db + 4 * g);
      *reinterpret_cast<f32x4_t *>(po + 16 * db + 4 * g) = st.o[0][db] * e0 + o1 * e1;
    }
    if (g == 0) a.part_ml[prow] = make_float2(mx, lt * e0 + l1 * e1);
  }
}

// ---------------------------------------------------------------------------
// Type B: 64 invariant rows, state from FACache, stream the block's keys.
// All global loads (queries, FACache, first key step, V^T) are issued before
// the first wait.
// ---------------------------------------------------------------------------
template <typename T, typename TO, int DH, int BMAX>
__device__ void invariant_rows(const SeqArgs &sa, const AttnArgs &a, int item, int h, char *smem) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  const int b = find_sample(sa.pre[2], sa.n, item);
  const int tile = item - sa.pre[2][b];
  const int bs = sa.bs[b], be = sa.be[b], B = be - bs, N = sa.len[b];
  const int nU = N - B;
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;
  const int off = sa.off[b];

  // Rows past the last invariant row load the last one (results dropped).
  const int u = tile * kRowsB + w * 16 + r16;
  const bool uvalid = u < nU;
  const int uc = min(u, nU - 1);
  const int row = off + (uc < bs ? uc : uc + B);
  const T *qrow[1] = {static_cast<const T *>(a.q) + ((size_t)row * a.H + h) * DH};
  Frag<T> qf[1][DH / 32];
  load_q<T, 1, DH>(qf, qrow, g);

  // FACache state of this row (Algorithm 1: initialise with the cache).
  AttnState<1, DH> st;
  const size_t crow = (size_t)row * a.H + h;
  st.m[0] = a.m_c[crow] * kLog2e;
  const float lc = a.l_c[crow];
  st.l[0] = g == 0 ? lc : 0.f;
#pragma unroll
  for (int db = 0; db < DH / 16; ++db)
    st.o[0][db] = *reinterpret_cast<const f32x4_t *>(a.o_c + crow * DH + 16 * db + 4 * g);
  const T *kbase = static_cast<const T *>(a.k) + (size_t)(off + bs) * kvstride + hk * DH;
  KStep<T, DH> kf[2];
  load_k_step<T, DH>(kf[0], kbase, kvstride, min(32, B), lane);

  T *vbuf = reinterpret_cast<T *>(smem);
  vtile_stage<T, DH, BMAX, 256>(vbuf, static_cast<const T *>(a.v) + (size_t)(off + bs) * kvstride + hk * DH, kvstride,
                                B, tid);
  __syncthreads();

  // Up to 4 steps (block <= 128 keys); the next step's keys load during this one.
  for (int c0 = 0; c0 < B; c0 += 64) {
    if (c0 + 32 < B) load_k_step<T, DH>(kf[1], kbase + (size_t)(c0 + 32) * kvstride, kvstride, min(32, B - c0 - 32), lane);
    attend_step_pre<T, 1, DH, BMAX>(st, qf, kf[0], min(32, B - c0), vbuf, c0, a.scale_log2, lane);
    if (c0 + 32 < B) {
      if (c0 + 64 < B) load_k_step<T, DH>(kf[0], kbase + (size_t)(c0 + 64) * kvstride, kvstride, min(32, B - c0 - 64), lane);
      attend_step_pre<T, 1, DH, BMAX>(st, qf, kf[1], min(32, B - c0 - 32), vbuf, c0 + 32, a.scale_log2, lane);
    }
  }

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

// BMAX: staged block keys (32, 64 or 128 >= every block of the launch).
template <typename T, typename TO, int DH, int BMAX>
__global__ __launch_bounds__(256) void step_attn_kernel(const SeqArgs sa, const AttnArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int gid = blockIdx.x;
  if (gid < a.nA) {
    block_rows_partial<T, TO, DH>(sa, a, gid / a.H, gid % a.H, smem);
  } else {
    const int j = gid - a.nA;
    invariant_rows<T, TO, DH, BMAX>(sa, a, j / a.H, j % a.H, smem);
  }
}

// Only type-A items: the DualCache block-query attention.
template <typename T, typename TO, int DH>
__global__ __launch_bounds__(256) void block_attn_kernel(const SeqArgs sa, const AttnArgs a) {
  extern __shared__ __align__(16) char smem[];
  block_rows_partial<T, TO, DH>(sa, a, blockIdx.x / a.H, blockIdx.x % a.H, smem);
}

// ---------------------------------------------------------------------------
// Merge of the type-A partial states: one wave per (block row, head).  Lane c
// reads chunk c's (max, normaliser); the feature sums read all chunks at once.
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
  const size_t pb = (size_t)(a.part_base + sa.pre[3][b] + r) * a.H + h;   // chunk c at pb + c*B*H
  const size_t cstride = (size_t)B * a.H;

  float mx = -INFINITY;
  for (int c = lane; c < nch; c += 64) mx = fmaxf(mx, a.part_ml[pb + c * cstride].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float lsum = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const float2 ml = a.part_ml[pb + c * cstride];
    lsum = fmaf(fast_exp2(ml.x - mx), ml.y, lsum);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lsum += __shfl_xor(lsum, o);

  constexpr int PER = DH / 64;
  float acc[PER] = {};
  for (int c0 = 0; c0 < nch; c0 += 8) {
    float v[8][PER], e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = c0 + j;
      e[j] = 0.f;
      if (c < nch) {
        const size_t prow = pb + c * cstride;
        e[j] = fast_exp2(a.part_ml[prow].x - mx);
#pragma unroll
        for (int k = 0; k < PER; ++k) v[j][k] = a.part_o[prow * DH + lane + 64 * k];
      } else {
#pragma unroll
        for (int k = 0; k < PER; ++k) v[j][k] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] = fmaf(e[j], v[j][k], acc[k]);
  }
  const int orow = a.omode == 0 ? sa.off[b] + sa.bs[b] + r : a.row_base + m;
  const float inv = 1.0f / lsum;
  TO *out = static_cast<TO *>(a.out) + ((size_t)orow * a.H + h) * DH;
#pragma unroll
  for (int k = 0; k < PER; ++k) out[lane + 64 * k] = from_f32<TO>(acc[k] * inv);
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
  const T *qrow[MB] = {q + ((size_t)(off + min(t, N - 1)) * a.H + h) * DH};
  Frag<T> qf[MB][DH / 32];
  load_q<T, MB, DH>(qf, qrow, g);

  AttnState<MB, DH> st;
  state_init_empty(st);
  T *vbuf = reinterpret_cast<T *>(smem);
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
      vtile_stage<T, DH, TK, 256>(vbuf, vb + (size_t)k0 * kvstride, kvstride, nk, tid);
      __syncthreads();
      for (int c0 = 0; c0 < nk; c0 += 32)
        attend_step<T, MB, DH, TK>(st, qf, kb + (size_t)(k0 + c0) * kvstride, kvstride, min(32, nk - c0), vbuf, c0,
                                   a.scale_log2, lane);
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
  constexpr size_t vt = VTile<T, DH, 128>::kBytes;                  // type A tile, type B block keys
  constexpr size_t merge_a = (64 + 32 * DH) * sizeof(float);
  return vt > merge_a ? vt : merge_a;
}
template <typename T, int DH> constexpr size_t refresh_smem() {
  return VTile<T, DH, 128>::kBytes;
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

hipError_t launch_step_attn(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks, hipStream_t s,
                            const LaunchEvents &ev) {
  if (n_blocks <= 0) return hipSuccess;
  int bmax = 0;
  for (int i = 0; i < sa.n; ++i) bmax = bmax > sa.be[i] - sa.bs[i] ? bmax : sa.be[i] - sa.bs[i];
  if (bmax <= 32)
    LC_DISPATCH(dt, dh, (lc_launch(step_attn_kernel<T, TO, DH, 32>, dim3(n_blocks), dim3(256), step_smem<T, DH>(), s, ev, sa, a)));
  else if (bmax <= 64)
    LC_DISPATCH(dt, dh, (lc_launch(step_attn_kernel<T, TO, DH, 64>, dim3(n_blocks), dim3(256), step_smem<T, DH>(), s, ev, sa, a)));
  else
    LC_DISPATCH(dt, dh, (lc_launch(step_attn_kernel<T, TO, DH, 128>, dim3(n_blocks), dim3(256), step_smem<T, DH>(), s, ev, sa, a)));
  return hipGetLastError();
}

hipError_t launch_block_attn(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks, hipStream_t s,
                             const LaunchEvents &ev) {
  if (n_blocks <= 0) return hipSuccess;
  LC_DISPATCH(dt, dh, (lc_launch(block_attn_kernel<T, TO, DH>, dim3(n_blocks), dim3(256), step_smem<T, DH>(), s, ev, sa, a)));
  return hipGetLastError();
}

hipError_t launch_merge(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int M, hipStream_t s,
                        const LaunchEvents &ev) {
  const int waves = M * a.H;
  if (waves <= 0) return hipSuccess;
  LC_DISPATCH(dt, dh, (lc_launch(merge_kernel<T, TO, DH>, dim3((waves + 3) / 4), dim3(256), 0, s, ev, sa, a, M)));
  return hipGetLastError();
}

hipError_t launch_refresh_attn(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks,
                               hipStream_t s, const LaunchEvents &ev) {
  if (n_blocks <= 0) return hipSuccess;
  LC_DISPATCH(dt, dh, (lc_launch(refresh_attn_kernel<T, TO, DH>, dim3(n_blocks), dim3(256), refresh_smem<T, DH>(), s, ev, sa, a)));
  return hipGetLastError();
}

hipError_t setup_kernel_attributes() {
  hipError_t e = hipSuccess;
#define LC_ATTR(K, BYTES)                                                                        \
  if (e == hipSuccess)                                                                           \
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(K), hipFuncAttributeMaxDynamicSharedMemorySize, \
                            (int)(BYTES));
#define LC_ATTR_STEP(BM)                                                   \
  LC_ATTR((step_attn_kernel<f16_t, bf16_t, 128, BM>), (step_smem<f16_t, 128>())); \
  LC_ATTR((step_attn_kernel<f16_t, bf16_t, 64, BM>), (step_smem<f16_t, 64>()));   \
  LC_ATTR((step_attn_kernel<float, float, 128, BM>), (step_smem<float, 128>()));  \
  LC_ATTR((step_attn_kernel<float, float, 64, BM>), (step_smem<float, 64>()));
  LC_ATTR_STEP(32)
  LC_ATTR_STEP(64)
  LC_ATTR_STEP(128)
#undef LC_ATTR_STEP
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
