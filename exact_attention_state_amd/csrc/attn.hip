// First-layer attention kernels of the cached block step (LaCache Section
// 3.3.3, Eqs. (2)-(6); Algorithm 1) and of the block-boundary refresh.
//
// All of them share one 32-key step on MFMA (attend_step):
//   S^T = K Q^T       A = 16 keys x 32 head-dim slots, B = Q^T; the key rows
//                     of a step are loaded in an order that leaves lane group
//                     g holding keys 8g..8g+7 of the step in the result.
//   online softmax    per query row (lane%16), max shared by the 4 lane
//                     groups, scores in log2 units so exp is v_exp_f32.
//   O^T += V^T P^T    A = V^T read from LDS, B = P^T straight from the
//                     softmax registers; the result keeps each query row in
//                     one lane, so the per-row rescale is lane-local.
// With 16-bit caches K and V tiles go through LDS, copied row-wise by the
// load unit (its full-rate access pattern); with fp32 caches K fragments are
// read straight from memory and only V is staged.  Every work item issues
// all of its global loads before its first wait, and its workgroup barriers
// order LDS traffic only, so one item costs one memory round trip per key
// tile.  The streaming kernels further down (block rows, invariant rows,
// refresh) instead keep a ring of tiles in flight.
//
// Work items of the one-tile kernels (one workgroup of 4 waves each, times
// the head count):
//   type A  block rows (<= 32) of one sample against one chunk of its keys
//           [prefix | fresh block | suffix]; wave w takes the w-th 32-key step
//           of every 128-key tile for all 32 rows, and the 4 waves merge their
//           states in LDS; the chunk's (m, l, O~/l) goes to the workspace
//           (split-KV).  This is also the DualCache step.
//   type B  64 invariant rows of one sample: the state starts from FACache and
//           streams only the block's keys, then O = O~/l and LSE = m + ln l.
//   merge   combines the type-A chunks of every block row into O and LSE.
//   refresh 64 rows of one sample against every key (fp32 caches; 16-bit
//           caches use refresh_stream_kernel): invariant keys first, a
//           snapshot of (m, l, O~/l) into FACache for invariant rows, then
//           the block's keys, then O and LSE.
//
// FACache and the partials hold O~/l (the state's output, normalised) in the
// cache type with l beside it: the state (m, l, O~) is restored exactly up to
// that one rounding, at half the bytes of an fp32 O~ for 16-bit caches.

#include <type_traits>

#include "internal.h"

namespace lc {

// ---------------------------------------------------------------------------
// Output slots.  In the P*V result of feature block db, lane (g, r16) slot v
// holds query row r16 and feature OMap<DH>::feat(g, db, v):
//   DH = 128: lane group g owns the 32 contiguous features 32g..32g+31, so a
//             lane moves its part of a row with 16-byte accesses;
//   DH = 64:  block db is features 16db..16db+15, 4 per lane group.
// The V^T operand is read in the matching order (vtile_frag).
// ---------------------------------------------------------------------------
template <int DH> struct OMap {
  static constexpr bool kWide = DH == 128;
  static constexpr int NDB = DH / 16;
  __device__ static constexpr int feat(int g, int db, int v) {
    return kWide ? 32 * g + 4 * db + v : 16 * db + 4 * g + v;
  }
};

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float2 unpack2(f16_t, uint32_t u) {
  const h2_t v = __builtin_bit_cast(h2_t, u);
  return make_float2((float)v[0], (float)v[1]);
}
__device__ __forceinline__ float2 unpack2(bf16_t, uint32_t u) {
  return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}
template <typename T> __device__ __forceinline__ f32x4_t unpack4(uint32_t lo, uint32_t hi) {
  const float2 a = unpack2(T{}, lo), b = unpack2(T{}, hi);
  return f32x4_t{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ uint32_t pack2(f16_t, float a, float b) {
  const h2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack2(bf16_t, float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// 4 consecutive elements <-> f32x4 (8-byte aligned for 16-bit types).
template <typename T> __device__ __forceinline__ f32x4_t ld4(const T *p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4_t *>(p);
  } else {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return unpack4<T>(u.x, u.y);
  }
}
template <typename T> __device__ __forceinline__ void st4(T *p, f32x4_t x) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4_t *>(p) = x;
  } else {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack2(T{}, x[0], x[1]), pack2(T{}, x[2], x[3]));
  }
}

// This lane's features of one row: x[db][v] = row[feat(g, db, v)].
template <typename T, int DH>
__device__ __forceinline__ void load_row(f32x4_t (&x)[DH / 16], const T *row, int g) {
  if constexpr (OMap<DH>::kWide && sizeof(T) == 2) {
    const uint4 *p = reinterpret_cast<const uint4 *>(row + 32 * g);
#pragma unroll
    for (int j = 0; j < DH / 32; ++j) {
      const uint4 u = p[j];
      x[2 * j] = unpack4<T>(u.x, u.y);
      x[2 * j + 1] = unpack4<T>(u.z, u.w);
    }
  } else {
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) x[db] = ld4(row + OMap<DH>::feat(g, db, 0));
  }
}

// row[feat(g, db, v)] = x[db][v] * scale.
template <typename T, int DH>
__device__ __forceinline__ void store_row(T *row, const f32x4_t (&x)[DH / 16], float scale, int g) {
  if constexpr (OMap<DH>::kWide && sizeof(T) == 2) {
    uint4 *p = reinterpret_cast<uint4 *>(row + 32 * g);
#pragma unroll
    for (int j = 0; j < DH / 32; ++j) {
      const f32x4_t a = x[2 * j] * scale, b = x[2 * j + 1] * scale;
      p[j] = make_uint4(pack2(T{}, a[0], a[1]), pack2(T{}, a[2], a[3]), pack2(T{}, b[0], b[1]),
                        pack2(T{}, b[2], b[3]));
    }
  } else {
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) st4(row + OMap<DH>::feat(g, db, 0), x[db] * scale);
  }
}

// ---------------------------------------------------------------------------
// V of up to MAXC keys staged in LDS, read back as the A operand of P*V (one
// feature block, 8 consecutive keys per lane).
//   16-bit types: V is copied global -> LDS by the load unit itself
//   (global_load_lds_dwordx4: lane l of an instruction fills 16 bytes at the
//   wave's LDS base + 16 l), key rows of DH elements, their 16-byte pieces
//   permuted within the row: piece p of key c sits in slot p ^ (c & 3).  The
//   operand is read with ds_read_b64_tr_b16, which hands lane i of a 16-lane
//   group element i%4 of the 8-byte chunks addressed by lanes 4j + i/4
//   (j = 0..3).  Lane t of group g points at key 8g + t/4 (+4 for the second
//   read) and the 4 features feat(t%4, db, 0..3): lane i then holds keys
//   8g..8g+7 of feature feat(i/4, db, i%4), which is A row i.  The slot
//   permutation puts the 16 lanes of one read on distinct banks.
//   fp32: V is staged through registers and stored transposed, V^T[d][c]
//   (rows of MAXC + 4), and read with plain loads.
// ---------------------------------------------------------------------------
template <typename T, int DH, int MAXC> struct VTile {
  static constexpr bool kTr = sizeof(T) == 2;
  static constexpr int kStride = kTr ? DH : MAXC + 4;       // elements per LDS row
  static constexpr size_t kBytes = (size_t)(kTr ? MAXC : DH) * kStride * sizeof(T);
};

typedef __fp16 h4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) h4_t lds_h4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Global -> LDS copy, 16 bytes per lane, to the wave-uniform LDS address
// `lds` + 16 * lane.  The builtin exists in the device pass only.
__device__ __forceinline__ void load_lds16(const void *src, void *lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (lds_void_t *)lds, 16, 0, 0);
#endif
}

template <typename T, int DH, int MAXC>
__device__ __forceinline__ void vtile_frag(Frag<T> &f, const T *buf, int c0, int db, int lane) {
  using VT = VTile<T, DH, MAXC>;
  const int g = lane >> 4, r16 = lane & 15;
  if constexpr (VT::kTr) {
    const int c = c0 + 8 * g + (r16 >> 2);
    const int fe = OMap<DH>::feat(r16 & 3, db, 0);
    const T *p = buf + (size_t)c * DH + (((fe >> 3) ^ (c & 3)) << 3) + (fe & 4);
    const h4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4_t *)(p));
    const h4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4_t *)(p + 4 * DH));
    typedef short s4_t __attribute__((ext_vector_type(4)));
    typedef short s8_t __attribute__((ext_vector_type(8)));
    const s4_t a = __builtin_bit_cast(s4_t, lo), b = __builtin_bit_cast(s4_t, hi);
    const s8_t v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    f.v = __builtin_bit_cast(decltype(f.v), v);
  } else {
    frag_load(f, buf + OMap<DH>::feat(r16 >> 2, db, r16 & 3) * VT::kStride + c0 + 8 * g);
  }
}

// Stage MAXC keys starting at vbase; keys >= nvalid (>= 1) get a copy of key
// nvalid-1 (finite values; their probabilities are zero).  NTHR threads
// cooperate.  16-bit types: the copies are in flight when this returns and
// vtile_wait() (before the barrier that publishes the tile) completes them.
// fp32: loads, then transposed stores (unconditional: any guard lets the
// compiler sink each load next to its store and serialise the round trips).
template <typename T, int DH, int MAXC, int NTHR>
__device__ __forceinline__ void vtile_stage(T *buf, const T *vbase, size_t vstride, int nvalid, int t) {
  using VT = VTile<T, DH, MAXC>;
  constexpr int EPC = 16 / sizeof(T);            // elements per 16-byte piece
  constexpr int CPK = DH / EPC;                  // pieces per key row
  static_assert((MAXC * CPK) % NTHR == 0, "staging threads must tile the buffer");
  constexpr int ITER = MAXC * CPK / NTHR;
  if constexpr (VT::kTr) {
    const int lane = t & 63, w = t >> 6;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int base = (it * (NTHR / 64) + w) * 64;        // first LDS slot of this wave's instruction
      const int idx = base + lane;
      const int c = idx / CPK, slot = idx % CPK;
      const int piece = slot ^ (c & 3);
      const T *src = vbase + (size_t)min(c, nvalid - 1) * vstride + piece * EPC;
      load_lds16(src, buf + (size_t)base * EPC);
    }
  } else {
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
      const uint32_t wd[4] = {u[it].x, u[it].y, u[it].z, u[it].w};
      uint32_t *v32 = reinterpret_cast<uint32_t *>(buf);
#pragma unroll
      for (int j = 0; j < 4; ++j) v32[(ch * 4 + j) * VT::kStride + c] = wd[j];
    }
  }
}

// K of up to MAXC keys staged in LDS (16-bit types), key rows of DH
// elements: key c's 16-byte piece p sits in slot p ^ kslot(c) (ppr pieces
// per row), so the 16 keys of one A-operand read (8a + b + 4kb, a, b < 4)
// hit distinct slots.  Copied global -> LDS by the load unit, row-wise;
// keys >= nvalid (>= 1) get a copy of key nvalid-1.
__device__ __forceinline__ int kslot(int c, int ppr) {
  return ppr == 16 ? (((c >> 1) & 12) | (c & 3)) : (((c >> 1) & 4) | (c & 3));
}
template <typename T, int DH, int MAXC, int NTHR>
__device__ __forceinline__ void ktile_stage(T *buf, const T *kbase, size_t kstride, int nvalid, int t) {
  static_assert(sizeof(T) == 2, "16-bit K tiles");
  constexpr int CPK = DH / 8;                    // 16-byte pieces per key row
  static_assert((MAXC * CPK) % NTHR == 0, "staging threads must tile the buffer");
  constexpr int ITER = MAXC * CPK / NTHR;
  const int lane = t & 63, w = t >> 6;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int base = (it * (NTHR / 64) + w) * 64;        // first LDS slot of this wave's instruction
    const int idx = base + lane;
    const int c = idx / CPK, slot = idx % CPK;
    const T *src = kbase + (size_t)min(c, nvalid - 1) * kstride + ((slot ^ kslot(c, CPK)) << 3);
    load_lds16(src, buf + (size_t)base * 8);
  }
}

// Completes this wave's global->LDS copies (and every other global load it
// has in flight); a barrier must follow before other waves read the tile.
__device__ __forceinline__ void vtile_wait() {
  __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0), expcnt and lgkmcnt untouched
}

template <int MB, int DH> struct AttnState {
  float m[MB];                 // running max, log2 units (same in the 4 lane groups)
  float l[MB];                 // this lane's share of the normaliser
  f32x4_t o[MB][DH / 16];      // O~ of row lane%16, features feat(g, db, 0..3)
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

// The same fragments from a K tile staged in LDS (ktile_stage), keys c0 ..
// c0+31 of the tile (keys past the valid ones are copies: masked later).
template <typename T, int DH>
__device__ __forceinline__ void load_k_step_lds(KStep<T, DH> &kf, const T *kbuf, int c0, int lane) {
  const int g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int c = c0 + 8 * (r16 >> 2) + 4 * kb + (r16 & 3);
#pragma unroll
    for (int kd = 0; kd < DH / 32; ++kd) {
      const int e0 = 64 * (kd >> 1) + 16 * g + 8 * (kd & 1);
      frag_load(kf.f[kb][kd], kbuf + (size_t)c * DH + (((e0 >> 3) ^ kslot(c, DH / 8)) << 3));
    }
  }
}

// Online-softmax update and P*V of one step of up to 32 keys, from its
// scores S^T (s[kb][mb]: key block kb, row block mb).  V of the step is keys
// c0 .. c0+31 of the staged tile `vbuf`.  Keys >= nvalid are masked; their
// staged V must be finite (the stager copies a valid key).  The scale
// (> 0, log2 units) enters through the exponent's fma: the row max is taken
// on raw scores (max(c s) = c max(s) for c > 0, bit for bit, as rounding is
// monotone), and p = 2^(c s - m) is one fused operation.  Steps with all 32
// keys valid skip the masking.
template <typename T, int MB, int DH, int MAXC>
__device__ __forceinline__ void softmax_pv(AttnState<MB, DH> &st, const f32x4_t (&s)[2][MB], int nvalid,
                                           const T *vbuf, int c0, float scale_log2, int lane) {
  const int g = lane >> 4;
  Frag<T> pf[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = s[j >> 2][mb][j & 3];
    if (nvalid < 32) {                          // wave-uniform
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (8 * g + j >= nvalid) x[j] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = group_max(mx) * scale_log2;
    const float mnew = fmaxf(st.m[mb], mx);
    const float alpha = fast_exp2(st.m[mb] - mnew);
    st.m[mb] = mnew;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = fast_exp2(fmaf(x[j], scale_log2, -mnew));   // masked: 2^-inf = 0
      ps += p;
      frag_set(pf[mb], j, p);
    }
    st.l[mb] = fmaf(st.l[mb], alpha, ps);
    // Once the running maxima stop moving, alpha is exactly 1 in every lane
    // and the rescale (a multiply per accumulator) is skipped; multiplying
    // by 1 is exact, so the result does not depend on the branch.
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < DH / 16; ++db) st.o[mb][db] *= alpha;
    }
  }
#pragma unroll
  for (int db = 0; db < DH / 16; ++db) {
    Frag<T> vf;
    vtile_frag<T, DH, MAXC>(vf, vbuf, c0, db, lane);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) mma16(st.o[mb][db], vf, pf[mb]);
  }
}

// The same update over one 64-key tile at once (two 32-key halves: sc[h]
// are the S^T blocks of keys 32h ..; nvalid in [1, 64]): one row max, one
// rescale and one normaliser update per tile, and the P*V products of both
// halves.  V of the tile is keys 0 .. 63 of `vbuf`.
template <typename T, int MB, int DH, int MAXC>
__device__ __forceinline__ void softmax_pv64(AttnState<MB, DH> &st, const f32x4_t (&sc)[2][2][MB], int nvalid,
                                             const T *vbuf, float scale_log2, int lane) {
  const int g = lane >> 4;
  Frag<T> pf[2][MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = sc[j >> 3][(j >> 2) & 1][mb][j & 3];
    if (nvalid < 64) {                          // wave-uniform
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (32 * (j >> 3) + 8 * g + (j & 7) >= nvalid) x[j] = -INFINITY;
    }
    float m8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m8[j] = fmaxf(x[j], x[j + 8]);
    float mx = fmaxf(fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3])), fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7])));
    mx = group_max(mx) * scale_log2;
    const float mnew = fmaxf(st.m[mb], mx);
    const float alpha = fast_exp2(st.m[mb] - mnew);
    st.m[mb] = mnew;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = fast_exp2(fmaf(x[j], scale_log2, -mnew));   // masked: 2^-inf = 0
      ps += p;
      frag_set(pf[j >> 3][mb], j & 7, p);
    }
    st.l[mb] = fmaf(st.l[mb], alpha, ps);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < DH / 16; ++db) st.o[mb][db] *= alpha;
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (32 * h >= nvalid) break;                // wave-uniform: the second half holds no key
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) {
      Frag<T> vf;
      vtile_frag<T, DH, MAXC>(vf, vbuf, 32 * h, db, lane);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) mma16(st.o[mb][db], vf, pf[h][mb]);
    }
  }
}

// One step of up to 32 keys with its key fragments and query fragments in
// registers.
template <typename T, int MB, int DH, int MAXC>
__device__ __forceinline__ void attend_step_pre(AttnState<MB, DH> &st, const Frag<T> (&qf)[MB][DH / 32],
                                                const KStep<T, DH> &kf, int nvalid, const T *vbuf, int c0,
                                                float scale_log2, int lane) {
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
  softmax_pv<T, MB, DH, MAXC>(st, s, nvalid, vbuf, c0, scale_log2, lane);
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
// Query rows staged in LDS (type A): row r of DH elements, its 16-byte piece
// p in slot p ^ (r & SWZ), so that the 16 rows of one operand read fall on
// distinct banks.  Filled with global -> LDS copies.
// ---------------------------------------------------------------------------
template <typename T, int DH> struct QTile {
  static constexpr int EPC = 16 / (int)sizeof(T);        // elements per piece
  static constexpr int PPR = DH / EPC;                   // pieces per row
  static constexpr int SWZ = (PPR < 16 ? PPR : 16) - 1;
};

// B-operand fragment of Q^T: row `row`, head-dim step kd (the slot mapping
// of load_q).
template <typename T, int DH>
__device__ __forceinline__ void qtile_frag(Frag<T> &f, const T *qbuf, int row, int kd, int g) {
  using QT = QTile<T, DH>;
  const int e0 = 64 * (kd >> 1) + 16 * g + 8 * (kd & 1);
  const T *rp = qbuf + (size_t)row * DH;
  if constexpr (sizeof(T) == 2) {
    frag_load(f, rp + ((e0 / QT::EPC) ^ (row & QT::SWZ)) * QT::EPC);
  } else {
    const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(rp + ((e0 / 4) ^ (row & QT::SWZ)) * 4);
    const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(rp + ((e0 / 4 + 1) ^ (row & QT::SWZ)) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.v[i] = lo[i];
      f.v[4 + i] = hi[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Type A: 32 block rows x one key chunk -> partial state in the workspace.
// Per 128-key tile, wave w takes keys 32w..32w+31 for both 16-row blocks.
// ---------------------------------------------------------------------------
constexpr int kTileA = 128;     // keys staged in LDS per tile (type A, refresh)

// LDS of the type-A state merge: per wave (m, l) of 32 rows, and the feature
// blocks each wave hands to the three others.
template <int DH> constexpr size_t merge_a_bytes() {
  return 4 * 2 * 32 * sizeof(float) + (size_t)(DH / 16) * 3 * 2 * 64 * sizeof(f32x4_t);
}


template <typename T, typename TO, int DH>
__device__ void block_rows_partial(const SeqArgs &sa, const AttnArgs &a, int item, int h, char *smem) {
  constexpr int MB = 2, NDB = DH / 16, DPW = NDB / 4;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  const int b = find_sample(sa.pre[1], sa.n, item);
  const int t = item - sa.pre[1][b];
  const int B = sa.be[b] - sa.bs[b], N = sa.len[b];
  const int nrg = (B + kRowsA - 1) / kRowsA;
  const int chunk = t / nrg, rg = t % nrg;
  const int key0 = chunk * a.split_keys;
  const int nkeys = min(a.split_keys, N - key0);
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;

  // The 32 query rows go to LDS once (rows past the block repeat its last
  // row; their results are dropped); each wave reads the fragments of one
  // head-dim step at a time.
  using QT = QTile<T, DH>;
  constexpr bool kLdsK = sizeof(T) == 2;     // 16-bit caches: K staged row-wise in LDS too
  T *qbuf = reinterpret_cast<T *>(smem);
  T *vbuf = qbuf + kRowsA * DH;
  T *kbuf = vbuf + VTile<T, DH, kTileA>::kBytes / sizeof(T);
  {
    const int qrow0 = a.qmode == 0 ? sa.off[b] + sa.bs[b] : a.row_base + sa.pre[0][b];
#pragma unroll
    for (int it = 0; it < kRowsA * QT::PPR / 256; ++it) {
      const int base = (it * 4 + w) * 64;
      const int idx = base + lane;
      const int r = idx / QT::PPR, slot = idx % QT::PPR;
      const int rq = min(rg * kRowsA + r, B - 1);
      const T *src = static_cast<const T *>(a.q) + ((size_t)(qrow0 + rq) * a.H + h) * DH +
                     (slot ^ (r & QT::SWZ)) * QT::EPC;
      load_lds16(src, qbuf + (size_t)base * QT::EPC);
    }
  }

  AttnState<MB, DH> st;
  state_init_empty(st);
  const T *kbase0 = static_cast<const T *>(a.k) + ((size_t)(sa.off[b] + key0)) * kvstride + hk * DH;
  const T *vbase0 = static_cast<const T *>(a.v) + ((size_t)(sa.off[b] + key0)) * kvstride + hk * DH;
  for (int t0 = 0; t0 < nkeys; t0 += kTileA) {
    const int nk = min(kTileA, nkeys - t0);
    const int c0 = 32 * w;
    const int nv = max(0, min(32, nk - c0));
    // A step past the tile's end reads the tile's first keys (and is skipped).
    KStep<T, DH> kf;
    if constexpr (!kLdsK)
      load_k_step<T, DH>(kf, kbase0 + (size_t)(t0 + (nv > 0 ? c0 : 0)) * kvstride, kvstride, max(nv, 1), lane);
    if (t0 > 0) lds_barrier();                 // the previous tile's K and V reads are done
    if constexpr (kLdsK) ktile_stage<T, DH, kTileA, 256>(kbuf, kbase0 + (size_t)t0 * kvstride, kvstride, nk, tid);
    vtile_stage<T, DH, kTileA, 256>(vbuf, vbase0 + (size_t)t0 * kvstride, kvstride, nk, tid);
    vtile_wait();
    lds_barrier();
    if constexpr (kLdsK) load_k_step_lds<T, DH>(kf, kbuf, nv > 0 ? c0 : 0, lane);
    if (nv > 0) {
      f32x4_t sc[2][MB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) sc[kb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kd = 0; kd < DH / 32; ++kd) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          Frag<T> qf;
          qtile_frag<T, DH>(qf, qbuf, mb * 16 + r16, kd, g);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma16(sc[kb][mb], kf.f[kb][kd], qf);
        }
      }
      softmax_pv<T, MB, DH, kTileA>(st, sc, nv, vbuf, c0, a.scale_log2, lane);
    }
  }

  // Merge the 4 waves' states.  Wave w finalises feature blocks
  // [w*DPW, (w+1)*DPW) of all 32 rows; the others hand it those blocks.
  lds_barrier();                               // V reads are done; reuse the LDS
  float *s_m = reinterpret_cast<float *>(smem);               // [wave][32 rows]
  float *s_l = s_m + 4 * 32;
  f32x4_t *s_o = reinterpret_cast<f32x4_t *>(s_l + 4 * 32);   // [db][3 givers][mb][lane]
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const float lt = group_sum(st.l[mb]);
    if (g == 0) {
      s_m[w * 32 + mb * 16 + r16] = st.m[mb];
      s_l[w * 32 + mb * 16 + r16] = lt;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int owner = db / DPW;
      if (owner != w) s_o[((db * 3 + (w < owner ? w : w - 1)) * MB + mb) * 64 + lane] = st.o[mb][db];
    }
  }
  lds_barrier();
  const size_t p0 = (size_t)(a.part_base + sa.pre[3][b]);         // partial row of (chunk c, row r): p0 + c*B + r
  T *part_o = static_cast<T *>(a.part_o);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = rg * kRowsA + mb * 16 + r16;
    float e[4], mx = -INFINITY;
#pragma unroll
    for (int ws = 0; ws < 4; ++ws) mx = fmaxf(mx, s_m[ws * 32 + mb * 16 + r16]);
    float L = 0.f;
#pragma unroll
    for (int ws = 0; ws < 4; ++ws) {
      e[ws] = fast_exp2(s_m[ws * 32 + mb * 16 + r16] - mx);
      L = fmaf(e[ws], s_l[ws * 32 + mb * 16 + r16], L);
    }
    const float inv = 1.0f / L;
    const size_t prow = (p0 + (size_t)chunk * B + r) * a.H + h;
    // db runs over compile-time values (a register array indexed by the wave
    // number would be placed in scratch memory); the branch is wave-uniform.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if (db / DPW != w) continue;
      f32x4_t acc = st.o[mb][db] * e[w];
#pragma unroll
      for (int ws = 0; ws < 4; ++ws)
        if (ws != w) acc += s_o[((db * 3 + (ws < w ? ws : ws - 1)) * MB + mb) * 64 + lane] * e[ws];
      if (r < B) st4(part_o + prow * DH + OMap<DH>::feat(g, db, 0), acc * inv);
    }
    if (r < B && w == 0 && g == 0) a.part_ml[prow] = make_float2(mx, L);
  }
}

// ---------------------------------------------------------------------------
// Type B: 64*MB invariant rows (MB row blocks of 16 per wave), state from
// FACache, stream the block's keys.  All global loads (queries, FACache,
// first key step, V) are issued before the first wait.
// ---------------------------------------------------------------------------
template <typename T, typename TO, int DH, int BMAX, int MB>
__device__ void invariant_rows(const SeqArgs &sa, const AttnArgs &a, int item, int h, char *smem) {
  constexpr int NDB = DH / 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  const int b = find_sample(sa.pre[2], sa.n, item);
  const int tile = item - sa.pre[2][b];
  const int bs = sa.bs[b], be = sa.be[b], B = be - bs, N = sa.len[b];
  const int nU = N - B;
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;
  const int off = sa.off[b];

  // Wave w owns row blocks w*MB .. w*MB+MB-1 of the item's 64*MB rows.
  // Rows past the last invariant row load the last one (results dropped).
  const T *qrow[MB];
  size_t crow[MB];
  bool uvalid[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int u = tile * (kRowsB * MB) + (w * MB + mb) * 16 + r16;
    uvalid[mb] = u < nU;
    const int uc = min(u, nU - 1);
    const int row = off + (uc < bs ? uc : uc + B);
    crow[mb] = (size_t)row * a.H + h;
    qrow[mb] = static_cast<const T *>(a.q) + crow[mb] * DH;
  }
  Frag<T> qf[MB][DH / 32];
  load_q<T, MB, DH>(qf, qrow, g);

  // FACache state of these rows (Algorithm 1: initialise with the cache).
  float mc[MB], lc[MB];
  f32x4_t oc[MB][NDB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    mc[mb] = a.m_c[crow[mb]];
    lc[mb] = a.l_c[crow[mb]];
    load_row<T, DH>(oc[mb], static_cast<const T *>(a.o_c) + crow[mb] * DH, g);
  }
  const T *kbase = static_cast<const T *>(a.k) + (size_t)(off + bs) * kvstride + hk * DH;
  // 16-bit caches: the block's K is staged row-wise in LDS once per
  // workgroup (one copy instead of one fragment load per wave).
  constexpr bool kLds = sizeof(T) == 2;
  KStep<T, DH> kf[2];
  T *vbuf = reinterpret_cast<T *>(smem);
  T *kbuf = vbuf + VTile<T, DH, BMAX>::kBytes / sizeof(T);
  if constexpr (kLds) ktile_stage<T, DH, BMAX, 256>(kbuf, kbase, kvstride, B, tid);
  else load_k_step<T, DH>(kf[0], kbase, kvstride, min(32, B), lane);

  vtile_stage<T, DH, BMAX, 256>(vbuf, static_cast<const T *>(a.v) + (size_t)(off + bs) * kvstride + hk * DH, kvstride,
                                B, tid);
  vtile_wait();
  lds_barrier();

  AttnState<MB, DH> st;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    st.m[mb] = mc[mb] * kLog2e;
    st.l[mb] = g == 0 ? lc[mb] : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.o[mb][db] = oc[mb][db] * lc[mb];
  }

  if constexpr (kLds) {
    for (int c0 = 0; c0 < B; c0 += 32) {
      load_k_step_lds<T, DH>(kf[0], kbuf, c0, lane);
      attend_step_pre<T, MB, DH, BMAX>(st, qf, kf[0], min(32, B - c0), vbuf, c0, a.scale_log2, lane);
    }
  } else
  // Up to 4 steps (block <= 128 keys); the next step's keys load during this one.
  for (int c0 = 0; c0 < B; c0 += 64) {
    if (c0 + 32 < B) load_k_step<T, DH>(kf[1], kbase + (size_t)(c0 + 32) * kvstride, kvstride, min(32, B - c0 - 32), lane);
    attend_step_pre<T, MB, DH, BMAX>(st, qf, kf[0], min(32, B - c0), vbuf, c0, a.scale_log2, lane);
    if (c0 + 32 < B) {
      if (c0 + 64 < B) load_k_step<T, DH>(kf[0], kbase + (size_t)(c0 + 64) * kvstride, kvstride, min(32, B - c0 - 64), lane);
      attend_step_pre<T, MB, DH, BMAX>(st, qf, kf[1], min(32, B - c0 - 32), vbuf, c0 + 32, a.scale_log2, lane);
    }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const float lt = group_sum(st.l[mb]);
    if (uvalid[mb]) {
      store_row<TO, DH>(static_cast<TO *>(a.out) + crow[mb] * DH, st.o[mb], 1.0f / lt, g);
      if (a.lse && g == 0) a.lse[crow[mb]] = (st.m[mb] + __log2f(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// Type B, streaming (16-bit caches, blocks of at most 32 * NKS keys): one
// wave per item (sample, head, segment of a.seg_rows invariant rows), taken
// in groups of 16 rows.  NW waves per workgroup, each on its own item with
// its own LDS; die d (workgroups d, d + 8, ...) takes the d-th eighth of the
// segments, every head of a segment on consecutive waves, so the rows' (m,
// l) reads and LSE writes (all heads of a row share their lines) and a
// sample's block keys stay within one die's L2.  Four waves per workgroup
// (one workgroup per CU by LDS) spread the segments evenly over the CUs
// (single-wave workgroups left some CUs with six waves and others with two:
// long4 101 -> 89.5 us, batched16 46.5 -> 40.1 us, varlen32 210 -> 194 us
// with 192-row segments).  The load unit only reaches full rate when
// consecutive lanes move consecutive 16-byte pieces, which the MFMA layouts
// (lane = row) never do; so every global access of the loop is row-wise:
// the queries, FACache rows and (m, l) of a group arrive by global -> LDS
// copies (pieces swizzled as in QTile), three groups ahead of their use,
// and the outputs leave through an LDS tile read back row-wise.  The block's
// K fragments stay in registers and its V in LDS for the whole item.
// ---------------------------------------------------------------------------
template <int DH, int NKS> struct StreamLds {
  static constexpr int ROWB = DH * 2;                         // bytes per 16-bit row
  static constexpr int PPR = ROWB / 16;                       // 16-byte pieces per row (<= 16)
  static constexpr int SWZ = PPR - 1;
  static constexpr int RPC = 1024 / ROWB;                     // rows per 1 KB copy
  static constexpr int TILE = 16 * ROWB;                      // a group's 16 rows
  static constexpr int CPT = TILE / 1024;                     // copies (or row-wise accesses) per tile
  static constexpr int V = (int)VTile<f16_t, DH, 32 * NKS>::kBytes;
  static constexpr int SLOT = TILE + 256;                     // queries, (m, l)
  static constexpr int NSLOT = 3;
  static constexpr int OUT = V + NSLOT * SLOT;                // P*V / l tile (fp16), then 16 row coefficients
  static constexpr int BYTES = OUT + TILE + 64;
  static constexpr int COPIES = CPT + 1;                      // copy instructions per group
  static constexpr int LOADS = CPT;                           // FACache row loads per group (row-wise, to registers)
  static_assert(4 * BYTES <= 160 * 1024, "four waves' LDS must fit a CU");
};

// V of up to MAXC keys into a VTile (16-bit) by one wave, with dma16.
template <int DH, int MAXC>
__device__ __forceinline__ void vtile_stage_wave(uint32_t lds, const f16_t *vbase, size_t vstride, int nvalid,
                                                 int lane) {
  constexpr int CPK = DH / 8;                                 // pieces per key row
  constexpr int ITER = MAXC * CPK / 64;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = it * 64 + lane;
    const int c = idx / CPK, slot = idx % CPK;
    dma16(vbase + (size_t)min(c, nvalid - 1) * vstride + ((slot ^ (c & 3)) << 3), lds + it * 1024);
  }
}

template <typename TO, int DH, int NKS, int NW>
__global__ __launch_bounds__(64 * NW) void invariant_stream_kernel(const SeqArgs sa, const AttnArgs a) {
  using T = f16_t;
  using L = StreamLds<DH, NKS>;
  constexpr int NDB = DH / 16, BMAX = 32 * NKS;
  extern __shared__ __align__(16) char smem_all[];
  char *const smem = smem_all + (threadIdx.x >> 6) * L::BYTES;
  const int nit = sa.pre[2][sa.n];
  const int die = blockIdx.x & 7, j = (blockIdx.x >> 3) * NW + (threadIdx.x >> 6);
  const int lo = (int)((long)die * nit / 8), hi = (int)((long)(die + 1) * nit / 8);
  const int item = lo + j / a.H, h = j % a.H;
  if (item >= hi) return;                                     // whole wave; no barriers below
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int b = find_sample(sa.pre[2], sa.n, item);
  const int seg = item - sa.pre[2][b];
  const int bs = sa.bs[b], B = sa.be[b] - bs, nU = sa.len[b] - B;
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;
  const int off = sa.off[b];
  const int u0 = seg * a.seg_rows, u1 = min(nU, u0 + a.seg_rows);   // u0 < u1 by construction
  const int ngroups = (u1 - u0 + 15) >> 4;
  const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const int rw0 = lane / L::PPR, piece = lane % L::PPR;           // row-wise lane: row rw0 (+ RPC c), piece

  // (cache row * H + h) of row r of group grp; rows past the segment repeat
  // its last row, whose results they reproduce bit for bit (so their stores
  // need no guard).
  auto crow_of = [&](int grp, int r) -> size_t {
    const int u = min(u0 + grp * 16 + r, u1 - 1);
    return (size_t)(off + (u < bs ? u : u + B)) * a.H + h;
  };
  // Copies of group grp's queries into slot sl (copy c: rows c*RPC.., LDS
  // slot s of row r <- piece s ^ (r & SWZ)) and its (m, l) (lanes 0-15: m
  // of rows 0-15, 16-31: l; the upper half repeats them).
  auto issue = [&](int grp, int sl) {
    const uint32_t sb = lbase + L::V + sl * L::SLOT;
#pragma unroll
    for (int c = 0; c < L::CPT; ++c) {
      const int r = c * L::RPC + rw0;
      dma16(static_cast<const T *>(a.q) + crow_of(grp, r) * DH + ((piece ^ (r & L::SWZ)) << 3), sb + c * 1024);
    }
    const size_t cm = crow_of(grp, lane & 15);
    dma4((lane & 16) ? static_cast<const void *>(a.l_c + cm) : static_cast<const void *>(a.m_c + cm), sb + L::TILE);
  };
  // FACache rows of group grp, row-wise into registers.  Ordinary loads:
  // the compiler waits for them itself before their use, counting only the
  // memory instructions it knows of (not the copies), so it can only wait
  // longer than needed, never less.
  typedef uint4 ORow[L::CPT];
  auto load_o = [&](ORow &o, int grp) {
#pragma unroll
    for (int c = 0; c < L::CPT; ++c)
      o[c] = *reinterpret_cast<const uint4 *>(static_cast<const T *>(a.o_c) + crow_of(grp, c * L::RPC + rw0) * DH +
                                              piece * 8);
  };

  // The block's K fragments (registers) and V (LDS), and the first three
  // groups' inputs; all complete before the loop.
  const T *kbase = static_cast<const T *>(a.k) + (size_t)(off + bs) * kvstride + hk * DH;
  KStep<T, DH> kf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    load_k_step<T, DH>(kf[ks], kbase + (size_t)min(32 * ks, B - 1) * kvstride, kvstride, max(1, min(32, B - 32 * ks)),
                       lane);
  // Six register sets: group i reads set i mod 6 and refills set
  // (i + 3) mod 6, so no set holds two live values at once (with three, the
  // old and new rows overlap and the loop needs moves that wait for loads).
  ORow o0, o1, o2, o3, o4, o5;
  issue(0, 0);
  load_o(o0, 0);
  if (ngroups > 1) { issue(1, 1); load_o(o1, 1); }
  if (ngroups > 2) { issue(2, 2); load_o(o2, 2); }
  vtile_stage_wave<DH, BMAX>(lbase, static_cast<const T *>(a.v) + (size_t)(off + bs) * kvstride + hk * DH, kvstride,
                             B, lane);
  vmcnt_wait<0>();
  const T *vbuf = reinterpret_cast<const T *>(smem);

  // One group.  Inputs of group i (slot sl, FACache rows in o) landed; in
  // flight behind them: the stores of groups i-3 .. i-1 (CPT each, plus
  // possibly an LSE store: not counted, which only waits longer) and the
  // inputs of the groups after i.
  auto group = [&](int i, auto SL, ORow &o, ORow &onext, auto REFILL) {
    constexpr int sl = decltype(SL)::value;
    if (i >= 3) {
      const int behind = min(2, ngroups - 1 - i);
      if (behind == 2) vmcnt_wait<3 * L::CPT + 2 * (L::COPIES + L::LOADS)>();
      else if (behind == 1) vmcnt_wait<3 * L::CPT + L::COPIES + L::LOADS>();
      else vmcnt_wait<3 * L::CPT>();
    }
    const char *sp = smem + L::V + sl * L::SLOT;
    Frag<T> qf[1][DH / 32];
#pragma unroll
    for (int kd = 0; kd < DH / 32; ++kd) qtile_frag<T, DH>(qf[0][kd], reinterpret_cast<const T *>(sp), r16, kd, g);
    const float mc = *reinterpret_cast<const float *>(sp + L::TILE + 4 * r16);
    const float lc = *reinterpret_cast<const float *>(sp + L::TILE + 64 + 4 * r16);
    // The slot and the registers are refilled only after these reads.
    __builtin_amdgcn_s_waitcnt(0xC07F);                       // lgkmcnt(0)
    if (decltype(REFILL)::value || i + 3 < ngroups) {
      issue(i + 3, sl);
      load_o(onext, i + 3);
    }

    // Softmax over the block's keys, starting from the FACache state
    // (Algorithm 1: initialise with the cache): P*V accumulates from zero,
    // the cached O~ = (O~/l) * l joins it in the row-wise pass below.
    AttnState<1, DH> st;
    st.m[0] = mc * kLog2e;
    st.l[0] = g == 0 ? lc : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.o[0][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      if (32 * ks < B) attend_step_pre<T, 1, DH, BMAX>(st, qf, kf[ks], min(32, B - 32 * ks), vbuf, 32 * ks, a.scale_log2, lane);
    // The cached part decayed by exp2(m_c - m): l = lc * alpha + sum p.
    const float alpha = fast_exp2(mc * kLog2e - st.m[0]);
    const float lt = group_sum(st.l[0]), inv = 1.0f / lt;
    // l summed the cached lc * (all alphas of the steps) already; coef
    // multiplies (O~/l)_cache in the row-wise pass.
    const float coef = lc * alpha * inv;

    // P*V / l (fp16) and coef per row through LDS, then row-wise:
    // O = (O~/l)_cache * coef + P*V / l.
    char *op = smem + L::OUT;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int fe = OMap<DH>::feat(g, db, 0);
      const f32x4_t x = st.o[0][db] * inv;
      *reinterpret_cast<uint2 *>(op + r16 * L::ROWB + (((fe >> 3) ^ (r16 & L::SWZ)) << 4) + (fe & 7) * 2) =
          make_uint2(pack2(T{}, x[0], x[1]), pack2(T{}, x[2], x[3]));
    }
    if (g == 0) *reinterpret_cast<float *>(op + L::TILE + 4 * r16) = coef;
    if (a.lse && g == 0) a.lse[crow_of(i, r16)] = (st.m[0] + __log2f(lt)) * kLn2;
#pragma unroll
    for (int c = 0; c < L::CPT; ++c) {
      const int r = c * L::RPC + rw0;
      const uint4 pv = *reinterpret_cast<const uint4 *>(op + r * L::ROWB + ((piece ^ (r & L::SWZ)) << 4));
      const float cf = *reinterpret_cast<const float *>(op + L::TILE + 4 * r);
      const uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w}, ow[4] = {o[c].x, o[c].y, o[c].z, o[c].w};
      uint32_t res[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float2 x = unpack2(T{}, pw[q]), y = unpack2(T{}, ow[q]);
        res[q] = pack2(TO{}, fmaf(y.x, cf, x.x), fmaf(y.y, cf, x.y));
      }
      *reinterpret_cast<uint4 *>(static_cast<TO *>(a.out) + crow_of(i, r) * DH + piece * 8) =
          make_uint4(res[0], res[1], res[2], res[3]);
    }
  };
  // While three more groups follow each group, refills are unconditional (a
  // conditional refill makes the loop carry two definitions of a set, and
  // merging them costs a wait for everything in flight); the last eight or
  // fewer groups refill only what exists.
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  int i = 0;
  for (; i + 8 < ngroups; i += 6) {
    group(i, C0{}, o0, o3, std::true_type{});
    group(i + 1, C1{}, o1, o4, std::true_type{});
    group(i + 2, C2{}, o2, o5, std::true_type{});
    group(i + 3, C0{}, o3, o0, std::true_type{});
    group(i + 4, C1{}, o4, o1, std::true_type{});
    group(i + 5, C2{}, o5, o2, std::true_type{});
  }
  for (; i < ngroups; i += 6) {
    group(i, C0{}, o0, o3, std::false_type{});
    if (i + 1 < ngroups) group(i + 1, C1{}, o1, o4, std::false_type{});
    if (i + 2 < ngroups) group(i + 2, C2{}, o2, o5, std::false_type{});
    if (i + 3 < ngroups) group(i + 3, C0{}, o3, o0, std::false_type{});
    if (i + 4 < ngroups) group(i + 4, C1{}, o4, o1, std::false_type{});
    if (i + 5 < ngroups) group(i + 5, C2{}, o5, o2, std::false_type{});
  }
}

// ---------------------------------------------------------------------------
// Type A, streaming (16-bit caches): one workgroup of 4 waves per (sample,
// head, 32 block rows, key chunk).  K and V of 64-key tiles go global -> LDS
// row-wise through an NST-stage ring (up to NST-1 tiles in flight while one
// is used); wave w takes row block w & 1 and keys 32 (w >> 1) .. +31 of every
// tile.  The two waves of a row block merge through LDS at the end; the
// chunk's state goes to the workspace, or, when a.direct (every chunk is a
// whole sequence), O and LSE go out directly.
// K tile: key c's 16-byte piece p in slot p ^ kslot(c); the 16 keys of one
// A-operand read (8a + b + 4kb, a, b < 4) then hit distinct slots.
// ---------------------------------------------------------------------------
template <int DH, int NST_> struct StreamA {
  static constexpr int ROWB = DH * 2, PPR = ROWB / 16, RPC = 1024 / ROWB;
  static constexpr int TK = 64;                                 // keys per tile
  static constexpr int KT = TK * ROWB;                          // bytes of a K (or V) tile
  static constexpr int STAGE = 2 * KT;
  static constexpr int NST = NST_;
  static constexpr int QB = kRowsA * ROWB;                      // the 32 query rows
  static constexpr int BYTES = QB + NST * STAGE;
  static constexpr int CPW = STAGE / 1024 / 4;                  // copies per wave per tile
};

template <typename TO, int DH, int NST>
__global__ __launch_bounds__(256) void block_rows_stream_kernel(const SeqArgs sa, const AttnArgs a) {
  using T = f16_t;
  using S = StreamA<DH, NST>;
  using QT = QTile<T, DH>;
  constexpr int NDB = DH / 16, HDB = NDB / 2;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int mb = w & 1, kh = w >> 1;
  const int item = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int b = find_sample(sa.pre[1], sa.n, item);
  const int t = item - sa.pre[1][b];
  const int B = sa.be[b] - sa.bs[b], N = sa.len[b];
  const int nrg = (B + kRowsA - 1) / kRowsA;
  const int chunk = t / nrg, rg = t % nrg;
  const int key0 = chunk * a.split_keys;
  const int nkeys = min(a.split_keys, N - key0);
  const int ntiles = (nkeys + S::TK - 1) / S::TK;
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;
  const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const T *kbase = static_cast<const T *>(a.k) + (size_t)(sa.off[b] + key0) * kvstride + hk * DH;
  const T *vbase = static_cast<const T *>(a.v) + (size_t)(sa.off[b] + key0) * kvstride + hk * DH;
  const int rr = lane / S::PPR, slot = lane % S::PPR;             // row-wise lane: row rr (+ RPC q), slot

  // Tile tt into stage tt % NST: wave w does copies q = w, w+4, .. of the
  // tile's K then V rows (keys past the chunk repeat its last key).  The
  // tile's first key sets a scalar base; a full tile's per-lane byte offsets
  // are the same for every tile and computed once.
  constexpr int NJ = S::CPW / 2;
  uint32_t koff[NJ], voff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = (j * 4 + w) * S::RPC + rr;
    koff[j] = (uint32_t)(c * kvstride + ((slot ^ kslot(c, S::PPR)) << 3)) * 2u;
    voff[j] = (uint32_t)(c * kvstride + ((slot ^ (c & 3)) << 3)) * 2u;
  }
  auto issue = [&](int tt) {
    const uint32_t st = lbase + S::QB + (uint32_t)(tt % S::NST) * S::STAGE;
    const int k0 = tt * S::TK;
    const T *bk = kbase + (size_t)k0 * kvstride, *bv = vbase + (size_t)k0 * kvstride;
    if (k0 + S::TK <= nkeys) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int q = j * 4 + w;
        dma16_s(bk, koff[j], st + q * 1024);
        dma16_s(bv, voff[j], st + S::KT + q * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int q = j * 4 + w;
        const int c = q * S::RPC + rr;
        const uint32_t key = (uint32_t)(min(c, nkeys - 1 - k0) * kvstride);
        dma16_s(bk, (key + ((slot ^ kslot(c, S::PPR)) << 3)) * 2u, st + q * 1024);
        dma16_s(bv, (key + ((slot ^ (c & 3)) << 3)) * 2u, st + S::KT + q * 1024);
      }
    }
  };
  // The 32 query rows (QTile), rows past the block repeat its last row.
  {
    const int qrow0 = a.qmode == 0 ? sa.off[b] + sa.bs[b] : a.row_base + sa.pre[0][b];
#pragma unroll
    for (int it = 0; it < S::QB / 1024 / 4; ++it) {
      const int q = it * 4 + w;
      const int r = q * S::RPC + rr;
      const int rq = min(rg * kRowsA + r, B - 1);
      dma16(static_cast<const T *>(a.q) + ((size_t)(qrow0 + rq) * a.H + h) * DH + ((slot ^ (r & QT::SWZ)) << 3),
            lbase + q * 1024);
    }
  }
  // All stages start filling; the queries and tile 0 are waited for.
#pragma unroll
  for (int j = 0; j < S::NST; ++j)
    if (j < ntiles) issue(j);
  {
    const int behind = min(S::NST - 1, ntiles - 1);
    if (S::NST > 3 && behind == 3) vmcnt_wait<3 * S::CPW>();
    else if (S::NST > 2 && behind == 2) vmcnt_wait<2 * S::CPW>();
    else if (S::NST > 1 && behind == 1) vmcnt_wait<S::CPW>();
    else vmcnt_wait<0>();
  }
  lds_barrier();
  Frag<T> qf[1][DH / 32];
#pragma unroll
  for (int kd = 0; kd < DH / 32; ++kd) qtile_frag<T, DH>(qf[0][kd], reinterpret_cast<const T *>(smem), mb * 16 + r16, kd, g);

  AttnState<1, DH> st;
  state_init_empty(st);
  for (int tt = 0; tt < ntiles; ++tt) {
    const char *stg = smem + S::QB + (tt % S::NST) * S::STAGE;
    const int nv = max(0, min(32, nkeys - tt * S::TK - 32 * kh));
    if (nv > 0) {
      // S^T = K Q^T over this wave's 32 keys: A row r16 of key block kb is key
      // 32 kh + 8 (r16 >> 2) + 4 kb + (r16 & 3) (lane group g then holds keys
      // 8g..8g+7 of the step in the result).
      f32x4_t sc[2][1];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int c = 32 * kh + 8 * (r16 >> 2) + 4 * kb + (r16 & 3);
#pragma unroll
        for (int kd = 0; kd < DH / 32; ++kd) {
          const int e0 = 64 * (kd >> 1) + 16 * g + 8 * (kd & 1);
          Frag<T> kfr;
          frag_load(kfr, reinterpret_cast<const T *>(stg + c * S::ROWB + (((e0 >> 3) ^ kslot(c, S::PPR)) << 4)));
          mma16(sc[kb][0], kfr, qf[0][kd]);
        }
      }
      softmax_pv<T, 1, DH, S::TK>(st, sc, nv, reinterpret_cast<const T *>(stg + S::KT), 32 * kh, a.scale_log2, lane);
    }
    if (tt + 1 < ntiles) {
      // This wave's copies of tile tt+1 landed (later tiles may not have);
      // the barrier publishes it and frees stage tt for tile tt+NST (tiles
      // 0..NST-1 were issued before the loop).
      const int behind = min(S::NST - 2, ntiles - 2 - tt);
      if (S::NST > 3 && behind == 2) vmcnt_wait<2 * S::CPW>();
      else if (S::NST > 2 && behind == 1) vmcnt_wait<S::CPW>();
      else vmcnt_wait<0>();
      lds_barrier();
      if (tt + S::NST < ntiles) issue(tt + S::NST);
    }
  }

  // Merge the two waves of each row block: wave kh finalises feature blocks
  // [kh*HDB, (kh+1)*HDB) and hands the other half to its partner (w ^ 2).
  lds_barrier();                                               // ring reads done; reuse the LDS
  float *s_m = reinterpret_cast<float *>(smem);                 // [wave][16 rows]
  float *s_l = s_m + 4 * 16;
  f32x4_t *s_o = reinterpret_cast<f32x4_t *>(s_l + 4 * 16);    // [wave][HDB][lane]
  const float lw = group_sum(st.l[0]);
  if (g == 0) {
    s_m[w * 16 + r16] = st.m[0];
    s_l[w * 16 + r16] = lw;
  }
  // Feature blocks by compile-time index (a register array indexed by the
  // wave number would go to scratch memory); the branch is wave-uniform.
  auto hand_over = [&](auto KHC) {
    constexpr int KH = decltype(KHC)::value;
#pragma unroll
    for (int j = 0; j < HDB; ++j) s_o[(w * HDB + j) * 64 + lane] = st.o[0][(1 - KH) * HDB + j];
  };
  if (kh == 0) hand_over(std::integral_constant<int, 0>{});
  else hand_over(std::integral_constant<int, 1>{});
  lds_barrier();
  const int pw = w ^ 2;
  const float mo = s_m[pw * 16 + r16], lo = s_l[pw * 16 + r16];
  const float mx = fmaxf(st.m[0], mo);
  const float e_s = fast_exp2(st.m[0] - mx), e_o = fast_exp2(mo - mx);
  const float L = lw * e_s + lo * e_o, inv = 1.0f / L;
  const int r = rg * kRowsA + mb * 16 + r16;
  if (r >= B) return;
  const int orow = a.omode == 0 ? sa.off[b] + sa.bs[b] + r : a.row_base + sa.pre[0][b] + r;
  const size_t prow = ((size_t)(a.part_base + sa.pre[3][b]) + (size_t)chunk * B + r) * a.H + h;
  auto finish = [&](auto KHC) {
    constexpr int KH = decltype(KHC)::value;
#pragma unroll
    for (int j = 0; j < HDB; ++j) {
      const int db = KH * HDB + j;
      const f32x4_t o = (st.o[0][KH * HDB + j] * e_s + s_o[(pw * HDB + j) * 64 + lane] * e_o) * inv;
      if (a.direct) st4(static_cast<TO *>(a.out) + ((size_t)orow * a.H + h) * DH + OMap<DH>::feat(g, db, 0), o);
      else st4(static_cast<T *>(a.part_o) + prow * DH + OMap<DH>::feat(g, db, 0), o);
    }
  };
  if (kh == 0) finish(std::integral_constant<int, 0>{});
  else finish(std::integral_constant<int, 1>{});
  if (kh == 0 && g == 0) {
    if (a.direct) {
      if (a.lse) a.lse[(size_t)orow * a.H + h] = (mx + __log2f(L)) * kLn2;
    } else {
      a.part_ml[prow] = make_float2(mx, L);
    }
  }
}

// Type-A items only: the block rows' partial states (block step and
// DualCache).
template <typename T, typename TO, int DH>
__global__ __launch_bounds__(256) void block_rows_kernel(const SeqArgs sa, const AttnArgs a) {
  extern __shared__ __align__(16) char smem[];
  block_rows_partial<T, TO, DH>(sa, a, blockIdx.x / a.H, blockIdx.x % a.H, smem);
}

// ---------------------------------------------------------------------------
// Merge of the type-A partial states of one (block row, head) per wave: each
// lane owns DH/64 consecutive features.  Chunks are read 8 at a time, every
// load of a batch before any use (one memory round trip for <= 8 chunks).
// ---------------------------------------------------------------------------
template <typename T, typename TO, int DH>
__device__ void merge_wave(const SeqArgs &sa, const AttnArgs &a, int M, int wid) {
  constexpr int FPL = DH / 64, CB = 8;
  const int lane = threadIdx.x & 63;
  if (wid >= M * a.H) return;
  const int m = wid / a.H, h = wid % a.H;
  const int b = find_sample(sa.pre[0], sa.n, m);
  const int r = m - sa.pre[0][b];
  const int B = sa.be[b] - sa.bs[b];
  const int nch = (sa.len[b] + a.split_keys - 1) / a.split_keys;
  const size_t pb = (size_t)(a.part_base + sa.pre[3][b] + r) * a.H + h;   // chunk c at pb + c*B*H
  const size_t cstride = (size_t)B * a.H;
  const T *part_o = static_cast<const T *>(a.part_o);

  float mx = -INFINITY, lsum = 0.f;
  float acc[FPL] = {};
  for (int c0 = 0; c0 < nch; c0 += CB) {
    float2 ml[CB];
    float v[CB][FPL];
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const size_t prow = pb + (size_t)min(c0 + j, nch - 1) * cstride;
      ml[j] = a.part_ml[prow];
      const T *src = part_o + prow * DH + lane * FPL;
      if constexpr (FPL == 2 && sizeof(T) == 2) {
        const float2 p2 = unpack2(T{}, *reinterpret_cast<const uint32_t *>(src));
        v[j][0] = p2.x;
        v[j][1] = p2.y;
      } else {
#pragma unroll
        for (int k = 0; k < FPL; ++k) v[j][k] = to_f32(src[k]);
      }
    }
    float bm = mx;
#pragma unroll
    for (int j = 0; j < CB; ++j)
      if (c0 + j < nch) bm = fmaxf(bm, ml[j].x);
    const float sc = fast_exp2(mx - bm);
    lsum *= sc;
#pragma unroll
    for (int k = 0; k < FPL; ++k) acc[k] *= sc;
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const float e = c0 + j < nch ? fast_exp2(ml[j].x - bm) * ml[j].y : 0.f;
      lsum += e;
#pragma unroll
      for (int k = 0; k < FPL; ++k) acc[k] = fmaf(e, v[j][k], acc[k]);
    }
    mx = bm;
  }
  const int orow = a.omode == 0 ? sa.off[b] + sa.bs[b] + r : a.row_base + m;
  const float inv = 1.0f / lsum;
  TO *out = static_cast<TO *>(a.out) + ((size_t)orow * a.H + h) * DH + lane * FPL;
  if constexpr (FPL == 2 && sizeof(TO) == 2) {
    *reinterpret_cast<uint32_t *>(out) = pack2(TO{}, acc[0] * inv, acc[1] * inv);
  } else {
#pragma unroll
    for (int k = 0; k < FPL; ++k) out[k] = from_f32<TO>(acc[k] * inv);
  }
  if (a.lse && lane == 0) a.lse[(size_t)orow * a.H + h] = (mx + __log2f(lsum)) * kLn2;
}

// Block step, small launches: type-A items (the block rows' partials) and
// type-B items (invariant rows) in one launch, their latencies overlapping;
// the merge of the partials follows as its own launch.  The first nA
// workgroups are type A.
template <typename T, typename TO, int DH, int BMAX>
__global__ __launch_bounds__(256) void attn_ab_kernel(const SeqArgs sa, const AttnArgs a, int nA) {
  extern __shared__ __align__(16) char smem[];
  if ((int)blockIdx.x < nA) {
    block_rows_partial<T, TO, DH>(sa, a, blockIdx.x / a.H, blockIdx.x % a.H, smem);
    return;
  }
  const int j = blockIdx.x - nA;
  invariant_rows<T, TO, DH, BMAX, 1>(sa, a, j / a.H, j % a.H, smem);
}

// DualCache: the merge alone, 4 (row, head) pairs per workgroup.
template <typename T, typename TO, int DH>
__global__ __launch_bounds__(256) void merge_kernel(const SeqArgs sa, const AttnArgs a, int M) {
  merge_wave<T, TO, DH>(sa, a, M, blockIdx.x * 4 + (threadIdx.x >> 6));
}

// Block step, after the type-A kernel: the first ceil(M*H/4) workgroups merge
// the block rows' partials, the rest are type-B items (invariant rows).  Both
// only read what earlier kernels wrote, so no workgroup waits for another.
// BMAX: staged block keys (32, 64 or 128 >= every block of the launch).
template <typename T, typename TO, int DH, int BMAX>
__global__ __launch_bounds__(256) void invariant_rows_kernel(const SeqArgs sa, const AttnArgs a, int M) {
  extern __shared__ __align__(16) char smem[];
  const int nmw = (M * a.H + 3) / 4;
  if ((int)blockIdx.x < nmw) {
    merge_wave<T, TO, DH>(sa, a, M, blockIdx.x * 4 + (threadIdx.x >> 6));
    return;
  }
  const int j = blockIdx.x - nmw;
  invariant_rows<T, TO, DH, BMAX, 1>(sa, a, j / a.H, j % a.H, smem);
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
        store_row<T, DH>(static_cast<T *>(a.o_w) + crow * DH, st.o[0], 1.0f / lt, g);
      }
    }
    for (int k0 = seg_lo[sgi]; k0 < seg_hi[sgi]; k0 += TK) {
      const int nk = min(TK, seg_hi[sgi] - k0);
      __syncthreads();
      vtile_stage<T, DH, TK, 256>(vbuf, vb + (size_t)k0 * kvstride, kvstride, nk, tid);
      vtile_wait();
      __syncthreads();
      for (int c0 = 0; c0 < nk; c0 += 32)
        attend_step<T, MB, DH, TK>(st, qf, kb + (size_t)(k0 + c0) * kvstride, kvstride, min(32, nk - c0), vbuf, c0,
                                   a.scale_log2, lane);
    }
  }
  const float lt = group_sum(st.l[0]);
  if (tvalid) {
    store_row<TO, DH>(static_cast<TO *>(a.out) + crow * DH, st.o[0], 1.0f / lt, g);
    if (a.lse && g == 0) a.lse[crow] = (st.m[0] + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Refresh, streaming (16-bit caches): one workgroup of 4 waves per (sample,
// head, 64 * MB rows); wave w owns MB row blocks (rows 16 MB w ..) and takes
// every key, so each K or V fragment read from LDS feeds MB matrix products.
// K and V of 64-key tiles arrive row-wise (the load unit's full-rate
// pattern) through an NST-stage ring, as in block_rows_stream_kernel.  Key
// order: the invariant keys [0, bs) and [be, N), then the block's [bs, be)
// (each segment in its own tiles, the last one ragged); the state after the
// last invariant tile is the FACache snapshot of the invariant rows
// (LaCache Section 3.3.3: the cache holds the online-softmax state over the
// invariant keys only).
// ---------------------------------------------------------------------------
template <int DH, int NST_> struct StreamR {
  static constexpr int ROWB = DH * 2, PPR = ROWB / 16, RPC = 1024 / ROWB;
  static constexpr int TK = 64;                                 // keys per tile
  static constexpr int KT = TK * ROWB;                          // bytes of a K (or V) tile
  static constexpr int STAGE = 2 * KT;
  static constexpr int NST = NST_;
  static constexpr int BYTES = NST * STAGE;
  static constexpr int CPW = STAGE / 1024 / 4;                  // copies per wave per tile
};

template <typename TO, int DH, int MB, int NST>
__global__ __launch_bounds__(256) void refresh_stream_kernel(const SeqArgs sa, const AttnArgs a) {
  using T = f16_t;
  using S = StreamR<DH, NST>;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int item = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int b = find_sample(sa.pre[1], sa.n, item);
  const int tile = item - sa.pre[1][b];
  const int bs = sa.bs[b], be = sa.be[b], N = sa.len[b], off = sa.off[b];
  const int hk = h / (a.H / a.Hkv);
  const size_t kvstride = (size_t)a.Hkv * DH;
  const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const T *kb = static_cast<const T *>(a.k) + (size_t)off * kvstride + hk * DH;
  const T *vb = static_cast<const T *>(a.v) + (size_t)off * kvstride + hk * DH;
  const int rr = lane / S::PPR, slot = lane % S::PPR;             // row-wise lane: row rr (+ RPC q), slot

  // Tiles of the three key segments; tile tt covers keys k0 .. k0 + nk - 1.
  const int nt0 = (bs + S::TK - 1) / S::TK, nt1 = (N - be + S::TK - 1) / S::TK;
  const int ntU = nt0 + nt1, ntiles = ntU + (be - bs + S::TK - 1) / S::TK;
  // (Values selected, not references: a choice between references to the
  // bounds would be compiled as pointers into scratch memory.)
  auto tile_keys = [=](int tt, int &k0, int &nk) {
    const int seg_base = tt < nt0 ? 0 : (tt < ntU ? be : bs);
    const int seg_end = tt < nt0 ? bs : (tt < ntU ? N : be);
    const int seg_t0 = tt < nt0 ? 0 : (tt < ntU ? nt0 : ntU);
    k0 = seg_base + (tt - seg_t0) * S::TK;
    nk = min(S::TK, seg_end - k0);
  };
  // Tile tt into stage tt % NST: wave w does copies q = w, w+4, .. of the
  // tile's K then V rows (keys past the tile repeat its last key).  The
  // tile's first key sets a scalar base; a full tile's per-lane byte offsets
  // are the same for every tile and computed once.
  constexpr int NJ = S::CPW / 2;
  uint32_t koff[NJ], voff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = (j * 4 + w) * S::RPC + rr;
    koff[j] = (uint32_t)(c * kvstride + ((slot ^ kslot(c, S::PPR)) << 3)) * 2u;
    voff[j] = (uint32_t)(c * kvstride + ((slot ^ (c & 3)) << 3)) * 2u;
  }
  auto issue = [&](int tt) {
    int k0, nk;
    tile_keys(tt, k0, nk);
    const uint32_t st = lbase + (uint32_t)(tt % S::NST) * S::STAGE;
    const T *bk = kb + (size_t)k0 * kvstride, *bv = vb + (size_t)k0 * kvstride;
    if (nk == S::TK) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int q = j * 4 + w;
        dma16_s(bk, koff[j], st + q * 1024);
        dma16_s(bv, voff[j], st + S::KT + q * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int q = j * 4 + w;
        const int c = q * S::RPC + rr;
        const uint32_t key = (uint32_t)(min(c, nk - 1) * kvstride);
        dma16_s(bk, (key + ((slot ^ kslot(c, S::PPR)) << 3)) * 2u, st + q * 1024);
        dma16_s(bv, (key + ((slot ^ (c & 3)) << 3)) * 2u, st + S::KT + q * 1024);
      }
    }
  };

  // This wave's query rows (rows past the sample repeat its last row; their
  // results are dropped).
  const T *qrow[MB];
  int trow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    trow[mb] = tile * (64 * MB) + (w * MB + mb) * 16 + r16;
    qrow[mb] = static_cast<const T *>(a.q) + ((size_t)(off + min(trow[mb], N - 1)) * a.H + h) * DH;
  }
  Frag<T> qf[MB][DH / 32];
  load_q<T, MB, DH>(qf, qrow, g);
  // All stages start filling; the queries and tile 0 are waited for.
#pragma unroll
  for (int j = 0; j < S::NST; ++j)
    if (j < ntiles) issue(j);
  {
    const int behind = min(S::NST - 1, ntiles - 1);
    if (S::NST > 3 && behind == 3) vmcnt_wait<3 * S::CPW>();
    else if (S::NST > 2 && behind == 2) vmcnt_wait<2 * S::CPW>();
    else if (S::NST > 1 && behind == 1) vmcnt_wait<S::CPW>();
    else vmcnt_wait<0>();
  }
  lds_barrier();

  AttnState<MB, DH> st;
  state_init_empty(st);
  // One tile (stage STG = tt % NST, a compile-time constant: the loop below
  // is unrolled by NST, so the stage's LDS offsets fold into the reads).
  auto one_tile = [&](const int tt, auto STGC) {
    constexpr int STG = decltype(STGC)::value;
    const char *stg = smem + STG * S::STAGE;
    int k0, nk;
    tile_keys(tt, k0, nk);
    // S^T = K Q^T over the tile's 64 keys (both halves before the softmax:
    // eight independent accumulation chains): A row r16 of key block kb of
    // half ks is key 32 ks + 8 (r16 >> 2) + 4 kb + (r16 & 3) of the tile
    // (keys past nk are copies of its last key, masked in the softmax).
    f32x4_t sc[2][2][MB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) sc[ks][kb2][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int c = 32 * ks + 8 * (r16 >> 2) + 4 * kb2 + (r16 & 3);
#pragma unroll
        for (int kd = 0; kd < DH / 32; ++kd) {
          const int e0 = 64 * (kd >> 1) + 16 * g + 8 * (kd & 1);
          Frag<T> kfr;
          frag_load(kfr, reinterpret_cast<const T *>(stg + c * S::ROWB + (((e0 >> 3) ^ kslot(c, S::PPR)) << 4)));
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) mma16(sc[ks][kb2][mb], kfr, qf[mb][kd]);
        }
      }
    softmax_pv64<T, MB, DH, S::TK>(st, sc, nk, reinterpret_cast<const T *>(stg + S::KT), a.scale_log2, lane);
    if (tt == ntU - 1) {
      // FACache snapshot of the invariant rows: (m, l, O~/l) over the
      // invariant keys.  Its stores join the copies in flight; vector memory
      // operations complete in issue order, so the waits below (which count
      // copies only) wait at most a little longer, once.
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int t = trow[mb];
        const size_t crow = (size_t)(off + min(t, N - 1)) * a.H + h;
        const float ls = group_sum(st.l[mb]);
        if (t < N && (t < bs || t >= be)) {
          if (g == 0) {
            a.m_w[crow] = st.m[mb] * kLn2;
            a.l_w[crow] = ls;
          }
          store_row<T, DH>(static_cast<T *>(a.o_w) + crow * DH, st.o[mb], 1.0f / ls, g);
        }
      }
    }
    if (tt + 1 < ntiles) {
      // This wave's copies of tile tt+1 landed (later tiles may not have);
      // the barrier publishes it and frees stage tt for tile tt+NST.
      const int behind = min(S::NST - 2, ntiles - 2 - tt);
      if (S::NST > 3 && behind == 2) vmcnt_wait<2 * S::CPW>();
      else if (S::NST > 2 && behind == 1) vmcnt_wait<S::CPW>();
      else vmcnt_wait<0>();
      lds_barrier();
      if (tt + S::NST < ntiles) issue(tt + S::NST);
    }
  };
  static_assert(S::NST == 2, "the tile loop is unrolled by two stages");
  for (int tt = 0; tt < ntiles; tt += 2) {
    one_tile(tt, std::integral_constant<int, 0>{});
    if (tt + 1 < ntiles) one_tile(tt + 1, std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = trow[mb];
    const size_t crow = (size_t)(off + min(t, N - 1)) * a.H + h;
    const float lt = group_sum(st.l[mb]);
    if (t < N) {
      store_row<TO, DH>(static_cast<TO *>(a.out) + crow * DH, st.o[mb], 1.0f / lt, g);
      if (a.lse && g == 0) a.lse[crow] = (st.m[mb] + __log2f(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// type A: query rows + key tile, then the state merge
template <typename T, int DH> constexpr size_t block_rows_smem() {
  constexpr size_t tile_a = (size_t)kRowsA * DH * sizeof(T) + VTile<T, DH, kTileA>::kBytes +
                            (sizeof(T) == 2 ? (size_t)kTileA * DH * sizeof(T) : 0);
  constexpr size_t merge_a = merge_a_bytes<DH>();
  return tile_a > merge_a ? tile_a : merge_a;
}
// type B: the block's keys
// type B: the block's V (and, 16-bit, its K)
template <typename T, int DH, int BMAX> constexpr size_t invariant_rows_smem() {
  return VTile<T, DH, BMAX>::kBytes + (sizeof(T) == 2 ? (size_t)BMAX * DH * sizeof(T) : 0);
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

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

hipError_t launch_block_rows(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks, hipStream_t s,
                             const LaunchEvents &ev) {
  if (n_blocks <= 0) return hipSuccess;
  if (dt == kBF16 && a.direct) {
    // A 4-stage ring (three tiles of lookahead) holds one workgroup per CU.
    // When the launch fits on the chip at two per CU but not at one, a
    // 2-stage ring runs it in one round instead of two.
    const int cus = device_cus();
    const bool two = n_blocks > cus && n_blocks <= 2 * cus;
    if (dh == 128) {
      if (two) lc_launch<block_rows_stream_kernel<bf16_t, 128, 2>>(dim3(n_blocks), dim3(256), StreamA<128, 2>::BYTES, s, ev, sa, a);
      else lc_launch<block_rows_stream_kernel<bf16_t, 128, 4>>(dim3(n_blocks), dim3(256), StreamA<128, 4>::BYTES, s, ev, sa, a);
    } else {
      if (two) lc_launch<block_rows_stream_kernel<bf16_t, 64, 2>>(dim3(n_blocks), dim3(256), StreamA<64, 2>::BYTES, s, ev, sa, a);
      else lc_launch<block_rows_stream_kernel<bf16_t, 64, 4>>(dim3(n_blocks), dim3(256), StreamA<64, 4>::BYTES, s, ev, sa, a);
    }
    return hipGetLastError();
  }
  LC_DISPATCH(dt, dh, (lc_launch<block_rows_kernel<T, TO, DH>>(dim3(n_blocks), dim3(256), block_rows_smem<T, DH>(), s, ev, sa, a)));
  return hipGetLastError();
}

template <typename T, int DH, int BM> constexpr size_t attn_ab_smem() {
  return block_rows_smem<T, DH>() > invariant_rows_smem<T, DH, BM>() ? block_rows_smem<T, DH>()
                                                                     : invariant_rows_smem<T, DH, BM>();
}

namespace {
int block_max(const SeqArgs &sa) {
  int bmax = 0;
  for (int i = 0; i < sa.n; ++i) bmax = bmax > sa.be[i] - sa.bs[i] ? bmax : sa.be[i] - sa.bs[i];
  return bmax;
}
// Workgroups of one combined launch resident on one CU (occupancy query, cached).
template <typename K> int resident_per_cu(K kernel, size_t smem) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(kernel), 256, smem) !=
          hipSuccess || n < 1)
    n = 1;
  return n;
}
}  // namespace

// Workgroups of a combined launch resident on the whole chip at once.
int attn_ab_capacity(DType dt, int dh, const SeqArgs &sa) {
  const int bmax = block_max(sa);
  static int cap[2][2][3] = {};                      // [fp32][dh == 128][block size class]
  const int fi = dt != kBF16, di = dh == 128, bi = bmax <= 32 ? 0 : bmax <= 64 ? 1 : 2;
  int &c = cap[fi][di][bi];
  if (c == 0) {
#define LC_CAP(BM) LC_DISPATCH(dt, dh, (c = resident_per_cu(attn_ab_kernel<T, TO, DH, BM>, attn_ab_smem<T, DH, BM>())))
    if (bi == 0) LC_CAP(32);
    else if (bi == 1) LC_CAP(64);
    else LC_CAP(128);
#undef LC_CAP
  }
  return c * device_cus();
}

hipError_t launch_attn_ab(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int nA, int nB, hipStream_t s,
                          const LaunchEvents &ev) {
  if (nA + nB <= 0) return hipSuccess;
  const int bmax = block_max(sa);
#define LC_AB(BM) \
  LC_DISPATCH(dt, dh, (lc_launch<attn_ab_kernel<T, TO, DH, BM>>(dim3(nA + nB), dim3(256), attn_ab_smem<T, DH, BM>(), s, ev, sa, a, nA)))
  if (bmax <= 32) LC_AB(32);
  else if (bmax <= 64) LC_AB(64);
  else LC_AB(128);
#undef LC_AB
  return hipGetLastError();
}


hipError_t launch_invariant_stream(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, hipStream_t s,
                                   const LaunchEvents &ev) {
  constexpr int waves = 4;
  const int nit = sa.pre[2][sa.n];
  if (nit <= 0) return hipSuccess;
  int bmax = 0;
  for (int i = 0; i < sa.n; ++i) bmax = bmax > sa.be[i] - sa.bs[i] ? bmax : sa.be[i] - sa.bs[i];
  if (bmax > kStreamMaxBlock) return hipErrorInvalidValue;
  if (dt != kBF16) return hipErrorInvalidValue;
  // Eight dies, each with at most ceil(nit / 8) segments x H waves.
  const unsigned grid = 8u * (unsigned)(((nit + 7) / 8 * a.H + waves - 1) / waves);
#define LC_STR(DH, NK, NW)                                                                                       \
  lc_launch<invariant_stream_kernel<bf16_t, DH, NK, NW>>(dim3(grid), dim3(64 * NW), NW * StreamLds<DH, NK>::BYTES, s, \
                                                         ev, sa, a)
#define LC_STR_W(DH, NK) LC_STR(DH, NK, waves)
  if (dh == 128) {
    if (bmax <= 32) LC_STR_W(128, 1);
    else LC_STR_W(128, 2);
  } else {
    if (bmax <= 32) LC_STR_W(64, 1);
    else LC_STR_W(64, 2);
  }
#undef LC_STR_W
#undef LC_STR
  return hipGetLastError();
}

hipError_t launch_invariant_rows(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks, int M,
                                 hipStream_t s, const LaunchEvents &ev) {
  const int grid = (M * a.H + 3) / 4 + n_blocks;
  if (grid <= 0) return hipSuccess;
  int bmax = 0;
  for (int i = 0; i < sa.n; ++i) bmax = bmax > sa.be[i] - sa.bs[i] ? bmax : sa.be[i] - sa.bs[i];
#define LC_INV(BM) \
  LC_DISPATCH(dt, dh, (lc_launch<invariant_rows_kernel<T, TO, DH, BM>>(dim3(grid), dim3(256), invariant_rows_smem<T, DH, BM>(), s, ev, sa, a, M)))
  if (bmax <= 32) LC_INV(32);
  else if (bmax <= 64) LC_INV(64);
  else LC_INV(128);
#undef LC_INV
  return hipGetLastError();
}

hipError_t launch_merge(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int M, hipStream_t s,
                        const LaunchEvents &ev) {
  const int waves = M * a.H;
  if (waves <= 0) return hipSuccess;
  LC_DISPATCH(dt, dh, (lc_launch<merge_kernel<T, TO, DH>>(dim3((waves + 3) / 4), dim3(256), 0, s, ev, sa, a, M)));
  return hipGetLastError();
}

hipError_t launch_refresh_stream(int dh, int mb, const SeqArgs &sa, const AttnArgs &a, int n_blocks, hipStream_t s,
                                 const LaunchEvents &ev) {
  if (n_blocks <= 0) return hipSuccess;
  if (mb != 1 && mb != 2) return hipErrorInvalidValue;
#define LC_RS(DHV, MBV) \
  lc_launch<refresh_stream_kernel<bf16_t, DHV, MBV, 2>>(dim3(n_blocks), dim3(256), StreamR<DHV, 2>::BYTES, s, ev, sa, a)
  if (dh == 128) {
    if (mb == 2) LC_RS(128, 2);
    else LC_RS(128, 1);
  } else if (dh == 64) {
    if (mb == 2) LC_RS(64, 2);
    else LC_RS(64, 1);
  } else {
    return hipErrorInvalidValue;
  }
#undef LC_RS
  return hipGetLastError();
}

hipError_t launch_refresh_attn(DType dt, int dh, const SeqArgs &sa, const AttnArgs &a, int n_blocks,
                               hipStream_t s, const LaunchEvents &ev) {
  if (n_blocks <= 0) return hipSuccess;
  LC_DISPATCH(dt, dh, (lc_launch<refresh_attn_kernel<T, TO, DH>>(dim3(n_blocks), dim3(256), refresh_smem<T, DH>(), s, ev, sa, a)));
  return hipGetLastError();
}

hipError_t setup_kernel_attributes() {
  hipError_t e = hipSuccess;
#define LC_ATTR(K, BYTES)                                                                        \
  if (e == hipSuccess)                                                                           \
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(K), hipFuncAttributeMaxDynamicSharedMemorySize, \
                            (int)(BYTES));
#define LC_ATTR_AB(BM)                                                                          \
  LC_ATTR((attn_ab_kernel<f16_t, bf16_t, 128, BM>), (attn_ab_smem<f16_t, 128, BM>()));              \
  LC_ATTR((attn_ab_kernel<f16_t, bf16_t, 64, BM>), (attn_ab_smem<f16_t, 64, BM>()));                \
  LC_ATTR((attn_ab_kernel<float, float, 128, BM>), (attn_ab_smem<float, 128, BM>()));               \
  LC_ATTR((attn_ab_kernel<float, float, 64, BM>), (attn_ab_smem<float, 64, BM>()));
  LC_ATTR_AB(32)
  LC_ATTR_AB(64)
  LC_ATTR_AB(128)
#undef LC_ATTR_AB
#define LC_ATTR_INV(BM)                                                   \
  LC_ATTR((invariant_rows_kernel<f16_t, bf16_t, 128, BM>), (invariant_rows_smem<f16_t, 128, BM>())); \
  LC_ATTR((invariant_rows_kernel<f16_t, bf16_t, 64, BM>), (invariant_rows_smem<f16_t, 64, BM>()));   \
  LC_ATTR((invariant_rows_kernel<float, float, 128, BM>), (invariant_rows_smem<float, 128, BM>()));  \
  LC_ATTR((invariant_rows_kernel<float, float, 64, BM>), (invariant_rows_smem<float, 64, BM>()));
  LC_ATTR_INV(32)
  LC_ATTR_INV(64)
  LC_ATTR_INV(128)
#undef LC_ATTR_INV
  LC_ATTR((block_rows_kernel<f16_t, bf16_t, 128>), (block_rows_smem<f16_t, 128>()));
  LC_ATTR((block_rows_kernel<f16_t, bf16_t, 64>), (block_rows_smem<f16_t, 64>()));
  LC_ATTR((block_rows_kernel<float, float, 128>), (block_rows_smem<float, 128>()));
  LC_ATTR((block_rows_kernel<float, float, 64>), (block_rows_smem<float, 64>()));
  LC_ATTR((refresh_attn_kernel<f16_t, bf16_t, 128>), (refresh_smem<f16_t, 128>()));
  LC_ATTR((refresh_attn_kernel<f16_t, bf16_t, 64>), (refresh_smem<f16_t, 64>()));
  LC_ATTR((refresh_attn_kernel<float, float, 128>), (refresh_smem<float, 128>()));
  LC_ATTR((refresh_attn_kernel<float, float, 64>), (refresh_smem<float, 64>()));
  LC_ATTR((refresh_stream_kernel<bf16_t, 128, 2, 2>), (StreamR<128, 2>::BYTES));
  LC_ATTR((refresh_stream_kernel<bf16_t, 64, 2, 2>), (StreamR<64, 2>::BYTES));
  LC_ATTR((refresh_stream_kernel<bf16_t, 128, 1, 2>), (StreamR<128, 2>::BYTES));
  LC_ATTR((refresh_stream_kernel<bf16_t, 64, 1, 2>), (StreamR<64, 2>::BYTES));
  LC_ATTR((block_rows_stream_kernel<bf16_t, 128, 4>), (StreamA<128, 4>::BYTES));
  LC_ATTR((block_rows_stream_kernel<bf16_t, 64, 4>), (StreamA<64, 4>::BYTES));
  LC_ATTR((block_rows_stream_kernel<bf16_t, 128, 2>), (StreamA<128, 2>::BYTES));
  LC_ATTR((block_rows_stream_kernel<bf16_t, 64, 2>), (StreamA<64, 2>::BYTES));
#define LC_ATTR_IS(DH, NK) \
  LC_ATTR((invariant_stream_kernel<bf16_t, DH, NK, 4>), (4 * StreamLds<DH, NK>::BYTES));
  LC_ATTR_IS(128, 1)
  LC_ATTR_IS(128, 2)
  LC_ATTR_IS(64, 1)
  LC_ATTR_IS(64, 2)
#undef LC_ATTR_IS
#undef LC_ATTR
  return e;
}

}  // namespace lc
