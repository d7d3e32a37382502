// Fused first-layer token-wise operators for the tokens of one launch
// (LaCache Section 3.3.2, Eq. (1)): embedding gather (EmbedCache write),
// RMSNorm, the QKV projection on MFMA, RoPE and the Q/K/V cache write, in one
// kernel.  Only the normalised activations' bf16 copy lives in registers; no
// intermediate touches HBM (the Flash-dLLM article's single-write argument).
//
// Tiling.  A workgroup owns a tile of 32 tokens x (3 x 16) output features
// and 8 waves split the contraction over d_model; their partial sums meet in
// LDS.  A 16-feature column block holds 8 RoPE pairs: features p..p+7 and
// p+d_h/2..p+d_h/2+7 of one head, so a rotation partner sits 8 lanes away in
// the MFMA result and is exchanged with a lane shuffle.  Each lane reads 16
// contiguous bytes of a weight row per step, every weight byte is read once
// per token tile, and for the small token counts of an inner step the grid
// is d_model-wide enough (F/48 tiles) to keep every CU streaming weights.
//
// RMSNorm is folded into the projection: the MFMA consumes gamma * H and the
// fp32 result is scaled per token by 1/sqrt(mean(H^2) + eps), whose sum of
// squares is accumulated from the same loads.  For bf16 parameters the
// product gamma * H (at most 16 significant bits) is split into two bf16
// terms, hi + lo, each multiplied on the MFMA, so the projection carries no
// rounding of its activations; W itself is exact in bf16.  Q, K and V are
// written in the cache type (fp16 for bf16 parameters, fp32 for fp32).

#include "internal.h"

namespace lc {

// NG > 0: the wave's contraction range is exactly NG groups of U steps and
// the pipeline is unrolled at compile time; NG == 0: runtime group count.
template <typename T, typename TC, int NB, int KW, bool SPLIT, int U, int NG>
__global__ __launch_bounds__(64 * KW) void qkv_fused_kernel(const SeqArgs sa, const QkvArgs a) {
  constexpr int MB = 2;                    // 16-row blocks per tile
  constexpr int BM = 16 * MB;
  __shared__ int s_id[BM], s_dst[BM], s_pos[BM];
  __shared__ float s_ssq[KW][BM];
  __shared__ f32x4_t s_red[KW][MB][NB][64];
  __shared__ __align__(16) T s_gamma[kQkvMaxD];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int dh = a.dh, D = a.D;
  const int cbh = dh / 16;                 // column blocks per head
  const int ncb = (a.H + 2 * a.Hkv) * cbh;
  const int cb0 = blockIdx.x * NB;
  const int m0 = blockIdx.y * BM;

  const T *E = static_cast<const T *>(a.E);
  const T *W = static_cast<const T *>(a.W);
  // Column blocks past the last feature read row 0 and are dropped in the
  // epilogue; rows without a valid token read row 0 and are zeroed there, so
  // every load of the main loop is unconditional.
  const T *brow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int cb = min(cb0 + nb, ncb - 1);
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    const int wrow = hh * dh + (r16 < 8 ? p0 + r16 : dh / 2 + p0 + (r16 - 8));
    brow[nb] = W + (size_t)wrow * D;
  }
  const T *arow[MB];

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t ssq[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) ssq[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Contraction steps of 32, in groups of U steps (U divides the step count).
  // The waves interleave: group i of wave w is steps (i*KW + w)*U .. +U-1, so
  // at any time the workgroup reads one contiguous KW*U*64-byte stretch of
  // each weight row (whole DRAM pages) rather than KW scattered pieces.
  const int kper = D / KW;
  const int ngroups = kper / (32 * U);
  auto kstep = [&](int grp, int u) { return ((grp * KW + w) * U + u) * 32; };

  struct Group {
    Frag<T> w[U][NB], e[U][MB];
  };
  auto load_w = [&](Group &G, int grp) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) frag_load(G.w[u][nb], brow[nb] + kstep(grp, u) + 8 * g);
  };
  auto load_e = [&](Group &G, int grp) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) frag_load(G.e[u][mb], arow[mb] + kstep(grp, u) + 8 * g);
  };
  auto load_group = [&](Group &G, int grp) {
    load_w(G, grp);
    load_e(G, grp);
  };
  auto compute_group = [&](const Group &G, int grp) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Frag<T> gm;
      frag_load(gm, s_gamma + kstep(grp, u) + 8 * g);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // Sum of squares on the matrix core: E_rows * E_rows^T, whose diagonal
        // is each row's sum of x^2 (exact products, fp32 accumulation).
        mma16(ssq[mb], G.e[u][mb], G.e[u][mb]);
        Frag<T> af, al;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float y = frag_get(G.e[u][mb], i) * frag_get(gm, i);
          frag_set(af, i, y);
          if constexpr (SPLIT) frag_set(al, i, y - frag_get(af, i));
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          mma16(acc[mb][nb], af, G.w[u][nb]);
          if constexpr (SPLIT) mma16(acc[mb][nb], al, G.w[u][nb]);
        }
      }
    }
  };

  // The weights of the first groups go out before anything else: their
  // addresses do not depend on the tokens.
  Group gbuf[3];
  load_w(gbuf[0], 0);
  if constexpr (NG > 1) load_w(gbuf[1], 1);

  // Prologue, one memory round trip: the RMSNorm gain (staged in LDS, read
  // per step) and the tile's token ids are loaded together.  When the tile
  // lies within one sample (always for one sample per launch) the block-table
  // lookup is uniform; otherwise each token searches the table.
  constexpr int GMAX = kQkvMaxD * (int)sizeof(T) / 16 / (64 * KW);   // gain pieces per thread, at most
  static_assert(GMAX <= 4, "gain staging registers");
  const int gpieces = D * (int)sizeof(T) / 16;
  const uint4 *gsrc = static_cast<const uint4 *>(a.gamma);
  const int mc = min(m0 + min(tid, BM - 1), a.M - 1);
  const int b0 = find_sample(sa.pre[0], sa.n, m0);
  int tdst, tpos;
  if (min(m0 + BM, a.M) <= sa.pre[0][b0 + 1]) {          // uniform
    const int local = mc - sa.pre[0][b0];
    tdst = a.mode == 0 ? sa.off[b0] + sa.bs[b0] + local : sa.off[b0] + local;
    tpos = a.mode == 0 ? sa.bs[b0] + local : local;
  } else {
    const int tb = find_sample(sa.pre[0], sa.n, mc);
    const int local = mc - sa.pre[0][tb];
    tdst = a.mode == 0 ? sa.off[tb] + sa.bs[tb] + local : sa.off[tb] + local;
    tpos = a.mode == 0 ? sa.bs[tb] + local : local;
  }
  const int tid_raw = a.ids[a.mode == 0 ? a.ids_base + mc : tdst];
  uint4 gv0 = gsrc[min(tid, gpieces - 1)], gv1 = gv0, gv2 = gv0, gv3 = gv0;
  if constexpr (GMAX > 1) gv1 = gsrc[min(tid + 64 * KW, gpieces - 1)];
  if constexpr (GMAX > 2) gv2 = gsrc[min(tid + 2 * 64 * KW, gpieces - 1)];
  if constexpr (GMAX > 3) gv3 = gsrc[min(tid + 3 * 64 * KW, gpieces - 1)];
  if (tid < BM) {
    const bool valid = m0 + tid < a.M;
    int id = valid ? tid_raw : -1;
    if (valid && (id < 0 || id >= a.vocab)) {
      atomicOr(a.flags, 1u);
      id = -1;
    }
    s_id[tid] = id;
    s_dst[tid] = valid ? tdst : -1;
    s_pos[tid] = valid ? tpos : 0;
  }
  uint4 *gdst = reinterpret_cast<uint4 *>(s_gamma);
  if (tid < gpieces) gdst[tid] = gv0;
  if constexpr (GMAX > 1) if (tid + 64 * KW < gpieces) gdst[tid + 64 * KW] = gv1;
  if constexpr (GMAX > 2) if (tid + 2 * 64 * KW < gpieces) gdst[tid + 2 * 64 * KW] = gv2;
  if constexpr (GMAX > 3) if (tid + 3 * 64 * KW < gpieces) gdst[tid + 3 * 64 * KW] = gv3;
  lds_barrier();

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int id = s_id[mb * 16 + r16];
    arow[mb] = E + (size_t)(id >= 0 ? id : 0) * D;
  }
  load_e(gbuf[0], 0);
  if constexpr (NG > 1) load_e(gbuf[1], 1);

  // Epilogue operands fetched now, so that no load is waited for after the
  // main loop: the RoPE (cos, sin) of this wave's output slots (wave w
  // finalises (row block, column block) item w) and this thread's first
  // EmbedCache piece (the tile's embedding rows are copied to h, spread over
  // the column tiles of the grid; rows with a bad id get zeros).
  static_assert(MB * NB <= KW, "one epilogue item per wave");
  const int nrot = (a.H + a.Hkv) * dh;     // features that get RoPE (Q and K)
  const int ep_mb = min(w, MB * NB - 1) / NB, ep_nb = min(w, MB * NB - 1) % NB;
  const int ep_cb = min(cb0 + ep_nb, ncb - 1);
  const int ep_pair = (ep_cb % cbh) * 8 + (r16 & 7);
  float2 ep_cs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ep_cs[i] = a.rope[(size_t)s_pos[ep_mb * 16 + 4 * g + i] * (dh / 2) + ep_pair];
  constexpr int NV = sizeof(T) * 8 / 16;   // uint4 pieces per 8 elements
  const int h_pieces = BM * (D / 8);
  const int h_per = (h_pieces + gridDim.x - 1) / gridDim.x;
  const int h_c = blockIdx.x * h_per + tid;
  const int h_row = min(h_c / (D / 8), BM - 1), h_col = (h_c % (D / 8)) * 8;
  const uint4 *h_src = reinterpret_cast<const uint4 *>(E + (size_t)max(s_id[h_row], 0) * D + h_col);
  const uint4 h_v0 = h_src[0], h_v1 = h_src[NV - 1];

  if constexpr (NG > 0) {
    // Two groups in flight while a third is multiplied.
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      // Keep the schedule as written: loads two groups ahead, then this
      // group's MFMAs (without the fences the scheduler hoists loads of later
      // groups and runs out of registers).
      if (gi + 2 < NG) load_group(gbuf[(gi + 2) % 3], gi + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute_group(gbuf[gi % 3], gi);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    Group &ga = gbuf[0], &gb = gbuf[1];
    for (int grp = 0; grp < ngroups; grp += 2) {
      if (grp + 1 < ngroups) load_group(gb, grp + 1);
      compute_group(ga, grp);
      if (grp + 1 < ngroups) {
        if (grp + 2 < ngroups) load_group(ga, grp + 2);
        compute_group(gb, grp + 1);
      }
    }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    // Diagonal entry (r, r) of the 16x16 result sits in lane r + 16*(r/4), slot r%4.
    if ((r16 >> 2) == g) {
      const int i = r16 & 3;
      s_ssq[w][mb * 16 + r16] = i == 0 ? ssq[mb][0] : i == 1 ? ssq[mb][1] : i == 2 ? ssq[mb][2] : ssq[mb][3];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s_red[w][mb][nb][lane] = acc[mb][nb];
  }
  lds_barrier();

  const float invD = 1.0f / (float)D;
  if (w < MB * NB && cb0 + ep_nb < ncb) {   // wave-uniform
    const int mb = ep_mb, nb = ep_nb;
    const int cb = cb0 + nb;
    f32x4_t sum = s_red[0][mb][nb][lane];
#pragma unroll
    for (int ww = 1; ww < KW; ++ww) sum += s_red[ww][mb][nb][lane];
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    const int pair = p0 + (r16 & 7);
    const bool first = r16 < 8;
    const int feat = hh * dh + (first ? pair : dh / 2 + pair);
    const bool rot = feat < nrot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mb * 16 + 4 * g + i;
      float ss = 0.f;
#pragma unroll
      for (int ww = 0; ww < KW; ++ww) ss += s_ssq[ww][row];
      const float y = s_id[row] >= 0 ? sum[i] * rsqrtf(ss * invD + a.eps) : 0.f;
      const float other = __shfl_xor(y, 8);
      float o = y;
      if (rot) o = first ? (y * ep_cs[i].x - other * ep_cs[i].y) : (other * ep_cs[i].y + y * ep_cs[i].x);
      const int dst = s_dst[row];
      if (dst >= 0) {
        if constexpr (sizeof(TC) == 2) {
          if (!(fabsf(o) <= kF16Max)) atomicOr(a.flags, 2u);
        }
        const int qf = a.H * dh, kf = a.Hkv * dh;
        if (feat < qf) {
          static_cast<TC *>(a.q)[(size_t)dst * qf + feat] = from_f32<TC>(o);
        } else if (feat < qf + kf) {
          static_cast<TC *>(a.k)[(size_t)dst * kf + (feat - qf)] = from_f32<TC>(o);
        } else {
          static_cast<TC *>(a.v)[(size_t)dst * kf + (feat - qf - kf)] = from_f32<TC>(o);
        }
      }
    }
  }

  // EmbedCache stores: the prefetched piece, then (only for very wide rows)
  // any further pieces of this thread.
  for (int t = tid; t < h_per; t += blockDim.x) {
    const int c = blockIdx.x * h_per + t;
    if (c >= h_pieces) break;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    const int dst = s_dst[row], id = s_id[row];
    if (dst < 0) continue;
    T *hp = static_cast<T *>(a.h) + (size_t)dst * D + col;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (id >= 0) v = t == tid ? (j == 0 ? h_v0 : h_v1) : reinterpret_cast<const uint4 *>(E + (size_t)id * D + col)[j];
      reinterpret_cast<uint4 *>(hp)[j] = v;
    }
  }
}

hipError_t launch_qkv(DType dt, const SeqArgs &sa, const QkvArgs &a, int F, hipStream_t s, const LaunchEvents &ev) {
  if (a.M <= 0) return hipSuccess;
  const int ncb = F / 16;
  dim3 grid((ncb + kQkvNB - 1) / kQkvNB, (a.M + kQkvRows - 1) / kQkvRows);
  dim3 block(64 * kQkvWaves);
  const int steps_per_wave = a.D / kQkvWaves / 32;
#define LC_QKV(TP, TC, SPLIT, U, NG) \
  lc_launch<qkv_fused_kernel<TP, TC, kQkvNB, kQkvWaves, SPLIT, U, NG>>(grid, block, 0, s, ev, sa, a)
  if (dt == kBF16) {
    switch (steps_per_wave) {
      case 2: LC_QKV(bf16_t, f16_t, true, 2, 1); break;
      case 4: LC_QKV(bf16_t, f16_t, true, 2, 2); break;
      case 8: LC_QKV(bf16_t, f16_t, true, 2, 4); break;
      case 16: LC_QKV(bf16_t, f16_t, true, 2, 8); break;
      case 32: LC_QKV(bf16_t, f16_t, true, 2, 16); break;
      default:
        if (steps_per_wave % 2 == 0) LC_QKV(bf16_t, f16_t, true, 2, 0);
        else LC_QKV(bf16_t, f16_t, true, 1, 0);
    }
  } else {
    switch (steps_per_wave) {
      case 1: LC_QKV(float, float, false, 1, 1); break;
      case 2: LC_QKV(float, float, false, 1, 2); break;
      default: LC_QKV(float, float, false, 1, 0);
    }
  }
#undef LC_QKV
  return hipGetLastError();
}

}  // namespace lc
