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

template <typename T, typename TC, int NB, int KW, bool SPLIT>
__global__ __launch_bounds__(64 * KW) void qkv_fused_kernel(const SeqArgs sa, const QkvArgs a) {
  constexpr int MB = 2;                    // 16-row blocks per tile
  constexpr int BM = 16 * MB;
  __shared__ int s_id[BM], s_dst[BM], s_pos[BM];
  __shared__ float s_ssq[KW][BM];
  __shared__ f32x4_t s_red[KW][MB][NB][64];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int dh = a.dh, D = a.D;
  const int cbh = dh / 16;                 // column blocks per head
  const int ncb = (a.H + 2 * a.Hkv) * cbh;
  const int cb0 = blockIdx.x * NB;
  const int m0 = blockIdx.y * BM;

  if (tid < BM) {
    const int m = m0 + tid;
    int id = -1, dst = -1, pos = 0;
    if (m < a.M) {
      const int b = find_sample(sa.pre[0], sa.n, m);
      const int local = m - sa.pre[0][b];
      if (a.mode == 0) {
        dst = sa.off[b] + sa.bs[b] + local;
        pos = sa.bs[b] + local;
        id = a.ids[a.ids_base + m];
      } else {
        dst = sa.off[b] + local;
        pos = local;
        id = a.ids[dst];
      }
      if (id < 0 || id >= a.vocab) {
        atomicOr(a.flags, 1u);
        id = -1;
      }
    }
    s_id[tid] = id;
    s_dst[tid] = dst;
    s_pos[tid] = pos;
  }
  __syncthreads();

  const T *E = static_cast<const T *>(a.E);
  const T *W = static_cast<const T *>(a.W);
  const T *gamma = static_cast<const T *>(a.gamma);

  const T *arow[MB];
  bool avalid[MB];
  int adst[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int id = s_id[mb * 16 + r16];
    avalid[mb] = id >= 0;
    adst[mb] = s_dst[mb * 16 + r16];
    arow[mb] = E + (size_t)(avalid[mb] ? id : 0) * D;
  }
  const T *brow[NB];
  bool bvalid[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int cb = cb0 + nb;
    bvalid[nb] = cb < ncb;
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    const int wrow = hh * dh + (r16 < 8 ? p0 + r16 : dh / 2 + p0 + (r16 - 8));
    brow[nb] = W + (size_t)(bvalid[nb] ? wrow : 0) * D;
  }
  const bool write_h = (blockIdx.x == 0) && (a.h != nullptr);
  T *hout = static_cast<T *>(a.h);

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float ssq[MB] = {};

  const int kper = D / KW;
  const int kbeg = w * kper;
#pragma unroll 4
  for (int k = kbeg; k < kbeg + kper; k += 32) {
    const int kk = k + 8 * g;
    Frag<T> gm, af[MB], al[MB], bf[NB], raw[MB];
    frag_load(gm, gamma + kk);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (bvalid[nb]) frag_load(bf[nb], brow[nb] + kk); else frag_zero(bf[nb]);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (avalid[mb]) frag_load(raw[mb], arow[mb] + kk); else frag_zero(raw[mb]);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (write_h && adst[mb] >= 0) {
        T *dstp = hout + (size_t)adst[mb] * D + kk;
#pragma unroll
        for (int i = 0; i < 8; ++i) dstp[i] = from_f32<T>(frag_get(raw[mb], i));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = frag_get(raw[mb], i);
        ssq[mb] = fmaf(x, x, ssq[mb]);
        const float y = x * frag_get(gm, i);
        frag_set(af[mb], i, y);
        if constexpr (SPLIT) frag_set(al[mb], i, y - frag_get(af[mb], i));
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        mma16(acc[mb][nb], af[mb], bf[nb]);
        if constexpr (SPLIT) mma16(acc[mb][nb], al[mb], bf[nb]);
      }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const float s = group_sum(ssq[mb]);
    if (g == 0) s_ssq[w][mb * 16 + r16] = s;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s_red[w][mb][nb][lane] = acc[mb][nb];
  }
  __syncthreads();

  const float invD = 1.0f / (float)D;
  const int nrot = (a.H + a.Hkv) * dh;     // features that get RoPE (Q and K)
  for (int c = w; c < MB * NB; c += KW) {
    const int mb = c / NB, nb = c % NB;
    const int cb = cb0 + nb;
    if (cb >= ncb) continue;                // wave-uniform
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
      const float y = sum[i] * rsqrtf(ss * invD + a.eps);
      const float other = __shfl_xor(y, 8);
      float o = y;
      if (rot) {
        const float2 cs = a.rope[(size_t)s_pos[row] * (dh / 2) + pair];
        o = first ? (y * cs.x - other * cs.y) : (other * cs.y + y * cs.x);
      }
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
}

hipError_t launch_qkv(DType dt, const SeqArgs &sa, const QkvArgs &a, int F, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  const int ncb = F / 16;
  dim3 grid((ncb + kQkvNB - 1) / kQkvNB, (a.M + kQkvRows - 1) / kQkvRows);
  dim3 block(64 * kQkvWaves);
  if (dt == kBF16)
    qkv_fused_kernel<bf16_t, f16_t, kQkvNB, kQkvWaves, true><<<grid, block, 0, s>>>(sa, a);
  else
    qkv_fused_kernel<float, float, kQkvNB, kQkvWaves, false><<<grid, block, 0, s>>>(sa, a);
  return hipGetLastError();
}

}  // namespace lc
