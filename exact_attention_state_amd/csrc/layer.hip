// The rest of layer 0 after its attention, in the parameter precision, and
// the sampler cut (LaCache, Figure 2; Section 3.4: the first layer stays out
// of the FP8 strategy, and only the current block's rows of the transformer
// output reach the final norm, the lm-head and the float softmax).
//
// * bf16 GEMM y = A W^T on the matrix cores (v_mfma 16x16x32 bf16, fp32
//   accumulation in the MFMA), both operands row-major with the contraction
//   contiguous (activations [M, K], nn.Linear weights [N, K]); epilogues:
//   bf16 output with an optional residual (out = bf16(res + bf16(acc))),
//   SwiGLU of a gate / up pair (y = bf16(silu(bf16(g)) bf16(u))), or fp32.
// * Row RMSNorm to bf16 (gamma r / sqrt(mean(r^2) + eps)), on every row or on
//   the block rows of a block table.
// * Float softmax of fp32 logit rows: argmax (first index among equal maxima),
//   its probability, and optionally every probability (three launches: chunk
//   partials, per-row combine, probabilities).
//
// Operand tiles move from HBM straight into LDS (global_load_lds_dwordx4).
// A tile row of one 64-wide contraction step is 128 bytes = eight 16-byte
// chunks; chunk c of row r sits in slot c ^ ((r >> 1) & 7), so the 16 rows a
// fragment read touches fall in 16 different bank groups.  The copy realises
// the swizzle from the source side: lane l of a copy fetches the chunk that
// belongs in its fixed LDS slot.

#include <algorithm>

#include "internal.h"

namespace lc {

// ---------------------------------------------------------------------------
// bf16 GEMM
// ---------------------------------------------------------------------------
// NW waves per workgroup: 8 (wave tiles TM/2 x TN/4, or TM x TN/8 below 128
// rows) or 4 (TM/2 x TN/2: a 128 x 128 tile gives 64 x 64 per wave, half the
// LDS fragment reads per MFMA of eight 64 x 32 waves).
template <int TM, int TN, int NW = 8> struct BT {
  static constexpr int WM = TM >= 128 ? 2 : 1, WN = NW / WM;     // wave grid
  static constexpr int WRB = TM / WM / 16, WCB = TN / WN / 16;   // 16 x 16 fragments per wave
  static constexpr int CB = TN / 16;
  static constexpr int STAGE = (TM + TN) * 128;                  // one 64-wide contraction step
  static constexpr int COPIES = (TM + TN) / (8 * NW);            // 1 KB copies (8 rows) per wave per stage
  static_assert(COPIES * 8 * NW == TM + TN, "copies must tile the stage");
  static_assert(WRB >= 1 && WCB >= 2 && WCB % 2 == 0, "wave tile");
};

enum { kLayerEpiBf16 = 0, kLayerEpiF32 = 1, kLayerEpiSwiglu = 2 };

__device__ __forceinline__ uint32_t swz_slot(int row, int chunk) { return (uint32_t)(chunk ^ ((row >> 1) & 7)); }

template <int TM, int TN, int NST, int EPI, int NW = 8>
__global__ __launch_bounds__(64 * NW) void bf16_gemm_kernel(const Bf16GemmArgs a) {
  using T = BT<TM, TN, NW>;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w % T::WM, wn = w / T::WM;
  // Output tiles: SwiGLU tiles cover TN / 2 features (their gate and up rows).
  const int NX = EPI == kLayerEpiSwiglu ? a.N / (TN / 2) : (a.N + TN - 1) / TN;
  const int MY = (a.M + TM - 1) / TM, ntiles = NX * MY;
  const int S = a.splits > 1 ? a.splits : 1, nunits = ntiles * S;
  // Workgroup wg runs on die wg % 8; each die takes a contiguous run of the
  // unit sequence (unit = tile x split; a tile's splits adjacent), which
  // walks groups of kGM row tiles column by column.
  const int per_die = (nunits + 7) / 8, wg = blockIdx.x;
  const int uu = (wg & 7) * per_die + (wg >> 3);
  if (uu >= nunits) return;                                    // whole workgroup
  const int u = uu / S, split = uu % S;
  constexpr int kGM = 8;
  const int grp = u / (kGM * NX), within = u % (kGM * NX);
  const int gm = min(kGM, MY - grp * kGM);
  const int m0 = (grp * kGM + within % gm) * TM, nt = within / gm;
  const int KGA = a.K / 64;
  const int kg0 = (int)((long)split * KGA / S), KG = (int)((long)(split + 1) * KGA / S) - kg0;
  const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_address(smem));

  // Copy c of a stage fills rows 8c .. 8c + 7 of the stage's [TM + TN] rows
  // (A rows, then W rows); rows past the operand's end repeat its last row.
  auto issue = [&](int g) {
    const uint32_t st = lbase + (g % NST) * T::STAGE;
#pragma unroll
    for (int j = 0; j < T::COPIES; ++j) {
      const int c = w * T::COPIES + j, lr0 = 8 * c;
      const bf16_t *base;
      int row0, R, ld;
      if (lr0 < TM) {
        base = a.A;
        row0 = m0 + lr0;
        R = a.M;
        ld = a.lda;
      } else if (EPI == kLayerEpiSwiglu) {
        const int br = lr0 - TM, half = TN / 2;
        base = br < half ? a.B : a.B2;
        row0 = nt * half + (br % half);
        R = a.N;
        ld = a.ldb;
      } else {
        base = a.B;
        row0 = nt * TN + (lr0 - TM);
        R = a.N;
        ld = a.ldb;
      }
      const int srow = min(row0, R - 1);                       // scalar base row
      const int lrow = lr0 + (lane >> 3);                      // stage row this lane fills
      const int grow = min(row0 + (lane >> 3), R - 1);
      const uint32_t voff = (uint32_t)(grow - srow) * (uint32_t)ld * 2u + (swz_slot(lrow, lane & 7) << 4);
      const char *sb = reinterpret_cast<const char *>(base) + ((size_t)srow * ld + (size_t)(kg0 + g) * 64) * 2;
      dma16_s(sb, voff, st + c * 1024);
    }
  };
  auto cb_of = [&](int j) {
    if constexpr (EPI == kLayerEpiSwiglu) {
      constexpr int H = T::WCB / 2;
      return (j < H ? 0 : T::CB / 2) + wn * H + (j % H);
    } else {
      return wn * T::WCB + j;
    }
  };

  f32x4_t acc[T::WRB][T::WCB];
#pragma unroll
  for (int i = 0; i < T::WRB; ++i)
#pragma unroll
    for (int j = 0; j < T::WCB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int pro = KG < NST ? KG : NST;
  for (int s = 0; s < pro; ++s) issue(s);
  vmcnt_wait_rt<NST * T::COPIES>((pro - 1) * T::COPIES);
  lds_barrier();

  const int r16 = lane & 15, q4 = lane >> 4;
  for (int g = 0; g < KG; ++g) {
    const char *st = smem + (g % NST) * T::STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int chunk = kk * 4 + q4;                           // lane's 8 contraction elements
      bf16x8_t bfr[T::WCB];
#pragma unroll
      for (int j = 0; j < T::WCB; ++j) {
        const int row = TM + cb_of(j) * 16 + r16;
        bfr[j] = *reinterpret_cast<const bf16x8_t *>(st + row * 128 + (swz_slot(row, chunk) << 4));
      }
#pragma unroll
      for (int i = 0; i < T::WRB; ++i) {
        const int row = (wm * T::WRB + i) * 16 + r16;
        const bf16x8_t afr = *reinterpret_cast<const bf16x8_t *>(st + row * 128 + (swz_slot(row, chunk) << 4));
#pragma unroll
        for (int j = 0; j < T::WCB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    if (g + 1 < KG) {
      // This wave's copies of step g + 1 landed; the barrier publishes the
      // stage and frees stage g for step g + NST.
      const int behind = (KG - 2 - g) < (NST - 2) ? (KG - 2 - g) : (NST - 2);
      vmcnt_wait_rt<NST * T::COPIES>(behind * T::COPIES);
      lds_barrier();
      if (g + NST < KG) issue(g + NST);
    }
  }
  __syncthreads();                                             // the ring's LDS is free

  // Results leave through this wave's LDS area, one 16-row fragment row
  // block at a time, as row-wise 16-byte pieces.  A fragment's lane l holds
  // rows 4 (l / 16) + v, column l % 16.
  if (S > 1) {
    // Split partial: the wave's 16 WCB columns of the tile (fragment j of
    // wave wn at tile column 16 (wn WCB + j)), raw fp32.
    constexpr int COLS = 16 * T::WCB, STRIDE = COLS + 4, CPL = COLS / 4;
    float *ws = reinterpret_cast<float *>(smem) + w * 16 * STRIDE;
    const int rr = lane >> 2, c0 = (lane & 3) * CPL;
    float *dst = a.part + (size_t)split * a.M * a.ldp + (size_t)nt * TN + wn * COLS + c0;
#pragma unroll
    for (int i = 0; i < T::WRB; ++i) {
#pragma unroll
      for (int j = 0; j < T::WCB; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) ws[(4 * q4 + v) * STRIDE + 16 * j + r16] = acc[i][j][v];
      wave_lds_sync();
      const int m = m0 + (wm * T::WRB + i) * 16 + rr;
      if (m < a.M) {
        const float *src = ws + rr * STRIDE + c0;
#pragma unroll
        for (int p = 0; p < CPL / 4; ++p)
          *reinterpret_cast<float4 *>(dst + (size_t)m * a.ldp + 4 * p) =
              make_float4(src[4 * p], src[4 * p + 1], src[4 * p + 2], src[4 * p + 3]);
      }
      wave_lds_sync();
    }
    return;
  }
  if constexpr (EPI == kLayerEpiSwiglu) {
    constexpr int H = T::WCB / 2, FC = 16 * H, STRIDE = FC + 4, PPR = FC / 8;   // features per wave, pieces per row
    float *ws = reinterpret_cast<float *>(smem) + w * 16 * STRIDE;
    bf16_t *out = static_cast<bf16_t *>(a.out);
#pragma unroll
    for (int i = 0; i < T::WRB; ++i) {
#pragma unroll
      for (int j = 0; j < H; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gt = bf2f(f2bf(acc[i][j][v])), up = bf2f(f2bf(acc[i][j + H][v]));
          ws[(4 * q4 + v) * STRIDE + 16 * j + r16] = gt / (1.0f + __expf(-gt)) * up;
        }
      wave_lds_sync();
      if (lane < 16 * PPR) {
        const int rr = lane / PPR, pc = lane % PPR;
        const int m = m0 + (wm * T::WRB + i) * 16 + rr;
        if (m < a.M) {
          const float *src = ws + rr * STRIDE + 8 * pc;
          uint32_t ow[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) ow[q] = (uint32_t)f2bf(src[2 * q]) | ((uint32_t)f2bf(src[2 * q + 1]) << 16);
          const int f = nt * (TN / 2) + wn * FC + 8 * pc;
          *reinterpret_cast<uint4 *>(out + (size_t)m * a.ldo + f) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        }
      }
      wave_lds_sync();
    }
  } else {
    constexpr int COLS = 16 * T::WCB, STRIDE = COLS + 4, CPL = COLS / 4;   // columns per lane: a multiple of 8
    float *ws = reinterpret_cast<float *>(smem) + w * 16 * STRIDE;
    const int rr = lane >> 2, c0 = (lane & 3) * CPL;
    const int ncol = nt * TN + wn * COLS + c0;
#pragma unroll
    for (int i = 0; i < T::WRB; ++i) {
#pragma unroll
      for (int j = 0; j < T::WCB; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) ws[(4 * q4 + v) * STRIDE + 16 * j + r16] = acc[i][j][v];
      wave_lds_sync();
      const int m = m0 + (wm * T::WRB + i) * 16 + rr;
      if (m < a.M) {
        const float *src = ws + rr * STRIDE + c0;
#pragma unroll
        for (int p = 0; p < CPL / 8; ++p) {
          const int n = ncol + 8 * p;
          if (n >= a.N) break;                                 // N is a multiple of 8
          if constexpr (EPI == kLayerEpiF32) {
            float *o = static_cast<float *>(a.out) + (size_t)m * a.ldo + n;
            *reinterpret_cast<float4 *>(o) = make_float4(src[8 * p], src[8 * p + 1], src[8 * p + 2], src[8 * p + 3]);
            *reinterpret_cast<float4 *>(o + 4) =
                make_float4(src[8 * p + 4], src[8 * p + 5], src[8 * p + 6], src[8 * p + 7]);
          } else {
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = bf2f(f2bf(src[8 * p + e]));   // the linear's bf16 output
            if (a.res) {
              const uint4 ru = *reinterpret_cast<const uint4 *>(a.res + (size_t)m * a.ldr + n);
              const uint32_t rw[4] = {ru.x, ru.y, ru.z, ru.w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                y[2 * q] += __uint_as_float(rw[q] << 16);
                y[2 * q + 1] += __uint_as_float(rw[q] & 0xffff0000u);
              }
            }
            uint32_t ow[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) ow[q] = (uint32_t)f2bf(y[2 * q]) | ((uint32_t)f2bf(y[2 * q + 1]) << 16);
            *reinterpret_cast<uint4 *>(static_cast<bf16_t *>(a.out) + (size_t)m * a.ldo + n) =
                make_uint4(ow[0], ow[1], ow[2], ow[3]);
          }
        }
      }
      wave_lds_sync();
    }
  }
}

// ---------------------------------------------------------------------------
// Sum of the split partials, in split order, and the epilogue: one thread per
// 8 consecutive outputs of a row.  Partial column of output n: n itself, or,
// for SwiGLU tiles of TN B rows (gate rows then up rows) whose waves hold
// HW = WCB / 2 gate and HW up fragments each, feature f = nt (TN / 2) + fi
// sits at tile column 16 (wn WCB + j) + fi % 16 with fi / 16 = wn HW + j
// (gate) and at 16 HW more (up).
// ---------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const Bf16GemmArgs a, int TN, int HW) {
  const int per_row = a.N / 8;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.M * per_row) return;
  const int m = (int)(idx / per_row), n = (int)(idx % per_row) * 8;
  const size_t sstride = (size_t)a.M * a.ldp;
  auto sum8 = [&](int col, float *y) {
    const float *p = a.part + (size_t)m * a.ldp + col;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = 0.f;
    for (int sp = 0; sp < a.splits; ++sp, p += sstride) {
      const float4 u0 = *reinterpret_cast<const float4 *>(p), u1 = *reinterpret_cast<const float4 *>(p + 4);
      y[0] += u0.x; y[1] += u0.y; y[2] += u0.z; y[3] += u0.w;
      y[4] += u1.x; y[5] += u1.y; y[6] += u1.z; y[7] += u1.w;
    }
  };
  float y[8];
  if constexpr (EPI == kLayerEpiSwiglu) {
    const int half = TN / 2, nt = n / half, fi = n % half, cb = fi / 16;
    const int col = nt * TN + 16 * (2 * HW * (cb / HW) + cb % HW) + fi % 16;
    float up[8];
    sum8(col, y);
    sum8(col + 16 * HW, up);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gt = bf2f(f2bf(y[e])), u = bf2f(f2bf(up[e]));
      y[e] = gt / (1.0f + __expf(-gt)) * u;
    }
  } else {
    sum8(n, y);
    if constexpr (EPI == kLayerEpiF32) {
      float *o = static_cast<float *>(a.out) + (size_t)m * a.ldo + n;
      *reinterpret_cast<float4 *>(o) = make_float4(y[0], y[1], y[2], y[3]);
      *reinterpret_cast<float4 *>(o + 4) = make_float4(y[4], y[5], y[6], y[7]);
      return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = bf2f(f2bf(y[e]));       // the linear's bf16 output
    if (a.res) {
      const uint4 ru = *reinterpret_cast<const uint4 *>(a.res + (size_t)m * a.ldr + n);
      const uint32_t rw[4] = {ru.x, ru.y, ru.z, ru.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        y[2 * q] += __uint_as_float(rw[q] << 16);
        y[2 * q + 1] += __uint_as_float(rw[q] & 0xffff0000u);
      }
    }
  }
  uint32_t ow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ow[q] = (uint32_t)f2bf(y[2 * q]) | ((uint32_t)f2bf(y[2 * q + 1]) << 16);
  *reinterpret_cast<uint4 *>(static_cast<bf16_t *>(a.out) + (size_t)m * a.ldo + n) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
}

// ---------------------------------------------------------------------------
// Row RMSNorm: one wave per output row (D = 512 NCH, each lane NCH 16-byte
// pieces); the sum of squares in fp32, 1 / sqrt(mean + eps) correctly
// rounded, out = bf16(gamma r inv).
// ---------------------------------------------------------------------------
template <int NCH>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const RowNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= a.M) return;                                        // whole wave
  constexpr int D = 512 * NCH;
  int src_row = m;
  if (a.gather) {                                              // block row m of the table
    const int b = find_sample(a.sa.pre[0], a.sa.n, m);
    src_row = a.sa.off[b] + a.sa.bs[b] + (m - a.sa.pre[0][b]);
  }
  const bf16_t *r = a.src + (size_t)src_row * a.lds;
  float rv[NCH][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const uint4 ru = *reinterpret_cast<const uint4 *>(r + 512 * j + 8 * lane);
    const uint32_t rw[4] = {ru.x, ru.y, ru.z, ru.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rv[j][2 * q] = __uint_as_float(rw[q] << 16);
      rv[j][2 * q + 1] = __uint_as_float(rw[q] & 0xffff0000u);
      ss = fmaf(rv[j][2 * q], rv[j][2 * q], ss);
      ss = fmaf(rv[j][2 * q + 1], rv[j][2 * q + 1], ss);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) ss += __shfl_xor(ss, o);
  const float inv = 1.0f / __fsqrt_rn(ss / (float)D + a.eps);
  bf16_t *out = a.out + (size_t)m * D;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const uint4 gu = *reinterpret_cast<const uint4 *>(a.gamma + 512 * j + 8 * lane);
    const uint32_t gw[4] = {gu.x, gu.y, gu.z, gu.w};
    uint32_t ow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x0 = __uint_as_float(gw[q] << 16) * rv[j][2 * q] * inv;
      const float x1 = __uint_as_float(gw[q] & 0xffff0000u) * rv[j][2 * q + 1] * inv;
      ow[q] = (uint32_t)f2bf(x0) | ((uint32_t)f2bf(x1) << 16);
    }
    *reinterpret_cast<uint4 *>(out + 512 * j + 8 * lane) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
}

// ---------------------------------------------------------------------------
// Float softmax of fp32 logit rows (V a multiple of 4), in three steps so a
// row spreads over many workgroups: (1) per chunk of kSmChunk logits, the
// chunk's maximum, its first index and sum exp(l - chunk max); (2) per row,
// one wave combines the chunks: the row maximum, its first index and
// sum = sum_c s_c exp(m_c - max); the argmax's probability is 1 / sum;
// (3) if requested, every probability exp(l - max) / sum.
// ---------------------------------------------------------------------------
constexpr int kSmChunk = 4096;

__device__ __forceinline__ void better(float &mx, int &ix, float m2, int i2) {
  if (m2 > mx || (m2 == mx && i2 < ix)) {
    mx = m2;
    ix = i2;
  }
}

__global__ __launch_bounds__(256) void softmax_partial_kernel(const SoftmaxArgs a) {
  __shared__ float s_m[4], s_s[4];
  __shared__ int s_i[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = blockIdx.y, c = blockIdx.x, nch = gridDim.x;
  const float *l = a.logits + (size_t)row * a.ld;
  const int v0 = c * kSmChunk, v1 = min(a.V, v0 + kSmChunk);
  float mx = -INFINITY;
  int ix = 0x7fffffff;
  float4 x[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {                                // 16 logits per thread
    const int i = v0 + 4 * (tid + 256 * k);
    x[k] = i < v1 ? *reinterpret_cast<const float4 *>(l + i) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (i < v1) {
      better(mx, ix, x[k].x, i);
      better(mx, ix, x[k].y, i + 1);
      better(mx, ix, x[k].z, i + 2);
      better(mx, ix, x[k].w, i + 3);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) better(mx, ix, __shfl_xor(mx, o), __shfl_xor(ix, o));
  if (lane == 0) {
    s_m[w] = mx;
    s_i[w] = ix;
  }
  __syncthreads();
  mx = s_m[0];
  ix = s_i[0];
#pragma unroll
  for (int k = 1; k < 4; ++k) better(mx, ix, s_m[k], s_i[k]);
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (v0 + 4 * (tid + 256 * k) < v1)
      sum += (expf(x[k].x - mx) + expf(x[k].y - mx)) + (expf(x[k].z - mx) + expf(x[k].w - mx));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) s_s[w] = sum;
  __syncthreads();
  if (tid == 0) {
    const size_t p = (size_t)row * nch + c;
    a.part[p] = make_float2(mx, (s_s[0] + s_s[1]) + (s_s[2] + s_s[3]));
    a.part_idx[p] = ix;
  }
}

__global__ __launch_bounds__(256) void softmax_combine_kernel(const SoftmaxArgs a, int nch) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.M) return;                                      // whole wave
  float mx = -INFINITY;
  int ix = 0x7fffffff;
  for (int c = lane; c < nch; c += 64) better(mx, ix, a.part[(size_t)row * nch + c].x, a.part_idx[(size_t)row * nch + c]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) better(mx, ix, __shfl_xor(mx, o), __shfl_xor(ix, o));
  float sum = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const float2 p = a.part[(size_t)row * nch + c];
    sum += p.y * expf(p.x - mx);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) {
    a.token[row] = ix;
    a.conf[row] = 1.0f / sum;
    a.row_stat[row] = make_float2(mx, sum);
  }
}

__global__ __launch_bounds__(256) void softmax_probs_kernel(const SoftmaxArgs a) {
  const int row = blockIdx.y;
  const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (i >= a.V) return;
  const float2 st = a.row_stat[row];
  const float4 x = *reinterpret_cast<const float4 *>(a.logits + (size_t)row * a.ld + i);
  *reinterpret_cast<float4 *>(a.probs + (size_t)row * a.ldp + i) = make_float4(
      expf(x.x - st.x) / st.y, expf(x.y - st.x) / st.y, expf(x.z - st.x) / st.y, expf(x.w - st.x) / st.y);
}

int softmax_chunks(int V) { return (V + kSmChunk - 1) / kSmChunk; }

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {
template <int TM, int TN, int NST> constexpr int bf16_gemm_smem() { return NST * BT<TM, TN>::STAGE; }
inline unsigned grid8(long tiles) { return (unsigned)((tiles + 7) / 8 * 8); }

// Splits of a skinny launch: as many as keep tiles x splits within one
// workgroup per CU (one round), with at least kMinSplitSteps contraction
// steps per split.  Measured at LLaDA-8B's layer on 32 rows against rounding
// up (a short second round) and 4 / 16 minimum steps: within 4 %, this the
// fastest (W_o 17.7, gate-up 55.4, down 30.9 us).
constexpr int kMinSplitSteps = 8;
int skinny_splits(long tiles, int K) {
  const long cus = device_cus();
  if (tiles >= cus) return 1;
  const long s = std::min<long>(cus / tiles, (K / 64) / kMinSplitSteps);
  return s > 1 ? (int)s : 1;
}
// Splits of a launch of 128 x 128 tiles that leaves compute units idle and
// contracts over many steps (the down projection at 768 rows: 192 tiles of
// 192 steps): up to four of at least kLongSplitSteps steps each, run with
// two-stage rings so that two workgroups share a CU.  Measured at LLaDA-8B's
// layer on 768 rows: down 176 -> 138 us (three splits 151 us; four with the
// four-stage ring 160 us); W_o, 64 steps, stays whole (63 us either way).
constexpr int kLongSplitSteps = 48;
int long_splits(long tiles, int K) {
  if (tiles >= device_cus()) return 1;
  const int s = std::min(4, (K / 64) / kLongSplitSteps);
  return s > 1 ? s : 1;
}
template <int TN, int EPI> long skinny_nx(int N) { return EPI == kLayerEpiSwiglu ? N / (TN / 2) : (N + TN - 1) / TN; }

enum { kSplitNone = 0, kSplitSkinny = 1, kSplitLong = 2 };
template <int TM, int TN, int NST, int EPI, int NW = 8>
hipError_t go(const Bf16GemmArgs &a0, hipStream_t s, const LaunchEvents &ev, int rule) {
  Bf16GemmArgs a = a0;
  const long NX = skinny_nx<TN, EPI>(a.N);
  const long tiles = NX * ((a.M + TM - 1) / TM);
  a.splits = !a.part                ? 1
             : rule == kSplitSkinny ? skinny_splits(tiles, a.K)
             : rule == kSplitLong   ? long_splits(tiles, a.K)
                                    : 1;
  a.ldp = (int)(NX * TN);
  if (a.splits == 1) {
    lc_launch<bf16_gemm_kernel<TM, TN, NST, EPI, NW>>(dim3(grid8(tiles)), dim3(64 * NW), bf16_gemm_smem<TM, TN, NST>(), s,
                                                      ev, a);
    return hipGetLastError();
  }
  // The two launches share one event pair: the first stamps the start, the last the end.
  const LaunchEvents first{ev.start, nullptr}, last{nullptr, ev.stop};
  lc_launch<bf16_gemm_kernel<TM, TN, NST, EPI, NW>>(dim3(grid8(tiles * a.splits)), dim3(64 * NW),
                                                    bf16_gemm_smem<TM, TN, NST>(), s, first, a);
  const long threads = (long)a.M * (a.N / 8);
  lc_launch<splitk_reduce_kernel<EPI>>(dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, last, a, TN,
                                       BT<TM, TN, NW>::WCB / 2);
  return hipGetLastError();
}

template <int EPI> hipError_t dispatch(const Bf16GemmArgs &a, int tile, hipStream_t s, const LaunchEvents &ev) {
  const long cus = device_cus();
  const long n256 = EPI == kLayerEpiSwiglu ? a.N / 128 : (a.N + 255) / 256;
  if (tile == 0) {
    const long t256 = n256 * ((a.M + 255) / 256);
    if (a.M <= 64) tile = 3;                                               // skinny: 64 x 256
    else if (EPI == kLayerEpiSwiglu && t256 >= cus && t256 < 4 * cus && 4 * t256 < 3 * ((t256 + cus - 1) / cus) * cus)
      tile = 4;            // 256 x 256 SwiGLU tiles would leave a short last round (768 rows: 237 -> 215 us)
    else if (t256 >= cus) tile = 1;                                        // 256 x 256
    else tile = EPI == kLayerEpiSwiglu ? 3 : 2;                            // 128 x 128 (SwiGLU: 64 x 256)
  }
  switch (tile) {
    case 1: return go<256, 256, 2, EPI>(a, s, ev, kSplitNone);
    case 2:
      if constexpr (EPI == kLayerEpiSwiglu) {
        return hipErrorInvalidValue;
      } else {
        const long t128 = (long)((a.N + 127) / 128) * ((a.M + 127) / 128);
        if (a.part && long_splits(t128, a.K) > 1) return go<128, 128, 2, EPI>(a, s, ev, kSplitLong);
        return go<128, 128, 4, EPI>(a, s, ev, kSplitNone);
      }
    case 3: return go<64, 256, 3, EPI>(a, s, ev, a.M <= 64 ? kSplitSkinny : kSplitNone);
    case 4: return go<128, 128, 2, EPI, 4>(a, s, ev, kSplitNone);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

size_t bf16_gemm_part_bytes(int M, int N, int K, int out_kind) {
  if (M <= 0 || K % 64) return 0;
  size_t bytes = 0;
  if (M <= 64) {                                               // 64 x 256 tiles
    const long NX = out_kind == kGemmOutSwiglu ? skinny_nx<256, kLayerEpiSwiglu>(N) : skinny_nx<256, kLayerEpiBf16>(N);
    const int sp = skinny_splits(NX, K);
    if (sp > 1) bytes = (size_t)sp * M * NX * 256 * sizeof(float);
  }
  if (out_kind != kGemmOutSwiglu) {                            // 128 x 128 tiles (any row count)
    const long NX = (N + 127) / 128;
    const int sp = long_splits(NX * ((M + 127) / 128), K);
    if (sp > 1) bytes = std::max(bytes, (size_t)sp * M * NX * 128 * sizeof(float));
  }
  return bytes;
}

hipError_t launch_bf16_gemm(const Bf16GemmArgs &a, int epi, int tile, hipStream_t s, const LaunchEvents &ev) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % 64 || a.N % 8 || a.N <= 0 || a.lda % 8 || a.ldb % 8 || a.ldo % 8) return hipErrorInvalidValue;
  switch (epi) {
    case kGemmOutBf16: return dispatch<kLayerEpiBf16>(a, tile, s, ev);
    case kGemmOutF32: return dispatch<kLayerEpiF32>(a, tile, s, ev);
    case kGemmOutSwiglu:
      if (a.N % 128 || !a.B2) return hipErrorInvalidValue;
      return dispatch<kLayerEpiSwiglu>(a, tile, s, ev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rmsnorm_rows(const RowNormArgs &a, hipStream_t s, const LaunchEvents &ev) {
  if (a.M <= 0) return hipSuccess;
  const dim3 grid((a.M + 3) / 4), block(256);
  switch (a.D) {
    case 512: lc_launch<rmsnorm_rows_kernel<1>>(grid, block, 0, s, ev, a); break;
    case 1024: lc_launch<rmsnorm_rows_kernel<2>>(grid, block, 0, s, ev, a); break;
    case 2048: lc_launch<rmsnorm_rows_kernel<4>>(grid, block, 0, s, ev, a); break;
    case 4096: lc_launch<rmsnorm_rows_kernel<8>>(grid, block, 0, s, ev, a); break;
    case 8192: lc_launch<rmsnorm_rows_kernel<16>>(grid, block, 0, s, ev, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_softmax_argmax(const SoftmaxArgs &a, hipStream_t s, const LaunchEvents &ev) {
  if (a.M <= 0) return hipSuccess;
  if (a.V % 4 || a.ld % 4 || (a.probs && a.ldp % 4) || !a.part || !a.part_idx || !a.row_stat) return hipErrorInvalidValue;
  const int nch = softmax_chunks(a.V);
  // The three launches share one event pair: the first stamps the start, the last the end.
  const LaunchEvents first{ev.start, nullptr}, last{nullptr, ev.stop};
  lc_launch<softmax_partial_kernel>(dim3(nch, a.M), dim3(256), 0, s, first, a);
  if (a.probs) {
    lc_launch<softmax_combine_kernel>(dim3((a.M + 3) / 4), dim3(256), 0, s, LaunchEvents{}, a, nch);
    lc_launch<softmax_probs_kernel>(dim3((a.V / 4 + 255) / 256, a.M), dim3(256), 0, s, last, a);
  } else {
    lc_launch<softmax_combine_kernel>(dim3((a.M + 3) / 4), dim3(256), 0, s, last, a, nch);
  }
  return hipGetLastError();
}

hipError_t setup_layer_attributes() {
  hipError_t e = hipSuccess;
#define LC_BGA(TM, TN, NST, EPI)                                                                              \
  if (e == hipSuccess)                                                                                        \
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(bf16_gemm_kernel<TM, TN, NST, EPI>),               \
                            hipFuncAttributeMaxDynamicSharedMemorySize, bf16_gemm_smem<TM, TN, NST>());
  LC_BGA(256, 256, 2, kLayerEpiBf16) LC_BGA(256, 256, 2, kLayerEpiF32) LC_BGA(256, 256, 2, kLayerEpiSwiglu)
  LC_BGA(128, 128, 4, kLayerEpiBf16) LC_BGA(128, 128, 4, kLayerEpiF32)
  LC_BGA(128, 128, 2, kLayerEpiBf16) LC_BGA(128, 128, 2, kLayerEpiF32)
  LC_BGA(64, 256, 3, kLayerEpiBf16) LC_BGA(64, 256, 3, kLayerEpiF32) LC_BGA(64, 256, 3, kLayerEpiSwiglu)
#undef LC_BGA
#define LC_BGA4(NST, EPI)                                                                                     \
  if (e == hipSuccess)                                                                                        \
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(bf16_gemm_kernel<128, 128, NST, EPI, 4>),          \
                            hipFuncAttributeMaxDynamicSharedMemorySize, bf16_gemm_smem<128, 128, NST>());
  LC_BGA4(2, kLayerEpiBf16) LC_BGA4(2, kLayerEpiF32) LC_BGA4(2, kLayerEpiSwiglu)
#undef LC_BGA4
  return e;
}

}  // namespace lc
