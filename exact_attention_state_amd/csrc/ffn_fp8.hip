// Per-group FP8 FFN of the layers after the first (LaCache Section 3.4,
// "Mixed precision strategy", Eqs. (7)-(8); Figure 2): the feed-forward
// AddNorm with the quantization of its output fused in, the gate-up linear on
// FP8 operands with SwiGLU and the quantization of its output fused into the
// epilogue, and the ffout (down) linear on FP8 operands with the residual add
// in its epilogue.
//
// Quantization (Eqs. (7)-(8)): a group g of 128 activations of one token, or
// a 128 x 128 block of a weight, gets scale_g = max|x| / 448 and codes
// E4M3(clip(x / scale_g, -448, 448)), rounded to nearest even by the
// hardware conversion (OCP E4M3, the FP8 format the gfx950 matrix cores
// take); scale and x / scale are fp32 (correctly rounded division).
//
// FP8 GEMM y = A W^T: one v_mfma 16x16x128 (E4M3 x E4M3, unit block scales)
// per 16 x 16 output tile and 128-wide group, so every MFMA result is one
// group's partial product; it is scaled by sa[row, g] * sw[col block, g] and
// added to fp32 accumulators.  The matrix core's own sum of its 128 products
// is not exact fp32 (measured: up to 2^-12.4 of sum |a_k b_k|), so the groups
// are combined in fp32 outside it.
//
// Operand layout in memory ("packed", written by the quantization kernels):
// 256-row tiles (rows of A, or columns of the output = rows of W), then
// 128-wide groups of the contraction, then 16-row fragments of 2 KB.  In a
// fragment, lane l (row l % 16, contraction bytes 32 (l / 16) .. +31 of the
// group) owns 32 bytes, split into two 1 KB halves (its bytes 0-15 at
// 16 l, 16-31 at 1024 + 16 l), so each half is one full-rate 1 KB copy and
// one conflict-free 16-byte LDS read per lane.  A 256-row tile's group is a
// contiguous 32 KB stage.  Activation scales are stored group-major
// ([K/128][M_pad]) so a stage's row scales are contiguous.

#include "internal.h"

namespace lc {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kF8Frag = 2048;                 // one 16 x 128 FP8 operand fragment
constexpr int kF8Tile = 16 * kF8Frag;         // 256 rows x one 128-wide group
constexpr float kE4M3Max = 448.0f;

__host__ __device__ inline size_t fp8_pack_offset(int i, int k, int KG) {
  const int kk = k & 127;
  const int lane = ((kk >> 5) << 4) | (i & 15);
  return ((size_t)(i >> 8) * KG + (k >> 7)) * kF8Tile + ((i >> 4) & 15) * kF8Frag + ((kk >> 4) & 1) * 1024 +
         lane * 16 + (kk & 15);
}

// E4M3 code of v (already divided by its scale), clipped to the format's range.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  v = fminf(fmaxf(v, -kE4M3Max), kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}
// Codes of four values, packed little-endian in a 32-bit word.
__device__ __forceinline__ uint32_t e4m3_code4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
  d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Value of lane 4 (l / 4) + v in lane l (a DPP quad permutation).
template <int V> __device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), V * 0x55, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_max16(float x) {    // max over the 16 lanes of a lane group
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 4));
  return fmaxf(x, __shfl_xor(x, 8));
}

// ---------------------------------------------------------------------------
// Weight quantization: one workgroup per 128 x 128 block (Eq. (8) over the
// block), codes written in the packed layout at output row n' = remap(n).
// mode 0: n' = n; mode 1 / 2: the gate / up half of a gate-up weight, whose
// 256-row packed tiles hold 128 gate rows then the 128 up rows of the same
// output features (so one GEMM tile sees both halves of its SwiGLU inputs).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_pack_weight_kernel(const bf16_t *W, int N, int K, int mode, uint8_t *Wp,
                                                              float *sw, int Np) {
  __shared__ float s_max[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nb = blockIdx.x, g = blockIdx.y;
  const int n = nb * 128 + (t >> 1), k0 = g * 128 + 64 * (t & 1);
  const uint4 *src = reinterpret_cast<const uint4 *>(W + (size_t)n * K + k0);
  uint4 raw[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) raw[j] = src[j];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t u[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(u[q] << 16)), fabsf(__uint_as_float(u[q] & 0xffff0000u))));
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if (lane == 0) s_max[w] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float scale = amax / kE4M3Max;
  const int np = mode == 0 ? n : 256 * (n >> 7) + (mode == 2 ? 128 : 0) + (n & 127);
  const int KG = K / 128;
#pragma unroll
  for (int u4 = 0; u4 < 4; ++u4) {
    // 16 consecutive contraction elements: one contiguous 16-byte run of the packed layout.
    uint32_t word[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 r2 = raw[2 * u4 + (q >> 1)];
      const uint32_t a = (q & 1) ? r2.z : r2.x, b = (q & 1) ? r2.w : r2.y;
      const float x0 = __uint_as_float(a << 16), x1 = __uint_as_float(a & 0xffff0000u);
      const float x2 = __uint_as_float(b << 16), x3 = __uint_as_float(b & 0xffff0000u);
      word[q] = scale > 0.f ? e4m3_code4(x0 / scale, x1 / scale, x2 / scale, x3 / scale) : 0u;
    }
    *reinterpret_cast<uint4 *>(Wp + fp8_pack_offset(np, k0 + 16 * u4, KG)) = make_uint4(word[0], word[1], word[2], word[3]);
  }
  if (t == 0) sw[(size_t)g * (Np / 128) + np / 128] = scale;
}

// ---------------------------------------------------------------------------
// AddNorm + quantization: one wave per token row.  r = bf16(h + a) (the
// residual stream), x = gamma * r / sqrt(mean(r^2) + eps), then every group of
// 128 features of x quantized (Eqs. (7)-(8)).  Lane l holds features
// 512 j + 8 l .. +7; a group is 16 lanes of one 512-feature chunk.  Rows in
// [M, M_pad) get zero codes and scale 0.
// ---------------------------------------------------------------------------
template <int NCH>
__global__ __launch_bounds__(256) void fp8_addnorm_quant_kernel(const Fp8NormArgs a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = blockIdx.x * 4 + w;
  constexpr int D = NCH * 512, KG = D / 128, nch = NCH;
  const int gl = lane >> 4;                                     // group within the chunk
  uint8_t *xq = static_cast<uint8_t *>(a.xq);
  // byte offset of this lane's 8 codes of chunk j
  auto code_off = [&](int j) {
    const int k = 512 * j + 8 * lane;
    return fp8_pack_offset(m, k, KG);
  };
  if (m >= a.M) {
    for (int j = 0; j < nch; ++j) {
      *reinterpret_cast<uint2 *>(xq + code_off(j)) = make_uint2(0u, 0u);
      if ((lane & 15) == 0) a.sx[(size_t)(4 * j + gl) * a.M_pad + m] = 0.f;
    }
    return;
  }
  const bf16_t *h = static_cast<const bf16_t *>(a.h) + (size_t)m * D;
  const bf16_t *ad = static_cast<const bf16_t *>(a.a) + (size_t)m * D;
  const bf16_t *gm = static_cast<const bf16_t *>(a.gamma);
  bf16_t *r = static_cast<bf16_t *>(a.r) + (size_t)m * D;
  float rv[NCH][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const uint4 hu = *reinterpret_cast<const uint4 *>(h + 512 * j + 8 * lane);
    const uint4 au = *reinterpret_cast<const uint4 *>(ad + 512 * j + 8 * lane);
    const uint32_t hw[4] = {hu.x, hu.y, hu.z, hu.w}, aw[4] = {au.x, au.y, au.z, au.w};
    uint32_t ow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float s0 = __uint_as_float(hw[q] << 16) + __uint_as_float(aw[q] << 16);
      const float s1 = __uint_as_float(hw[q] & 0xffff0000u) + __uint_as_float(aw[q] & 0xffff0000u);
      const bf16_t b0 = f2bf(s0), b1 = f2bf(s1);
      rv[j][2 * q] = bf2f(b0);
      rv[j][2 * q + 1] = bf2f(b1);
      ss = fmaf(rv[j][2 * q], rv[j][2 * q], ss);
      ss = fmaf(rv[j][2 * q + 1], rv[j][2 * q + 1], ss);
      ow[q] = (uint32_t)b0 | ((uint32_t)b1 << 16);
    }
    *reinterpret_cast<uint4 *>(r + 512 * j + 8 * lane) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) ss += __shfl_xor(ss, o);
  const float inv = 1.0f / __fsqrt_rn(ss / (float)D + a.eps);
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const uint4 gu = *reinterpret_cast<const uint4 *>(gm + 512 * j + 8 * lane);
    const uint32_t gw[4] = {gu.x, gu.y, gu.z, gu.w};
    float x[8], amax = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = __uint_as_float(gw[q] << 16) * rv[j][2 * q] * inv;
      x[2 * q + 1] = __uint_as_float(gw[q] & 0xffff0000u) * rv[j][2 * q + 1] * inv;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = wave_max16(amax);
    const float scale = amax / kE4M3Max;
    uint2 c = make_uint2(0u, 0u);
    if (scale > 0.f) {
      c.x = e4m3_code4(x[0] / scale, x[1] / scale, x[2] / scale, x[3] / scale);
      c.y = e4m3_code4(x[4] / scale, x[5] / scale, x[6] / scale, x[7] / scale);
    }
    *reinterpret_cast<uint2 *>(xq + code_off(j)) = c;
    if ((lane & 15) == 0) a.sx[(size_t)(4 * j + gl) * a.M_pad + m] = scale;
  }
}

// ---------------------------------------------------------------------------
// FP8 GEMM: one workgroup of 8 waves per TM x TN output tile; wave w owns rows
// (w & 1) * TM/2 .. and its WCB column blocks (EPI_RESID: the (w >> 1)-th
// quarter of the tile's columns; EPI_SWIGLU: gate blocks 2 wn, 2 wn + 1 and
// the up blocks 8 + 2 wn, 9 + 2 wn of the same output features).  Groups of
// 128 pass through an NST-stage LDS ring of direct-to-LDS copies.
// ---------------------------------------------------------------------------
template <int TM, int TN> struct F8T {
  static constexpr int RB = TM / 16, CB = TN / 16;
  static constexpr int A_BYTES = RB * kF8Frag, B_BYTES = CB * kF8Frag, SA_BYTES = TM * 4, SW_BYTES = 256;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SW_BYTES;
  static constexpr int COPIES = (A_BYTES + B_BYTES) / 1024 / 8;  // 1 KB copies per wave per stage
  static constexpr int SA_COPIES = SA_BYTES / 256;               // 256-byte row-scale copies (waves 0 ..)
  // The tile's weight scales of the group (TN / 128 values) are one more
  // 256-byte copy, by wave 7.
  static constexpr int WRB = RB / 2, WCB = CB / 4;               // fragments per wave
  static_assert(COPIES * 8 * 1024 == A_BYTES + B_BYTES, "copies must tile the stage");
  static_assert(SA_COPIES <= 8, "scale copies");
};

enum { kEpiResid = 0, kEpiSwiglu = 1 };

template <int TM, int TN, int NST, int EPI>
__global__ __launch_bounds__(512) void fp8_gemm_kernel(const Fp8GemmArgs a) {
  using L = F8T<TM, TN>;
  static_assert(EPI != kEpiSwiglu || (TM == 256 && TN == 256), "SwiGLU tiles hold 128 features of both halves");
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1;
  // Tile order: workgroup wg runs on compute-die wg % 8 (the dispatcher deals
  // workgroups round-robin over the 8 dies); each die takes a contiguous run
  // of the tile sequence, which walks groups of kGM row tiles column tile by
  // column tile.  The ~32 workgroups a die runs at once then share 4 weight
  // tiles and 8 activation tiles through its L2.
  const int NX = a.N / TN, MY = a.M_pad / TM, ntiles = NX * MY;
  // Units: tile x split of the contraction (a tile's splits adjacent).
  const int S = EPI == kEpiResid && a.splits > 1 ? a.splits : 1, nunits = ntiles * S;
  const int per_die = (nunits + 7) / 8;
  const int wg = blockIdx.x;
  const int uu = (wg & 7) * per_die + (wg >> 3);
  if (uu >= nunits) return;                                    // whole workgroup: no barrier is skipped by part of it
  const int u = uu / S, split = uu % S;
  constexpr int kGM = 8;
  const int grp = u / (kGM * NX), within = u % (kGM * NX);
  const int gm = min(kGM, MY - grp * kGM);                     // row tiles in this (last, maybe partial) group
  const int m0 = (grp * kGM + within % gm) * TM, n0 = (within / gm) * TN;
  const int KGA = a.K / 128, NB = a.N / 128;
  const int kg0 = (int)((long)split * KGA / S), KG = (int)((long)(split + 1) * KGA / S) - kg0;   // this split's groups
  const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const char *Ab = static_cast<const char *>(a.A) + (size_t)(m0 >> 8) * KGA * kF8Tile + ((m0 & 255) >> 4) * kF8Frag;
  const char *Bb = static_cast<const char *>(a.B) + (size_t)(n0 >> 8) * KGA * kF8Tile + ((n0 & 255) >> 4) * kF8Frag;
  const int my_copies = L::COPIES + (w < L::SA_COPIES ? 1 : 0) + (w == 7 ? 1 : 0);

  auto issue = [&](int g) {
    const uint32_t st = lbase + (g % NST) * L::STAGE;
    const int gg = kg0 + g;                                    // absolute group
    const char *ag = Ab + (size_t)gg * kF8Tile, *bg = Bb + (size_t)gg * kF8Tile;
#pragma unroll
    for (int j = 0; j < L::COPIES; ++j) {
      const int c = w * L::COPIES + j;
      const char *src = c < 2 * L::RB ? ag + c * 1024 : bg + (c - 2 * L::RB) * 1024;
      dma16_s(src, lane_bytes(lane, 4), st + c * 1024);
    }
    if (w < L::SA_COPIES) dma4_s(a.sa + (size_t)gg * a.M_pad + m0 + w * 64, lane_bytes(lane, 2), st + L::A_BYTES + L::B_BYTES + w * 256);
    if (w == 7) dma4_s(a.sw + (size_t)gg * NB + n0 / 128, lane_bytes(min(lane, TN / 128 - 1), 2), st + L::A_BYTES + L::B_BYTES + L::SA_BYTES);
  };
  // The wave's column blocks within the tile.
  auto cb_of = [&](int j) {
    if constexpr (EPI == kEpiSwiglu) return (j < 2 ? 0 : 8) + 2 * wn + (j & 1);
    else return wn * L::WCB + j;
  };

  f32x4_t acc[L::WRB][L::WCB];
#pragma unroll
  for (int i = 0; i < L::WRB; ++i)
#pragma unroll
    for (int j = 0; j < L::WCB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int pro = KG < NST ? KG : NST;
  for (int s = 0; s < pro; ++s) issue(s);
  vmcnt_wait_rt<NST * (L::COPIES + 2)>((pro - 1) * my_copies);
  lds_barrier();

  for (int g = 0; g < KG; ++g) {
    const char *st = smem + (g % NST) * L::STAGE;
    // Operands of the first MFMA first: row fragment 0, then the column
    // fragments, then the row scales.
    i32x8_t afr[2];
    auto load_a = [&](int i) {
      const int rb = wm * L::WRB + i;
      const uint4 lo = *reinterpret_cast<const uint4 *>(st + rb * kF8Frag + lane * 16);
      const uint4 hi = *reinterpret_cast<const uint4 *>(st + rb * kF8Frag + 1024 + lane * 16);
      afr[i & 1] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    load_a(0);
    i32x8_t bfr[L::WCB];
    float swv[L::WCB];
#pragma unroll
    for (int j = 0; j < L::WCB; ++j) {
      const int cb = cb_of(j);
      const uint4 lo = *reinterpret_cast<const uint4 *>(st + L::A_BYTES + cb * kF8Frag + lane * 16);
      const uint4 hi = *reinterpret_cast<const uint4 *>(st + L::A_BYTES + cb * kF8Frag + 1024 + lane * 16);
      bfr[j] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      // wave-uniform: kept in a scalar register
      swv[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                   int, *reinterpret_cast<const float *>(st + L::A_BYTES + L::B_BYTES + L::SA_BYTES + 4 * (cb / 8)))));
    }
    // Row scales: an MFMA result's lane l holds rows 4 (l / 16) + v, v < 4,
    // of its 16-row block.  Lane l reads the scale of row 4 (l / 16) + l % 4,
    // so the four lanes of each quad hold exactly the four rows their
    // results need; a quad broadcast hands value v to every lane of the quad.
    // One 4-byte read per lane and row block instead of a replicated 16-byte one.
    float sar[L::WRB];
#pragma unroll
    for (int i = 0; i < L::WRB; ++i)
      sar[i] = *reinterpret_cast<const float *>(st + L::A_BYTES + L::B_BYTES +
                                                ((wm * L::WRB + i) * 16 + 4 * (lane >> 4) + (lane & 3)) * 4);
    // The wave's column blocks span one (EPI_RESID with 64 columns, or 32)
    // or two (EPI_SWIGLU: gate and up) 128-column weight blocks.
    constexpr int NSW = EPI == kEpiSwiglu ? 2 : 1, PER = L::WCB / NSW;
    // Scale of each lane's four result rows times the weight block's scale,
    // prepared one row block ahead of its FMAs.
    f32x4_t sc[2][NSW];
    auto prep = [&](int i) {
#pragma unroll
      for (int u = 0; u < NSW; ++u) {
        const float s1 = sar[i] * swv[u * PER];
        sc[i & 1][u] = f32x4_t{quad_bcast<0>(s1), quad_bcast<1>(s1), quad_bcast<2>(s1), quad_bcast<3>(s1)};
      }
    };
    prep(0);
    // Each MFMA's product is scaled and added one MFMA later, so a wave
    // issues the next MFMA before it waits for the previous result.
    f32x4_t tq[2];
    constexpr int NQ = L::WRB * L::WCB;
#pragma unroll
    for (int q = 0; q <= NQ; ++q) {
      const int i = q / L::WCB, j = q % L::WCB;
      if (q < NQ) {
        if (j == 0) {
          // Row block i + 1's fragment is read while row block i computes;
          // later ones stay unloaded (hoisted, they would need registers the
          // accumulators hold).
          asm volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          if (i + 1 < L::WRB) load_a(i + 1);
        }
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        tq[q & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr[i & 1], bfr[j], zero, 0, 0, 0, 127, 0, 127);
      }
      if (q > 0) {
        const int pi = (q - 1) / L::WCB, pj = (q - 1) % L::WCB;
        const f32x4_t t = tq[(q - 1) & 1], s4 = sc[pi & 1][pj / PER];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[pi][pj][v] = fmaf(t[v], s4[v], acc[pi][pj][v]);
      }
      if (q < NQ && j == L::WCB - 1 && i + 1 < L::WRB) prep(i + 1);
      // Issue order within a row block: each MFMA, then the previous
      // product's FMAs; the next row fragment's reads after the first MFMA,
      // the next row block's scales after the last.
      if (q < NQ) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (j == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (q > 0) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        if (j == L::WCB - 1 && i + 1 < L::WRB) __builtin_amdgcn_sched_group_barrier(0x002, 5 * NSW, 0);
      }
    }
    // The group's products are complete here, before the wait and barrier
    // below (sunk past them, every fragment of the group would be live at once).
#pragma unroll
    for (int i = 0; i < L::WRB; ++i)
#pragma unroll
      for (int j = 0; j < L::WCB; ++j) asm volatile("" : "+v"(acc[i][j]));
    if (g + 1 < KG) {
      // This wave's copies of group g + 1 landed (later ones may not have);
      // the barrier publishes the stage and frees stage g for group g + NST.
      const int behind = (KG - 2 - g) < (NST - 2) ? (KG - 2 - g) : (NST - 2);
      vmcnt_wait_rt<NST * (L::COPIES + 2)>(behind * my_copies);
      lds_barrier();
      if (g + NST < KG) issue(g + NST);
    }
  }
  __syncthreads();                                             // the ring's LDS is free

  if constexpr (EPI == kEpiResid) {
    // out = bf16(res + acc), staged per 16-row fragment through this wave's
    // LDS area so global traffic is row-wise 16-byte pieces.
    constexpr int COLS = 16 * L::WCB, STRIDE = COLS + 4, CPL = COLS / 4;   // CPL columns per lane (8 or 16)
    float *ws = reinterpret_cast<float *>(smem) + w * 16 * STRIDE;
    const int rr = lane >> 2, c0 = (lane & 3) * CPL;
    const int ncol = n0 + wn * COLS + c0;
    if (S > 1) {
      // Split partial: this split's fp32 sums, row-wise, for the reduction.
#pragma unroll
      for (int i = 0; i < L::WRB; ++i) {
#pragma unroll
        for (int j = 0; j < L::WCB; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) ws[(4 * (lane >> 4) + v) * STRIDE + 16 * j + (lane & 15)] = acc[i][j][v];
        wave_lds_sync();
        const int m = m0 + (wm * L::WRB + i) * 16 + rr;
        if (m < a.M) {
          float *dst = a.part + ((size_t)split * a.M + m) * a.N + ncol;
#pragma unroll
          for (int p = 0; p < CPL / 4; ++p)
            *reinterpret_cast<float4 *>(dst + 4 * p) =
                make_float4(ws[rr * STRIDE + c0 + 4 * p], ws[rr * STRIDE + c0 + 4 * p + 1],
                            ws[rr * STRIDE + c0 + 4 * p + 2], ws[rr * STRIDE + c0 + 4 * p + 3]);
        }
        wave_lds_sync();
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < L::WRB; ++i) {
#pragma unroll
      for (int j = 0; j < L::WCB; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) ws[(4 * (lane >> 4) + v) * STRIDE + 16 * j + (lane & 15)] = acc[i][j][v];
      wave_lds_sync();
      const int m = m0 + (wm * L::WRB + i) * 16 + rr;
      if (m < a.M) {
        const bf16_t *res = static_cast<const bf16_t *>(a.res) + (size_t)m * a.N + ncol;
        bf16_t *out = static_cast<bf16_t *>(a.out) + (size_t)m * a.N + ncol;
#pragma unroll
        for (int p = 0; p < CPL / 8; ++p) {
          const uint4 ru = *reinterpret_cast<const uint4 *>(res + 8 * p);
          const uint32_t rw[4] = {ru.x, ru.y, ru.z, ru.w};
          uint32_t ow[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float y0 = ws[rr * STRIDE + c0 + 8 * p + 2 * q] + __uint_as_float(rw[q] << 16);
            const float y1 = ws[rr * STRIDE + c0 + 8 * p + 2 * q + 1] + __uint_as_float(rw[q] & 0xffff0000u);
            ow[q] = (uint32_t)f2bf(y0) | ((uint32_t)f2bf(y1) << 16);
          }
          *reinterpret_cast<uint4 *>(out + 8 * p) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        }
      }
      wave_lds_sync();
    }
  } else {
    // SwiGLU: acc[i][0..1] are gate and acc[i][2..3] up of the same 32
    // output features of this wave (features 32 wn + 16 jj + lane % 16 of the
    // tile's 128).  y = silu(gate) * up, one 128-feature group per row over
    // the 4 waves of a row half: maxima meet in LDS, then codes go to LDS in
    // the packed layout of the down projection's operand and leave as one
    // contiguous 32 KB block (rows m0.., group n0 / 256 of the down projection).
    float *s_amax = reinterpret_cast<float *>(smem);                       // [4 wn][256 rows]
    uint8_t *s_codes = reinterpret_cast<uint8_t *>(smem) + 4 * 256 * 4;    // 32 KB
#pragma unroll
    for (int i = 0; i < L::WRB; ++i) {
      float pm[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const float gt = acc[i][jj][v], up = acc[i][2 + jj][v];
          acc[i][jj][v] = gt / (1.0f + fast_exp2(-gt * kLog2e)) * up;
        }
        pm[v] = wave_max16(fmaxf(fabsf(acc[i][0][v]), fabsf(acc[i][1][v])));
      }
      if ((lane & 15) == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s_amax[wn * 256 + wm * 128 + i * 16 + 4 * (lane >> 4) + v] = pm[v];
      }
    }
    __syncthreads();
    const int KG2 = a.N / 256;                                 // groups of the down projection's operand
#pragma unroll
    for (int i = 0; i < L::WRB; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 128 + i * 16 + 4 * (lane >> 4) + v;
        const float amax = fmaxf(fmaxf(s_amax[row], s_amax[256 + row]), fmaxf(s_amax[512 + row], s_amax[768 + row]));
        const float scale = amax / kE4M3Max;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const uint32_t c = scale > 0.f ? e4m3_code(acc[i][jj][v] / scale) : 0u;
          s_codes[(wm * 8 + i) * kF8Frag + jj * 1024 + (16 * wn + 4 * (lane >> 4) + v) * 16 + (lane & 15)] = (uint8_t)c;
        }
        if (wn == 0 && (lane & 15) == 0) a.sy[(size_t)(n0 / TN) * a.M_pad + m0 + row] = scale;
      }
    }
    __syncthreads();
    uint4 *dst = reinterpret_cast<uint4 *>(static_cast<uint8_t *>(a.yq) + ((size_t)(m0 >> 8) * KG2 + n0 / TN) * kF8Tile);
    const uint4 *srcl = reinterpret_cast<const uint4 *>(s_codes);
#pragma unroll
    for (int p = 0; p < kF8Tile / 16 / 512; ++p) dst[p * 512 + tid] = srcl[p * 512 + tid];
  }
}

// out = bf16(res + the sum of the split partials, in split order): one
// thread per 8 consecutive outputs of a row.
__global__ __launch_bounds__(256) void fp8_splitk_reduce_kernel(const Fp8GemmArgs a) {
  const int per_row = a.N / 8;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.M * per_row) return;
  const int m = (int)(idx / per_row), n = (int)(idx % per_row) * 8;
  const float *p = a.part + (size_t)m * a.N + n;
  const size_t sstride = (size_t)a.M * a.N;
  float y[8] = {};
  for (int sp = 0; sp < a.splits; ++sp, p += sstride) {
    const float4 u0 = *reinterpret_cast<const float4 *>(p), u1 = *reinterpret_cast<const float4 *>(p + 4);
    y[0] += u0.x; y[1] += u0.y; y[2] += u0.z; y[3] += u0.w;
    y[4] += u1.x; y[5] += u1.y; y[6] += u1.z; y[7] += u1.w;
  }
  const uint4 ru = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.res) + (size_t)m * a.N + n);
  const uint32_t rw[4] = {ru.x, ru.y, ru.z, ru.w};
  uint32_t ow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float y0 = y[2 * q] + __uint_as_float(rw[q] << 16), y1 = y[2 * q + 1] + __uint_as_float(rw[q] & 0xffff0000u);
    ow[q] = (uint32_t)f2bf(y0) | ((uint32_t)f2bf(y1) << 16);
  }
  *reinterpret_cast<uint4 *>(static_cast<bf16_t *>(a.out) + (size_t)m * a.N + n) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
size_t fp8_packed_bytes(int N, int K) { return (size_t)((N + 255) / 256) * (K / 128) * kF8Tile; }

namespace {
// Splits of a down projection on 128 x 128 tiles that leaves compute units
// idle and contracts over many 128-wide groups (768 rows of LLaDA-8B's FFN:
// 192 tiles, 96 groups): two halves of at least kF8SplitGroups groups, run
// with two-stage rings so that two workgroups share a CU.  Measured there:
// 82 us whole, 73 us in two, 75 us in four, 87 us in six (the fp32
// partials' traffic grows with the count).
constexpr int kF8SplitGroups = 24;
int fp8_splits(int N, int M_pad, int K) {
  const long tiles = (long)(N / 128) * (M_pad / 128);
  if (tiles >= device_cus()) return 1;
  return (K / 128) / kF8SplitGroups >= 2 ? 2 : 1;
}
bool fp8_resid_big(int N, int M_pad, int tile) {
  return tile == 1 || (tile == 0 && (long)(N / 256) * (M_pad / 256) >= device_cus());
}
}  // namespace

size_t fp8_part_bytes(int M, int M_pad, int N, int K, int tile) {
  if (M <= 0 || N % 256 || K % 128 || M_pad % 256 || fp8_resid_big(N, M_pad, tile)) return 0;
  const int sp = fp8_splits(N, M_pad, K);
  return sp > 1 ? (size_t)sp * M * N * sizeof(float) : 0;
}

hipError_t launch_fp8_pack_weight(const void *W, int N, int K, int mode, void *Wp, float *sw, int Np, hipStream_t s) {
  if (N % 128 || K % 128 || N <= 0 || K <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fp8_pack_weight_kernel, dim3(N / 128, K / 128), dim3(256), 0, s, static_cast<const bf16_t *>(W),
                     N, K, mode, static_cast<uint8_t *>(Wp), sw, Np);
  return hipGetLastError();
}

hipError_t launch_fp8_addnorm_quant(const Fp8NormArgs &a, hipStream_t s, const LaunchEvents &ev) {
  if (a.M_pad <= 0) return hipSuccess;
  if (a.M_pad % 256) return hipErrorInvalidValue;
  switch (a.D) {
    case 512: lc_launch<fp8_addnorm_quant_kernel<1>>(dim3(a.M_pad / 4), dim3(256), 0, s, ev, a); break;
    case 1024: lc_launch<fp8_addnorm_quant_kernel<2>>(dim3(a.M_pad / 4), dim3(256), 0, s, ev, a); break;
    case 2048: lc_launch<fp8_addnorm_quant_kernel<4>>(dim3(a.M_pad / 4), dim3(256), 0, s, ev, a); break;
    case 4096: lc_launch<fp8_addnorm_quant_kernel<8>>(dim3(a.M_pad / 4), dim3(256), 0, s, ev, a); break;
    case 8192: lc_launch<fp8_addnorm_quant_kernel<16>>(dim3(a.M_pad / 4), dim3(256), 0, s, ev, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int TM, int TN, int NST> constexpr int fp8_gemm_smem() { return NST * F8T<TM, TN>::STAGE; }
// Workgroups for `tiles` output tiles: a multiple of the 8 compute dies (the
// kernel's tile order gives each die a contiguous run; surplus workgroups exit).
inline unsigned fp8_grid(int tiles) { return (unsigned)((tiles + 7) / 8 * 8); }

hipError_t launch_fp8_gemm_swiglu(const Fp8GemmArgs &a, hipStream_t s, const LaunchEvents &ev) {
  if (a.M_pad <= 0) return hipSuccess;
  if (a.N % 256 || a.K % 128 || a.M_pad % 256) return hipErrorInvalidValue;
  lc_launch<fp8_gemm_kernel<256, 256, 2, kEpiSwiglu>>(dim3(fp8_grid(a.N / 256 * (a.M_pad / 256))), dim3(512),
                                                      fp8_gemm_smem<256, 256, 2>(), s, ev, a);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm_resid(const Fp8GemmArgs &a, int tile, hipStream_t s, const LaunchEvents &ev) {
  if (a.M_pad <= 0) return hipSuccess;
  if (a.N % 256 || a.K % 128 || a.M_pad % 256) return hipErrorInvalidValue;
  // 256 x 256 tiles when they give every compute unit a workgroup, else 128 x 128.
  Fp8GemmArgs b = a;
  b.splits = 1;
  if (fp8_resid_big(a.N, a.M_pad, tile)) {
    lc_launch<fp8_gemm_kernel<256, 256, 2, kEpiResid>>(dim3(fp8_grid(a.N / 256 * (a.M_pad / 256))), dim3(512),
                                                       fp8_gemm_smem<256, 256, 2>(), s, ev, b);
    return hipGetLastError();
  }
  const int tiles = a.N / 128 * (a.M_pad / 128);
  if (a.part) b.splits = fp8_splits(a.N, a.M_pad, a.K);
  if (b.splits == 1) {
    lc_launch<fp8_gemm_kernel<128, 128, 4, kEpiResid>>(dim3(fp8_grid(tiles)), dim3(512), fp8_gemm_smem<128, 128, 4>(), s,
                                                       ev, b);
    return hipGetLastError();
  }
  // The two launches share one event pair: the first stamps the start, the last the end.
  const LaunchEvents first{ev.start, nullptr}, last{nullptr, ev.stop};
  lc_launch<fp8_gemm_kernel<128, 128, 2, kEpiResid>>(dim3(fp8_grid((long)tiles * b.splits)), dim3(512),
                                                     fp8_gemm_smem<128, 128, 2>(), s, first, b);
  const long threads = (long)a.M * (a.N / 8);
  lc_launch<fp8_splitk_reduce_kernel>(dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, last, b);
  return hipGetLastError();
}

hipError_t setup_fp8_attributes() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fp8_gemm_kernel<256, 256, 2, kEpiSwiglu>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, fp8_gemm_smem<256, 256, 2>());
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(fp8_gemm_kernel<256, 256, 2, kEpiResid>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, fp8_gemm_smem<256, 256, 2>());
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(fp8_gemm_kernel<128, 128, 4, kEpiResid>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, fp8_gemm_smem<128, 128, 4>());
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(fp8_gemm_kernel<128, 128, 2, kEpiResid>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, fp8_gemm_smem<128, 128, 2>());
  return e;
}

}  // namespace lc
