// The skinny QKV projection with the prep kernel's work folded in, as a
// device function: the body of qkv_skinny_fused_kernel (gemm.hip) and the
// projection role of the fused block-step kernel (attn.hip).  Also the
// tiling constants and helpers the packed weight's layout defines.
#pragma once

#include <type_traits>
#include <utility>

#include "internal.h"

namespace lc {

typedef _Float16 gh2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f16pair(float a, float b) {
  const gh2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Tiling shared by prep, the pack kernel and the GEMMs.
constexpr int kGBM = 128, kGBN = 192, kGBK = 64, kGStages = 4, kGWaves = 8;
constexpr int kGStageA = kGBM * kGBK * 2;          // bytes: fp16 A tile
constexpr int kGStageW = kGBN * kGBK * 2;          // bytes: W tile (fp16; bf16 until converted)
constexpr int kGStage = kGStageA + kGStageW;
constexpr int kGemmSmem = kGStages * kGStage;      // 160 KB
constexpr int kGCopyA = kGStageA / 1024 / kGWaves;  // copy instructions per wave per stage (1 KB each)
constexpr int kGCopyW = kGStageW / 1024 / kGWaves;
constexpr int kGCopies = kGCopyA + kGCopyW;
static_assert(kGCopyA * 1024 * kGWaves == kGStageA && kGCopyW * 1024 * kGWaves == kGStageW, "copy tiling");

// Byte offset of fragment (row block rb, contraction half ks) in a fragment-major tile.
__device__ __forceinline__ int frag_off(int rb, int ks) { return (rb * 2 + ks) << 10; }

template <int I, int N> struct Unroll {
  template <class F> __device__ __forceinline__ static void run(F &f) {
    f(std::integral_constant<int, I>{});
    Unroll<I + 1, N>::run(f);
  }
};
template <int N> struct Unroll<N, N> {
  template <class F> __device__ __forceinline__ static void run(F &) {}
};

// The skinny GEMM with the prep kernel's work folded in (block steps and
// prefill passes of at most 64 tokens): every workgroup gathers the launch's
// embedding rows itself, in the operand layout, straight from the table
// (the few rows stay in L2), converts gamma * E to fp16 while they wait in
// registers, and adds up each token's sum of squares on the way.  The
// matrix cores contract fp16(gamma * E) with the weight, so the RMS factor
// 1 / sqrt(mean(E^2) + eps) multiplies the fp32 sums in the epilogue,
// before RoPE.  Workgroups also write the EmbedCache rows, one 64-wide slice
// of 16 tokens each.  One launch instead of two: no round trip through the
// activation workspace and no launch boundary.
// A workgroup of 512 threads owns the three 16-column fragments cb0, cb1,
// cb2 of the packed weight (global fragment indices; their features follow
// from the fragment: head cb / (d_h / 16), the 8 RoPE pairs of the
// fragment).  wg / nwg: this workgroup's index among the nwg that share
// the EmbedCache writes (and the first reports bad ids).  smem: at least
// skinny_fused_smem<TB, NPW>() bytes.
template <int DH, int TB, int NPW, bool CONTIG>
__device__ __forceinline__ void skinny_project(const SeqArgs &sa, const PrepArgs &p, const GemmArgs &a, char *smem,
                                               int wg, int nwg, int cb0, int cb1, int cb2) {
  constexpr int NFB = 3, NBLK = NFB * TB, D = 512 * NPW;
  constexpr int RED = 8 * NBLK * 64 * 16;                        // partial sums of the 8 waves
  float *s_gamma = reinterpret_cast<float *>(smem + RED);        // [D]
  float *s_ss = s_gamma + D;                                     // [8 waves][64 tokens]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int cbh = DH / 16, ncb = a.F / 16;
  // A tile of the packed weight holds kGBN / 16 fragments over D / 64
  // contraction tiles.  CONTIG: fragments cb0 .. cb0 + 2 of one tile (one
  // base); otherwise each fragment from its own tile.
  const int cbs[NFB] = {cb0, cb1, cb2};
  const char *wt[NFB];                                           // workgroup-uniform bases
#pragma unroll
  for (int f = 0; f < NFB; ++f)
    wt[f] = static_cast<const char *>(a.Wp) + (size_t)(cbs[f] / (kGBN / 16)) * 8 * NPW * kGStageW +
            frag_off(cbs[f] % (kGBN / 16), 0);
  const char *wt0 = static_cast<const char *>(a.Wp) + (size_t)(cb0 / (kGBN / 16)) * 8 * NPW * kGStageW +
                    frag_off(cb0 % (kGBN / 16), 0) + lane * 16;
  const uint32_t wlane = (uint32_t)lane * 16u;

  struct Tile {
    uint4 w[NFB][2];
    uint4 x[TB][2];
  };
  auto fetch_w = [&](Tile &t, int kt) {
    if constexpr (CONTIG) {
      const char *wp = wt0 + (size_t)kt * kGStageW;
#pragma unroll
      for (int f = 0; f < NFB; ++f)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) t.w[f][ks] = *reinterpret_cast<const uint4 *>(wp + frag_off(f, ks));
    } else {
#pragma unroll
      for (int f = 0; f < NFB; ++f)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          t.w[f][ks] = *reinterpret_cast<const uint4 *>(wt[f] + (size_t)kt * kGStageW + (ks << 10) + wlane);
    }
  };

  // Lane l of every wave resolves token l (clamped to the launch): its
  // embedding row (row 0 for an out-of-range id, zeroed below), cache row
  // and position, as the prep kernel does.  The sample of token mg is the
  // last whose first token is <= mg (the loop runs over samples, so every
  // table read is wave-uniform).
  int dst_l, pos_l, id_raw;
  {
    const int mg = p.row0 + min(lane, p.M - 1);
    int off = 0, bs = 0, first = 0;
    for (int i = 0; i < sa.n; ++i) {
      const int st = sa.pre[0][i];
      if (st <= mg) {
        off = sa.off[i];
        bs = sa.bs[i];
        first = st;
      }
    }
    const int local = mg - first;
    if (p.mode == 0) {
      dst_l = off + bs + local;
      pos_l = bs + local;
      id_raw = p.ids[p.ids_base + mg];
    } else {
      dst_l = off + local;
      pos_l = local;
      id_raw = p.ids[dst_l];
    }
  }
  constexpr int GPT = (D / 8 + 511) / 512;                      // gamma pieces per thread
  uint4 graw[GPT];
#pragma unroll
  for (int j = 0; j < GPT; ++j) graw[j] = static_cast<const uint4 *>(p.gamma)[min(tid + 512 * j, D / 8 - 1)];

  // The weight stream starts before the ids arrive.  Tiles in flight: three
  // ahead for two token blocks, two for four (the conversions need the
  // registers).
  constexpr int PD = TB <= 2 ? 3 : 2;
  Tile tl[PD];
#pragma unroll
  for (int j = 0; j < PD; ++j)
    if (j < NPW) fetch_w(tl[j], w + 8 * j);
  __builtin_amdgcn_sched_barrier(0);

  const bool bad_l = id_raw < 0 || id_raw >= p.vocab;
  const int id_l = bad_l ? 0 : id_raw;
  if (bad_l && lane < p.M && wg == 0 && w == 0) atomicOr(p.flags, 1u);

  // The embedding rows move row-wise (the load unit's full-rate pattern):
  // load j of a k-tile brings tokens 8j .. 8j+7, lane l holding 16 bytes
  // (piece l & 7) of token 8j + l/8.  Offsets are 32-bit byte offsets from
  // the table (the launcher checks that it is below 4 GB).
  const bf16_t *E = static_cast<const bf16_t *>(p.E);
  const char *Eb = static_cast<const char *>(p.E);
  const int c8 = lane & 7, t8 = lane >> 3;
  uint32_t eoff[2 * TB], badbits = 0;                          // bit j: token 8j + l/8 has a bad id
#pragma unroll
  for (int j = 0; j < 2 * TB; ++j) {
    const int id = __shfl(id_l, 8 * j + t8);
    badbits |= (uint32_t)__shfl((int)bad_l, 8 * j + t8) << j;
    eoff[j] = (uint32_t)id * (uint32_t)(2 * D) + 16u * (uint32_t)c8;
  }
  auto fetch_x = [&](Tile &t, int kt) {
#pragma unroll
    for (int j = 0; j < 2 * TB; ++j)
      t.x[j >> 1][j & 1] = *reinterpret_cast<const uint4 *>(Eb + (size_t)(eoff[j] + (uint32_t)(kt * 128)));
  };
  auto fetch = [&](Tile &t, int kt) {
    fetch_w(t, kt);
    fetch_x(t, kt);
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int j = 0; j < PD; ++j)
    if (j < NPW) fetch_x(tl[j], w + 8 * j);
  __builtin_amdgcn_sched_barrier(0);

  // EmbedCache rows: slice (token block, 64-wide column tile) of this
  // workgroup, by wave 0 (lane: token lane/4, two 16-byte pieces).  Its
  // wait for these loads also covers the first tiles, which step 0 needs
  // at about the same time.
  if (w == 0) {
    for (int sl = wg; sl < TB * 8 * NPW; sl += nwg) {
      const int tb = sl / (8 * NPW), kt = sl % (8 * NPW);
      const int tok = tb * 16 + (lane >> 2);
      const int src_l = min(tok, 63);
      const int id = __shfl(id_l, src_l), dst = __shfl(dst_l, src_l);
      const uint32_t m = __shfl((int)bad_l, src_l) ? 0u : ~0u;
      const uint4 *src = reinterpret_cast<const uint4 *>(E + (size_t)id * D + kt * 64) + (lane & 3) * 2;
      uint4 v0 = src[0], v1 = src[1];
      v0 = make_uint4(v0.x & m, v0.y & m, v0.z & m, v0.w & m);
      v1 = make_uint4(v1.x & m, v1.y & m, v1.z & m, v1.w & m);
      if (tok < p.M) {
        uint4 *hrow = reinterpret_cast<uint4 *>(static_cast<bf16_t *>(p.h) + (size_t)dst * D + kt * 64) + (lane & 3) * 2;
        hrow[0] = v0;
        hrow[1] = v1;
      }
    }
  }

  // gamma as fp32 in LDS (read by every step's conversion).
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int pc = tid + 512 * j;
    if (pc < D / 8) {
      const uint32_t gw[4] = {graw[j].x, graw[j].y, graw[j].z, graw[j].w};
      float4 lo, hi;
      lo.x = __uint_as_float(gw[0] << 16); lo.y = __uint_as_float(gw[0] & 0xffff0000u);
      lo.z = __uint_as_float(gw[1] << 16); lo.w = __uint_as_float(gw[1] & 0xffff0000u);
      hi.x = __uint_as_float(gw[2] << 16); hi.y = __uint_as_float(gw[2] & 0xffff0000u);
      hi.z = __uint_as_float(gw[3] << 16); hi.w = __uint_as_float(gw[3] & 0xffff0000u);
      reinterpret_cast<float4 *>(s_gamma)[2 * pc] = lo;
      reinterpret_cast<float4 *>(s_gamma)[2 * pc + 1] = hi;
    }
  }
  lds_barrier();

  f32x4_t acc[NFB][TB];
#pragma unroll
  for (int f = 0; f < NFB; ++f)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[f][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float ss[2 * TB] = {};                                         // token 8j + l/8, this lane's pieces
  float amax = 0.f;                                             // largest |gamma * E| (fp16 range check)
  // fp16 operand tile of the step, row-major with 16-byte piece p of token
  // t in slot p ^ (t & 7) (fragment reads of 16 tokens spread over the
  // banks); inside this wave's own part of the reduction area.
  char *xs = smem + w * NBLK * 64 * 16;
  auto step = [&](auto IC) {
    constexpr int i = decltype(IC)::value;
    Tile &cur = tl[i % PD];
    const int kt = w + 8 * i;
    // Nothing of a later step (its gamma reads, conversions) moves up here.
    __builtin_amdgcn_sched_barrier(0);
    {
      const float4 ga = reinterpret_cast<const float4 *>(s_gamma + kt * 64 + 8 * c8)[0];
      const float4 gb = reinterpret_cast<const float4 *>(s_gamma + kt * 64 + 8 * c8)[1];
      const float gm[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
      for (int j = 0; j < 2 * TB; ++j) {
        const uint4 raw = cur.x[j >> 1][j & 1];
        const uint32_t xm = (badbits >> j) & 1u ? 0u : ~0u;
        const uint32_t u[4] = {raw.x & xm, raw.y & xm, raw.z & xm, raw.w & xm};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e0 = __uint_as_float(u[q] << 16), e1 = __uint_as_float(u[q] & 0xffff0000u);
          ss[j] = fmaf(e0, e0, fmaf(e1, e1, ss[j]));
          const float y0 = e0 * gm[2 * q], y1 = e1 * gm[2 * q + 1];
          amax = fmaxf(amax, fmaxf(fabsf(y0), fabsf(y1)));
          o[q] = f16pair(y0, y1);
        }
        const int t = 8 * j + t8;
        *reinterpret_cast<uint4 *>(xs + t * 128 + ((c8 ^ (t & 7)) << 4)) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Frag<f16_t> fx[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const int t = b * 16 + r16;
        fx[b].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(xs + t * 128 + (((ks * 4 + g) ^ (t & 7)) << 4)));
      }
#pragma unroll
      for (int f = 0; f < NFB; ++f) {
        Frag<f16_t> fw;
        fw.v = __builtin_bit_cast(f16x8_t, cur.w[f][ks]);
#pragma unroll
        for (int b = 0; b < TB; ++b) mma16(acc[f][b], fw, fx[b]);
      }
    }
    // The step's squares and range check are finished here, not carried to
    // the end (which would keep every converted value live until then).
    asm volatile("" : "+v"(amax));
#pragma unroll
    for (int j = 0; j < 2 * TB; ++j) asm volatile("" : "+v"(ss[j]));
    if (i + PD < NPW) fetch(cur, w + 8 * (i + PD));
  };
  Unroll<0, NPW>::run(step);

  // Partial sums and sums of squares of the 8 waves, then wave w finishes
  // blocks w, w + 8 (fixed order: results do not depend on the token count).
  f32x4_t *red = reinterpret_cast<f32x4_t *>(smem);
#pragma unroll
  for (int f = 0; f < NFB; ++f)
#pragma unroll
    for (int b = 0; b < TB; ++b) red[(w * NBLK + f * TB + b) * 64 + lane] = acc[f][b];
  // (The reduction area overlaps this wave's own operand tile only.)
#pragma unroll
  for (int j = 0; j < 2 * TB; ++j) {
    float t = ss[j];
    t += __shfl_xor(t, 1);
    t += __shfl_xor(t, 2);
    t += __shfl_xor(t, 4);
    if (c8 == 0) s_ss[w * 64 + 8 * j + t8] = t;
  }
  __syncthreads();
  bool range = amax <= kF16Max;
  const int nrot = (a.H + a.Hkv) * DH, qf = a.H * DH, kf = a.Hkv * DH;
  for (int blk = w; blk < NBLK; blk += 8) {
    f32x4_t y = red[blk * 64 + lane];
#pragma unroll
    for (int ww = 1; ww < 8; ++ww) y += red[(ww * NBLK + blk) * 64 + lane];
    const int f = blk / TB, b = blk % TB;
    const int cb = CONTIG ? cb0 + f : f == 0 ? cb0 : f == 1 ? cb1 : cb2;
    const int tok = b * 16 + r16;
    float sst = s_ss[tok];
#pragma unroll
    for (int ww = 1; ww < 8; ++ww) sst += s_ss[ww * 64 + tok];
    const float rr = rsqrtf(sst / (float)D + p.eps);
    const int dst = __shfl(dst_l, tok), pos = __shfl(pos_l, tok);
    if (cb >= ncb || tok >= a.M) continue;
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    y *= rr;
    float o0 = y[0], o1 = y[1], o2 = y[2], o3 = y[3];
    if (hh * DH < nrot) {
      const uint4 c = *reinterpret_cast<const uint4 *>(p.rope + (size_t)pos * (DH / 2) + p0 + 2 * g);
      const float c0 = __uint_as_float(c.x), s0 = __uint_as_float(c.y);
      const float c1 = __uint_as_float(c.z), s1 = __uint_as_float(c.w);
      o0 = y[0] * c0 - y[1] * s0;
      o1 = y[1] * c0 + y[0] * s0;
      o2 = y[2] * c1 - y[3] * s1;
      o3 = y[3] * c1 + y[2] * s1;
    }
    range = range && fabsf(o0) <= kF16Max && fabsf(o1) <= kF16Max && fabsf(o2) <= kF16Max && fabsf(o3) <= kF16Max;
    const int fa = hh * DH + p0 + 2 * g, fbf = fa + DH / 2;   // first-half pair, partners
    f16_t *base;
    size_t off;                                              // cache rows reach 2^31 / (H d_h) and beyond
    if (fa < qf) { base = static_cast<f16_t *>(a.q); off = (size_t)dst * qf + fa; }
    else if (fa < qf + kf) { base = static_cast<f16_t *>(a.k); off = (size_t)dst * kf + (fa - qf); }
    else { base = static_cast<f16_t *>(a.v); off = (size_t)dst * kf + (fa - qf - kf); }
    *reinterpret_cast<uint32_t *>(base + off) = f16pair(o0, o2);
    *reinterpret_cast<uint32_t *>(base + off + (fbf - fa)) = f16pair(o1, o3);
  }
  if (!range) atomicOr(a.flags, 2u);
}
template <int TB, int NPW> constexpr int skinny_fused_smem() { return 8 * 3 * TB * 64 * 16 + 512 * NPW * 4 + 8 * 64 * 4; }

}  // namespace lc
