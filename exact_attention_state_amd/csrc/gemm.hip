// First-layer token-wise operators for many tokens at once (the block step
// of a large batch, and the refresh): LaCache Section 3.3.2, Eq. (1) -
// embedding gather (EmbedCache write), RMSNorm, QKV projection on MFMA, RoPE
// and the Q/K/V cache write - as two kernels.
//
//   prep   one wave per token: gathers E[x], writes the EmbedCache row,
//          forms the normalised activation A = fp16(gamma * E[x] * r),
//          r = 1/sqrt(mean(E[x]^2) + eps), and the token's (cache row,
//          position) and the RoPE (cos, sin) row of its position into the
//          workspace.
//   gemm   C = A W^T on v_mfma_f32_16x16x32_f16, then RoPE and the fp16
//          cache write in the epilogue.
//
// Operand tiles: 128 tokens x 64 contraction elements of A (16 KB) and 192
// GEMM columns x 64 elements of W (24 KB) per stage of a 4-stage LDS ring,
// filled global -> LDS by the load unit (global_load_lds_dwordx4).  (The
// packed GEMM can also take half of the 192 columns per workgroup when whole
// tiles would leave half of the chip idle, or 256 tokens x 192 columns in
// 32-wide contraction stages for large launches; both with a 5-stage ring
// of 28 KB stages.)  A tile
// row is 128 bytes; its 16-byte piece p sits in slot p ^ ((r >> 1) & 7), so
// the 16 rows of one MFMA operand read hit all 64 banks once.  prep writes A
// in exactly that tile order ([row tile][contraction tile][128 x 64],
// swizzled), so each 1 KB copy instruction reads 1 KB of contiguous memory.
//
// Two GEMM kernels, by the form of W:
//   packed  W converted once to fp16 in the same tile order (see
//           pack_qkv_weight_kernel): contiguous copies, no conversion in the
//           loop.  The contraction is split over two groups of four waves
//           (64 or 32 tokens x 96 columns per wave); the kernel computes C^T so a
//           lane's four accumulator values are four GEMM columns of one token,
//           and the column order puts both members of two RoPE pairs in one
//           lane: RoPE needs no lane exchange.
//   bf16    W as stored, row-major bf16: rows gathered per copy, each wave
//           converts the pieces it copied to fp16 in place one tile ahead,
//           between the MFMAs of the current tile; 8 waves of 64 x 48.
// Both convert bf16 weights to fp16 the same way (exact for weights in
// fp16's normal range).  Consecutive workgroups take consecutive column
// tiles, so the row tiles of one column tile land on one XCD and share its
// weight tile in that XCD's L2.
//
// Precision: one fp16 rounding of the normalised activation (11-bit
// significand, 8x finer than bf16) and fp32 accumulation; the small-batch
// kernel instead keeps gamma * E exact with a bf16 hi/lo split, which costs
// twice the matrix-core work - affordable only where the step is bound by
// streaming the weights.

#include <type_traits>
#include <utility>

#include "internal.h"

namespace lc {

typedef _Float16 gh2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f16pair(float a, float b) {
  const gh2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// tiling shared by prep, the pack kernel and the GEMMs
// ---------------------------------------------------------------------------
constexpr int kGBM = 128, kGBN = 192, kGBK = 64, kGStages = 4, kGWaves = 8;
constexpr int kGStageA = kGBM * kGBK * 2;          // bytes: fp16 A tile
constexpr int kGStageW = kGBN * kGBK * 2;          // bytes: W tile (fp16; bf16 until converted)
constexpr int kGStage = kGStageA + kGStageW;
constexpr int kGemmSmem = kGStages * kGStage;      // 160 KB
constexpr int kGCopyA = kGStageA / 1024 / kGWaves;  // copy instructions per wave per stage (1 KB each)
constexpr int kGCopyW = kGStageW / 1024 / kGWaves;
constexpr int kGCopies = kGCopyA + kGCopyW;
static_assert(kGCopyA * 1024 * kGWaves == kGStageA && kGCopyW * 1024 * kGWaves == kGStageW, "copy tiling");

__device__ __forceinline__ int gslot(int r, int p) { return p ^ ((r >> 1) & 7); }
__device__ __forceinline__ int gswz(int r, int p) { return r * 128 + (gslot(r, p) << 4); }

// Fragment-major operand tiles.  An MFMA operand fragment (16 rows x 32
// contraction elements, lane g*16 + r holding row r, elements 8g..8g+7) is
// one contiguous KB in lane order, so a wave loads it with consecutive lanes
// on consecutive 16-byte pieces (the load unit's full-rate pattern) and
// reads it back from LDS without bank conflicts.  A 64-wide contraction tile
// of 16*R rows is 2R fragments, fragment (row block rb, half ks) at KB
// 2 rb + ks.
// Byte offset, in the tiled A ([M_pad/128][D/64][128 x 64]), of the
// 8-element piece starting at element e (a multiple of 8) of token row m;
// nk = D / 64.
__device__ __forceinline__ size_t a_piece(int m, int e, int nk) {
  return ((size_t)(m >> 7) * nk + (e >> 6)) * kGStageA + ((((m & 127) >> 4) * 2 + ((e >> 5) & 1)) << 10) +
         ((((e >> 3) & 3) * 16 + (m & 15)) << 4);
}
__device__ __forceinline__ int frag_off(int rb, int ks) { return (rb * 2 + ks) << 10; }

// ---------------------------------------------------------------------------
// prep: one wave per token row m of the launch (rows past M of the padded
// tile are written as zeros).  Each lane owns D/64 consecutive elements.
// ---------------------------------------------------------------------------
// NP = D / 512: 16-byte pieces per lane; lane l moves pieces l, l + 64, ...
// of a row (consecutive lanes on consecutive pieces), all in one round trip.
template <int NP>
__global__ __launch_bounds__(256) void qkv_prep_kernel(const SeqArgs sa, const PrepArgs a) {
  constexpr int D = NP * 512, nk = D / kGBK;
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= a.M_pad) return;
  char *abase = static_cast<char *>(a.A);
  float2 *csrow = a.cs + (size_t)m * (a.dh / 2);
  if (m >= a.M) {
#pragma unroll
    for (int j = 0; j < NP; ++j)
      *reinterpret_cast<uint4 *>(abase + a_piece(m, (j * 64 + lane) * 8, nk)) = make_uint4(0, 0, 0, 0);
    if (lane < a.dh / 2) csrow[lane] = make_float2(0.f, 0.f);
    return;
  }
  const int mg = a.row0 + m;                       // token index within the whole call
  const int b = find_sample(sa.pre[0], sa.n, mg);
  const int local = mg - sa.pre[0][b];
  int dst, pos, id;
  if (a.mode == 0) {
    dst = sa.off[b] + sa.bs[b] + local;
    pos = sa.bs[b] + local;
    id = a.ids[a.ids_base + mg];
  } else {
    dst = sa.off[b] + local;
    pos = local;
    id = a.ids[dst];
  }
  const bool bad = id < 0 || id >= a.vocab;
  if (bad && lane == 0) atomicOr(a.flags, 1u);
  // Unconditional loads (a bad id reads row 0 and is zeroed after).
  const uint4 *erow = reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.E) + (size_t)(bad ? 0 : id) * D);
  const uint4 *grow = static_cast<const uint4 *>(a.gamma);
  uint4 ev[NP], gv[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) ev[j] = erow[j * 64 + lane];
#pragma unroll
  for (int j = 0; j < NP; ++j) gv[j] = grow[j * 64 + lane];
  const float2 csv = a.rope[(size_t)pos * (a.dh / 2) + min(lane, a.dh / 2 - 1)];
  uint4 *hrow = reinterpret_cast<uint4 *>(static_cast<bf16_t *>(a.h) + (size_t)dst * D);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    if (bad) ev[j] = make_uint4(0, 0, 0, 0);
    hrow[j * 64 + lane] = ev[j];
    const uint32_t wd[4] = {ev[j].x, ev[j].y, ev[j].z, ev[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x0 = __uint_as_float(wd[q] << 16), x1 = __uint_as_float(wd[q] & 0xffff0000u);
      ss = fmaf(x0, x0, fmaf(x1, x1, ss));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  const float r = rsqrtf(ss / (float)D + a.eps);
  bool range = true;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const uint32_t wd[4] = {ev[j].x, ev[j].y, ev[j].z, ev[j].w}, gw[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float y0 = __uint_as_float(wd[q] << 16) * __uint_as_float(gw[q] << 16) * r;
      const float y1 = __uint_as_float(wd[q] & 0xffff0000u) * __uint_as_float(gw[q] & 0xffff0000u) * r;
      range = range && fabsf(y0) <= kF16Max && fabsf(y1) <= kF16Max;
      o[q] = f16pair(y0, y1);
    }
    *reinterpret_cast<uint4 *>(abase + a_piece(m, (j * 64 + lane) * 8, nk)) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (!range) atomicOr(a.flags, 2u);
  if (lane == 0) a.map[m] = make_int2(dst, pos);
  if (lane < a.dh / 2) csrow[lane] = csv;
}

constexpr int kGWN = 4, kGRB = kGBM / 2 / 16, kGCB = kGBN / kGWN / 16;   // 2 x 4 waves of 64 x 48

template <int DH>
__global__ __launch_bounds__(64 * kGWaves) void qkv_gemm_bf16_kernel(const GemmArgs a) {
  extern __shared__ __align__(16) char smem[];    // kGStages x (A tile, W tile)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = w / kGWN, wn = w % kGWN;          // this wave: rows 64*wm.., columns 48*wn..
  const int n0 = blockIdx.x * kGBN, m0 = blockIdx.y * kGBM;
  const int D = a.D;
  const int cbh = DH / 16;
  const int ncb = a.F / 16;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));

  // Sources of this wave's copy instructions: instruction j fills LDS pieces
  // [(j*kGWaves + w)*64, +64) of the tile, 8 rows of 8 pieces; piece slot s
  // of row r receives global piece s ^ ((r >> 1) & 7).  A is tiled already;
  // W tile rows are GEMM columns, mapped to weight rows (columns past F
  // repeat the last block).
  const int nk = D / kGBK;
  const char *asrc[kGCopyA];
  int aoff[kGCopyA];
#pragma unroll
  for (int j = 0; j < kGCopyA; ++j) {
    const int base = (j * kGWaves + w) * 64;
    asrc[j] = static_cast<const char *>(a.A) + (size_t)blockIdx.y * nk * kGStageA + (size_t)(base + lane) * 16;
    aoff[j] = __builtin_amdgcn_readfirstlane(base * 16);
  }
  const bf16_t *wsrc[kGCopyW];
  int woff[kGCopyW];
#pragma unroll
  for (int j = 0; j < kGCopyW; ++j) {
    const int base = (j * kGWaves + w) * 64, idx = base + lane;
    const int c = idx >> 3, slot = idx & 7;
    const int cb = min((n0 + c) >> 4, ncb - 1), cc = (n0 + c) & 15;
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    const int wrow = hh * DH + (cc < 8 ? p0 + cc : DH / 2 + p0 + (cc - 8));
    wsrc[j] = static_cast<const bf16_t *>(a.W) + (size_t)wrow * D + (gslot(c, slot) << 3);
    woff[j] = __builtin_amdgcn_readfirstlane(kGStageA + base * 16);
  }
  auto issue = [&](int kt) {
    const uint32_t st = smem_lds + (kt % kGStages) * kGStage;
    const int k0 = kt * kGBK;
#pragma unroll
    for (int j = 0; j < kGCopyA; ++j) dma16(asrc[j] + (size_t)kt * kGStageA, st + aoff[j]);
#pragma unroll
    for (int j = 0; j < kGCopyW; ++j) dma16(wsrc[j] + k0, st + woff[j]);
  };
  // bf16 -> fp16 in place, for the W pieces this wave copied (exact for
  // values in fp16's normal range); run once this wave's copies landed.
  auto convert = [&](int kt) {
    char *st = smem + (kt % kGStages) * kGStage;
#pragma unroll
    for (int j = 0; j < kGCopyW; ++j) {
      uint4 *p = reinterpret_cast<uint4 *>(st + woff[j]) + lane;
      const uint4 u = *p;
      *p = make_uint4(f16pair(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u)),
                      f16pair(__uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)),
                      f16pair(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u)),
                      f16pair(__uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u)));
    }
  };

  f32x4_t acc[kGRB][kGCB];
#pragma unroll
  for (int i = 0; i < kGRB; ++i)
#pragma unroll
    for (int j = 0; j < kGCB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Tile kt+1 is converted during iteration kt, its conversion arithmetic
  // interleaved with the MFMAs of tile kt.
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  if (nk > 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kGCopies));
  else if (nk > 1) __builtin_amdgcn_s_waitcnt(0x0F70 | kGCopies);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  convert(0);
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (kt + 3 < nk) issue(kt + 3);
    // This wave's copies of tile kt+1 landed (later tiles may stay in flight).
    if (kt + 3 < nk) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kGCopies));
    else if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(0x0F70 | kGCopies);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    const char *st = smem + (kt % kGStages) * kGStage;
    char *stn = smem + ((kt + 1) % kGStages) * kGStage;   // past the last tile: stale data, unread
    uint4 craw[kGCopyW];
#pragma unroll
    for (int j = 0; j < kGCopyW; ++j) craw[j] = reinterpret_cast<const uint4 *>(stn + woff[j])[lane];
    Frag<f16_t> af[2][kGRB], wf[2][kGCB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < kGRB; ++i)
        af[ks][i].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(st + frag_off(wm * kGRB + i, ks) + lane * 16));
#pragma unroll
      for (int j = 0; j < kGCB; ++j)
        wf[ks][j].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(st + kGStageA + gswz((wn * kGCB + j) * 16 + r16, 4 * ks + g)));
    }
#pragma unroll
    for (int i = 0; i < kGRB; ++i)
#pragma unroll
      for (int j = 0; j < kGCB; ++j) mma16(acc[i][j], af[0][i], wf[0][j]);
    uint4 cvt[kGCopyW];
#pragma unroll
    for (int j = 0; j < kGCopyW; ++j) {
      const uint4 u = craw[j];
      cvt[j] = make_uint4(f16pair(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u)),
                          f16pair(__uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)),
                          f16pair(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u)),
                          f16pair(__uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u)));
    }
#pragma unroll
    for (int j = 0; j < kGCopyW; ++j) reinterpret_cast<uint4 *>(stn + woff[j])[lane] = cvt[j];
#pragma unroll
    for (int i = 0; i < kGRB; ++i)
#pragma unroll
      for (int j = 0; j < kGCB; ++j) mma16(acc[i][j], af[1][i], wf[1][j]);
    // Schedule: all reads first, the first k-step's MFMAs interleaved with
    // the conversion arithmetic, the converted pieces written back, then the
    // second k-step's MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x100, kGCopyW + 2 * (kGRB + kGCB), 0);
#pragma unroll
    for (int q = 0; q < kGRB * kGCB; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x200, kGCopyW, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kGRB * kGCB, 0);
  }

  // Epilogue.  The ring is free once every wave is past its last reads: the
  // tile's per-token (cos, sin) rows are copied into it, RoPE is applied to
  // the Q and K features from there into an fp16 output tile, and that tile
  // leaves in 16-byte stores (the 8 columns of each half of a 16-column
  // block are 8 consecutive features).
  constexpr int OST = kGBN + 8;                      // fp16 elements per LDS output row (pad: banks)
  constexpr int OT_BYTES = kGBM * OST * 2;
  constexpr int CS_BYTES = kGBM * (DH / 2) * 8;
  static_assert(OT_BYTES + CS_BYTES + kGBM * 4 <= kGemmSmem, "epilogue tiles fit the ring");
  _Float16 *otile = reinterpret_cast<_Float16 *>(smem);
  const float2 *cst = reinterpret_cast<const float2 *>(smem + OT_BYTES);
  int *s_dst = reinterpret_cast<int *>(smem + OT_BYTES + CS_BYTES);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  {
    constexpr int NCP = CS_BYTES / 1024;             // 1 KB copies of the contiguous (cos, sin) block
    const char *src = reinterpret_cast<const char *>(a.cs + (size_t)m0 * (DH / 2));
    for (int j = w; j < NCP; j += kGWaves)
      dma16(src + j * 1024 + lane * 16, __builtin_amdgcn_readfirstlane(smem_lds + OT_BYTES + j * 1024));
    if (tid < kGBM) s_dst[tid] = a.map[min(m0 + tid, a.M - 1)].x;
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  __syncthreads();
  const int nrot = (a.H + a.Hkv) * DH, qf = a.H * DH, kf = a.Hkv * DH;
  bool range = true;
#pragma unroll
  for (int j = 0; j < kGCB; ++j) {
    const int cb = min((n0 >> 4) + wn * kGCB + j, ncb - 1);
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    const int pair = p0 + (r16 & 7);
    const bool first = r16 < 8;
    const bool rot = hh * DH < nrot;
#pragma unroll
    for (int i = 0; i < kGRB; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = (wm * kGRB + i) * 16 + 4 * g + v;
        const float y = acc[i][j][v];
        const float other = __shfl_xor(y, 8);
        float o = y;
        if (rot) {
          const float2 c2 = cst[row * (DH / 2) + pair];
          o = first ? (y * c2.x - other * c2.y) : (other * c2.y + y * c2.x);
        }
        range = range && fabsf(o) <= kF16Max;
        otile[row * OST + (wn * kGCB + j) * 16 + r16] = (_Float16)o;
      }
    }
  }
  if (!range) atomicOr(a.flags, 2u);
  __syncthreads();
  // 128 rows x 24 runs of 8 features per tile.
  for (int t = tid; t < kGBM * (kGBN / 8); t += 64 * kGWaves) {
    const int row = t / (kGBN / 8), run = t % (kGBN / 8);
    const int m = m0 + row;
    const int cb = (n0 >> 4) + (run >> 1);
    if (m >= a.M || cb >= ncb) continue;
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    const int feat = hh * DH + ((run & 1) ? DH / 2 + p0 : p0);
    const int dst = s_dst[row];
    const uint4 val = *reinterpret_cast<const uint4 *>(otile + row * OST + run * 8);
    f16_t *out;
    if (feat < qf) out = static_cast<f16_t *>(a.q) + (size_t)dst * qf + feat;
    else if (feat < qf + kf) out = static_cast<f16_t *>(a.k) + (size_t)dst * kf + (feat - qf);
    else out = static_cast<f16_t *>(a.v) + (size_t)dst * kf + (feat - qf - kf);
    *reinterpret_cast<uint4 *>(out) = val;
  }
}

// ---------------------------------------------------------------------------
// packed GEMM.  A workgroup takes CT halves (96 GEMM columns each) of one
// packed 192-column tile: CT = 2, the whole tile, or CT = 1, one half, for
// launches whose whole tiles would leave at least half of the compute units
// without a workgroup (twice the workgroups, each with half the work).  The
// 8 waves form two groups of four; both groups cover the whole tile, group 0
// on the first 32 of each tile's 64 contraction elements and group 1 on the
// second.  A wave owns 16*RB tokens x 96 columns (6 x RB accumulator blocks;
// RB = 2 CT): per contraction tile it reads 6 + RB operand fragments for
// 6 RB MFMAs.  The fragments of tile kt+1 are read right after the barrier
// that publishes it, interleaved with the MFMAs of tile kt.  At the end each
// wave hands half of its blocks to its partner in the other group through
// LDS, and each finishes the half it keeps.
//
// Column order inside a 16-column block cb of head hh (pairs p0..p0+7,
// p0 = 8 * (cb mod d_h/16)): column 4g + v is feature p0 + 2g + (v >> 1)
// of the head's first half for even v and its RoPE partner in the second
// half for odd v.  With C^T on the matrix core, lane (g, t) holds columns
// 4g..4g+3 of token t: two complete pairs.
// ---------------------------------------------------------------------------
constexpr int kPCB = 6;                               // column blocks per wave

template <int CT> struct PackedTile {
  static_assert(CT == 1 || CT == 2, "one or two column halves");
  static constexpr int BN = 96 * CT;                  // GEMM columns per workgroup
  static constexpr int RB = 2 * CT;                   // 16-token blocks per wave
  static constexpr int StW = kGStageW / 2 * CT;       // W bytes per stage
  static constexpr int Stage = kGStageA + StW;
  static constexpr int NST = CT == 2 ? 4 : 5;         // ring stages: 160 KB or 140 KB
  static constexpr int Smem = NST * Stage;
  static constexpr int CopiesW = StW / 1024;          // 1 KB copies of W per stage: 24 or 12
  static constexpr int RedBytes = kGWaves * kPCB * (RB / 2) * 1024;   // blocks handed over
};


__device__ __forceinline__ int packed_weight_row(int gc, int F, int dh) {
  const int ncb = F / 16, cbh = dh / 16;
  const int cb = min(gc >> 4, ncb - 1), cc = gc & 15;  // columns past F repeat the last block
  const int hh = cb / cbh, p0 = (cb % cbh) * 8;
  return hh * dh + (cc & 1) * (dh / 2) + p0 + 2 * (cc >> 2) + ((cc >> 1) & 1);
}

// Wp[n][kt][fb][ks][lane] (16-byte pieces): column tile n of kGBN GEMM
// columns, contraction tile kt, fragment-major (see a_piece): fragment
// (16-column block fb, half ks), lane g*16 + r holds elements
// kt*64 + 32 ks + 8 g .. +7 of weight row packed_weight_row(n*kGBN + 16 fb + r),
// as fp16.
__global__ __launch_bounds__(256) void pack_qkv_weight_kernel(const bf16_t *W, uint4 *Wp, int D, int F, int dh,
                                                              size_t n_pieces) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_pieces) return;
  const int nk = D / kGBK;
  const int L = (int)(idx & 63), f = (int)((idx >> 6) % (kGBN / 8));   // 24 fragments per tile
  const size_t tk = idx / (kGStageW / 16);
  const int kt = (int)(tk % nk), n = (int)(tk / nk);
  const int c = (f >> 1) * 16 + (L & 15), ks = f & 1, g = L >> 4;
  const int wrow = packed_weight_row(n * kGBN + c, F, dh);
  const uint4 u = *reinterpret_cast<const uint4 *>(W + (size_t)wrow * D + kt * kGBK + 32 * ks + 8 * g);
  Wp[idx] = make_uint4(f16pair(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u)),
                       f16pair(__uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)),
                       f16pair(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u)),
                       f16pair(__uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u)));
}

template <int DH, int CT>
__global__ __launch_bounds__(512) void qkv_gemm_packed_kernel(const GemmArgs a) {
  using T = PackedTile<CT>;
  constexpr int RB = T::RB, HB = RB / 2, NST = T::NST;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int kg = w >> 2, wq = w & 3;
  const int wm = CT == 2 ? wq >> 1 : wq, wn = CT == 2 ? (wq & 1) : 0;
  const int D = a.D, nk = D / kGBK;                  // nk: a multiple of 8
  const int cbh = DH / 16, ncb = a.F / 16;
  const int n0 = blockIdx.x * T::BN, m0 = blockIdx.y * kGBM;
  const int ntile = CT == 2 ? blockIdx.x : blockIdx.x >> 1, half = CT == 2 ? 0 : blockIdx.x & 1;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));
  // Cache row of tile row tid, for the stores; its latency hides behind the loop.
  const int my_dst = tid < kGBM ? a.map[min(m0 + tid, a.M - 1)].x : 0;

  // Copy j of wave w moves pieces [(j*8 + w)*64, +64) of an operand's
  // stage: 1 KB at byte j*8192 + w*1024 of both the tiled source and the
  // LDS tile.  With CT = 1 a stage holds 12 KB of W: waves 0-3 copy two of
  // them, waves 4-7 one.
  const uint32_t lw = __builtin_amdgcn_readfirstlane(w * 1024);
  const char *asrc = static_cast<const char *>(a.A) + (size_t)blockIdx.y * nk * kGStageA + (size_t)(w * 64 + lane) * 16;
  const char *wsrc = static_cast<const char *>(a.Wp) + (size_t)ntile * nk * kGStageW + (size_t)half * T::StW +
                     (size_t)(w * 64 + lane) * 16;
  auto issue = [&](int kt) {
    const uint32_t st = smem_lds + (kt % NST) * T::Stage + lw;
    const char *as = asrc + (size_t)kt * kGStageA, *ws = wsrc + (size_t)kt * kGStageW;
#pragma unroll
    for (int j = 0; j < kGCopyA; ++j) dma16(as + j * 8192, st + j * 8192);
#pragma unroll
    for (int j = 0; j < (T::CopiesW + 7) / 8; ++j)
      if (j * 8 + w < T::CopiesW) dma16(ws + j * 8192, st + kGStageA + j * 8192);
  };
  // Wait until at most `t` (0..3) later tiles' copies of this wave are in
  // flight.
  auto wait_tiles = [&](int t) {
    constexpr int C = kGCopyA + (T::CopiesW + 7) / 8, C4 = kGCopyA + T::CopiesW / 8;   // waves 0-3, 4-7
    auto wait = [&](auto CC) {
      constexpr int c = decltype(CC)::value;
      if (t >= 3) vmcnt_wait<3 * c>();
      else if (t == 2) vmcnt_wait<2 * c>();
      else if (t == 1) vmcnt_wait<c>();
      else vmcnt_wait<0>();
    };
    if (C4 != C && w >= 4) wait(std::integral_constant<int, C4>{});
    else wait(std::integral_constant<int, C>{});
  };
  auto frags = [&](int kt, Frag<f16_t> (&fa)[RB], Frag<f16_t> (&fw)[kPCB]) {
    const char *st = smem + (kt % NST) * T::Stage;
#pragma unroll
    for (int i = 0; i < RB; ++i)
      fa[i].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(st + frag_off(wm * RB + i, kg) + lane * 16));
#pragma unroll
    for (int j = 0; j < kPCB; ++j)
      fw[j].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(st + kGStageA + frag_off(wn * kPCB + j, kg) + lane * 16));
  };

  f32x4_t acc[kPCB][RB];                             // C^T blocks: lane (g, t) holds columns 4g..4g+3 of token t
#pragma unroll
  for (int j = 0; j < kPCB; ++j)
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One contraction tile (kt + 1 < nk): tile kt+1 published (this wave's
  // copies landed, then the barrier), the fragments of tile kt+1 read, the
  // MFMAs of tile kt, and the copy of tile kt+NST-1 issued into the stage
  // tile kt-1 left (its fragments were consumed before the barrier).
  // Copies in flight on entry: tiles kt+1 .. kt+NST-2 (those below nk).
  constexpr int NM = kPCB * RB, R = RB + kPCB;       // MFMAs, fragment reads per tile
  constexpr int F1 = CT == 2 ? NM / 2 : R;           // MFMAs before the copy goes out
  static_assert(F1 >= R && F1 <= NM, "reads fit before the copy");
  auto step = [&](int kt, const Frag<f16_t> (&ca)[RB], const Frag<f16_t> (&cw)[kPCB],
                  Frag<f16_t> (&na)[RB], Frag<f16_t> (&nw)[kPCB]) {
    wait_tiles(min(NST - 3, nk - 2 - kt));
    lds_barrier();
    frags(kt + 1, na, nw);
    // Fragment reads first, interleaved with the first MFMAs; the copy of
    // tile kt+NST-1 goes out after them, so its LDS writes do not compete
    // with this wave's reads.
#pragma unroll
    for (int q = 0; q < F1; ++q) mma16(acc[q / RB][q % RB], cw[q / RB], ca[q % RB]);
#pragma unroll
    for (int q = 0; q < R; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if constexpr (F1 > R) __builtin_amdgcn_sched_group_barrier(0x008, F1 - R, 0);
    if (kt + NST - 1 < nk) issue(kt + NST - 1);
#pragma unroll
    for (int q = F1; q < NM; ++q) mma16(acc[q / RB][q % RB], cw[q / RB], ca[q % RB]);
  };
#pragma unroll
  for (int t = 0; t < NST - 1; ++t) issue(t);
  wait_tiles(NST - 2);
  lds_barrier();
  Frag<f16_t> fa0[RB], fw0[kPCB], fa1[RB], fw1[kPCB];
  frags(0, fa0, fw0);
  // No branch around the fragment reads inside the loop: the wait before the
  // MFMAs then covers only the previous tile's reads.
  for (int kt = 0; kt < nk - 2; kt += 2) {
    step(kt, fa0, fw0, fa1, fw1);
    step(kt + 1, fa1, fw1, fa0, fw0);
  }
  step(nk - 2, fa0, fw0, fa1, fw1);
#pragma unroll
  for (int j = 0; j < kPCB; ++j)
#pragma unroll
    for (int i = 0; i < RB; ++i) mma16(acc[j][i], fw1[j], fa1[i]);

  // Epilogue.  Group kg keeps token blocks kg*HB .. kg*HB+HB-1 of its wave's
  // RB and hands the others to its partner (wave w ^ 4, same region, other
  // half of the contraction).  Then RoPE per lane into an fp16 output tile
  // [128 tokens][BN columns in run order: per block the 8 first-half
  // features, then their 8 partners], which all waves store as 16-byte runs.
  constexpr int OST = T::BN + 8;                     // fp16 elements per output row (pad: banks)
  constexpr int OT_BYTES = kGBM * OST * 2;
  static_assert(OT_BYTES + kGBM * 4 <= T::Smem && T::RedBytes <= T::Smem, "epilogue fits the ring");
  f32x4_t *red = reinterpret_cast<f32x4_t *>(smem);
  _Float16 *otile = reinterpret_cast<_Float16 *>(smem);
  int *s_dst = reinterpret_cast<int *>(smem + OT_BYTES);
  const int nrot = (a.H + a.Hkv) * DH;
  bool range = true;
  auto finish = [&](auto KG) {
    constexpr int own = HB * decltype(KG)::value, other = HB - own;
    // (cos, sin) of pairs p0+2g and p0+2g+1 for each kept block's token.
    uint4 csv[kPCB][HB];
#pragma unroll
    for (int j = 0; j < kPCB; ++j) {
      const int cb = min((n0 >> 4) + wn * kPCB + j, ncb - 1);
      const int hh = cb / cbh, p0 = (cb % cbh) * 8;
#pragma unroll
      for (int ii = 0; ii < HB; ++ii) {
        const int t = (wm * RB + own + ii) * 16 + r16;
        csv[j][ii] = hh * DH < nrot ? *reinterpret_cast<const uint4 *>(a.cs + (size_t)(m0 + t) * (DH / 2) + p0 + 2 * g)
                                    : make_uint4(0, 0, 0, 0);
      }
    }
    lds_barrier();                                   // every wave is past its last ring reads
#pragma unroll
    for (int j = 0; j < kPCB; ++j)
#pragma unroll
      for (int ii = 0; ii < HB; ++ii) red[(w * kPCB * HB + j * HB + ii) * 64 + lane] = acc[j][other + ii];
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kPCB; ++j)
#pragma unroll
      for (int ii = 0; ii < HB; ++ii) acc[j][own + ii] += red[((w ^ 4) * kPCB * HB + j * HB + ii) * 64 + lane];
    lds_barrier();                                   // hand-over area free for the output tile
#pragma unroll
    for (int j = 0; j < kPCB; ++j) {
      const int jb = wn * kPCB + j;
      const int cb = min((n0 >> 4) + jb, ncb - 1);
      const bool rot = cb / cbh * DH < nrot;
#pragma unroll
      for (int ii = 0; ii < HB; ++ii) {
        const int t = (wm * RB + own + ii) * 16 + r16;
        const f32x4_t y = acc[j][own + ii];
        float o0 = y[0], o1 = y[1], o2 = y[2], o3 = y[3];
        if (rot) {
          const uint4 c = csv[j][ii];
          const float c0 = __uint_as_float(c.x), s0 = __uint_as_float(c.y);
          const float c1 = __uint_as_float(c.z), s1 = __uint_as_float(c.w);
          o0 = y[0] * c0 - y[1] * s0;
          o1 = y[1] * c0 + y[0] * s0;
          o2 = y[2] * c1 - y[3] * s1;
          o3 = y[3] * c1 + y[2] * s1;
        }
        range = range && fabsf(o0) <= kF16Max && fabsf(o1) <= kF16Max && fabsf(o2) <= kF16Max && fabsf(o3) <= kF16Max;
        *reinterpret_cast<uint32_t *>(otile + t * OST + jb * 16 + 2 * g) = f16pair(o0, o2);
        *reinterpret_cast<uint32_t *>(otile + t * OST + jb * 16 + 8 + 2 * g) = f16pair(o1, o3);
      }
    }
  };
  vmcnt_wait<0>();
  if (kg == 0) finish(std::integral_constant<int, 0>{});
  else finish(std::integral_constant<int, 1>{});
  if (tid < kGBM) s_dst[tid] = my_dst;
  if (!range) atomicOr(a.flags, 2u);
  lds_barrier();
  // 128 rows x BN/8 runs of 8 features per tile.
  const int qf = a.H * DH, kf = a.Hkv * DH;
  for (int t = tid; t < kGBM * (T::BN / 8); t += 64 * kGWaves) {
    const int row = t / (T::BN / 8), run = t % (T::BN / 8);
    const int m = m0 + row;
    const int cb = (n0 >> 4) + (run >> 1);
    if (m >= a.M || cb >= ncb) continue;
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    const int feat = hh * DH + ((run & 1) ? DH / 2 + p0 : p0);
    const int dst = s_dst[row];
    const uint4 val = *reinterpret_cast<const uint4 *>(otile + row * OST + run * 8);
    f16_t *out;
    if (feat < qf) out = static_cast<f16_t *>(a.q) + (size_t)dst * qf + feat;
    else if (feat < qf + kf) out = static_cast<f16_t *>(a.k) + (size_t)dst * kf + (feat - qf);
    else out = static_cast<f16_t *>(a.v) + (size_t)dst * kf + (feat - qf - kf);
    *reinterpret_cast<uint4 *>(out) = val;
  }
}

// ---------------------------------------------------------------------------
// Wide packed GEMM, for launches with at least one full round of 256 x 192
// tiles: per CU 1.43x fewer operand bytes per flop than 128 x 192.  A stage
// is one 32-wide half of a 64-wide contraction tile: the 16 A fragments of
// the two 128-token row tiles (16 KB) and the 12 W fragments of the column
// tile (12 KB), each a contiguous KB of the tiled operands; a 5-stage ring
// (140 KB).  Wave w owns tokens 64 (w & 3) .. +63 and columns 96 (w >> 2)
// .. +95 over the whole contraction (no hand-over): per stage 10 fragment
// reads and 24 MFMAs.  A second row tile past the launch repeats the last
// one (its rows are not stored).  Epilogue as in the packed GEMM.
// ---------------------------------------------------------------------------
struct WideTile {
  static constexpr int BM = 256, BN = 192, RB = 4;
  static constexpr int StA = 16 * 1024, StW = 12 * 1024, Stage = StA + StW, NST = 5;
  static constexpr int Smem = NST * Stage;            // 140 KB
  static constexpr int Copies = Stage / 1024;         // 28: waves 0-3 issue four, waves 4-7 three
};

template <int DH>
__global__ __launch_bounds__(512) void qkv_gemm_packed_wide_kernel(const GemmArgs a) {
  using T = WideTile;
  constexpr int RB = T::RB, NST = T::NST;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = w & 3, wn = w >> 2;
  const int D = a.D, nk = D / kGBK, ns = 2 * nk;     // ns: 32-wide stages
  const int cbh = DH / 16, ncb = a.F / 16;
  const int n0 = blockIdx.x * T::BN, m0 = blockIdx.y * T::BM;
  const int mt_last = (a.M + kGBM - 1) / kGBM - 1;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));
  // Cache row of tile row tid, for the stores; its latency hides behind the loop.
  const int my_dst = tid < T::BM ? a.map[min(m0 + tid, a.M - 1)].x : 0;

  // Copy j of wave w is fragment c = 8 j + w of the stage (c < 16: A
  // fragment c, c >= 16: W fragment c - 16), 1 KB to LDS byte c * 1024.
  const char *src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = min(8 * j + w, T::Copies - 1);
    if (c < 16) {
      const int mt = min(2 * (int)blockIdx.y + (c >> 3), mt_last);
      src[j] = static_cast<const char *>(a.A) + (size_t)mt * nk * kGStageA + (size_t)((c & 7) * 2) * 1024;
    } else {
      src[j] = static_cast<const char *>(a.Wp) + (size_t)blockIdx.x * nk * kGStageW + (size_t)((c - 16) * 2) * 1024;
    }
    src[j] += lane * 16;
  }
  auto issue = [&](int sg) {
    const uint32_t st = smem_lds + (sg % NST) * T::Stage;
    const int kt = sg >> 1, ks = sg & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 8 * j + w;
      if (c < T::Copies) {
        const size_t step = c < 16 ? (size_t)kGStageA : (size_t)kGStageW;
        dma16(src[j] + (size_t)kt * step + ks * 1024, st + c * 1024);
      }
    }
  };
  // Wait until at most `t` (0..3) later stages' copies of this wave are in flight.
  auto wait_stages = [&](int t) {
    auto wait = [&](auto CC) {
      constexpr int c = decltype(CC)::value;
      if (t >= 3) vmcnt_wait<3 * c>();
      else if (t == 2) vmcnt_wait<2 * c>();
      else if (t == 1) vmcnt_wait<c>();
      else vmcnt_wait<0>();
    };
    if (w >= 4) wait(std::integral_constant<int, 3>{});
    else wait(std::integral_constant<int, 4>{});
  };
  auto frags = [&](int sg, Frag<f16_t> (&fa)[RB], Frag<f16_t> (&fw)[kPCB]) {
    const char *st = smem + (sg % NST) * T::Stage;
#pragma unroll
    for (int i = 0; i < RB; ++i)
      fa[i].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(st + ((wm * RB + i) << 10) + lane * 16));
#pragma unroll
    for (int j = 0; j < kPCB; ++j)
      fw[j].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(st + T::StA + ((wn * kPCB + j) << 10) + lane * 16));
  };

  f32x4_t acc[kPCB][RB];                             // C^T blocks: lane (g, t) holds columns 4g..4g+3 of token t
#pragma unroll
  for (int j = 0; j < kPCB; ++j)
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One stage (sg + 1 < ns): stage sg+1 published, its fragments read, the
  // MFMAs of stage sg, and the copy of stage sg+NST-1 issued into the ring
  // slot stage sg-1 left.  Copies in flight on entry: stages sg+1 .. sg+3.
  constexpr int NM = kPCB * RB, R = RB + kPCB, F1 = NM / 2;
  static_assert(F1 >= R, "reads fit before the copy");
  auto step = [&](int sg, const Frag<f16_t> (&ca)[RB], const Frag<f16_t> (&cw)[kPCB],
                  Frag<f16_t> (&na)[RB], Frag<f16_t> (&nw)[kPCB]) {
    wait_stages(min(NST - 3, ns - 2 - sg));
    lds_barrier();
    frags(sg + 1, na, nw);
#pragma unroll
    for (int q = 0; q < F1; ++q) mma16(acc[q / RB][q % RB], cw[q / RB], ca[q % RB]);
#pragma unroll
    for (int q = 0; q < R; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, F1 - R, 0);
    if (sg + NST - 1 < ns) issue(sg + NST - 1);
#pragma unroll
    for (int q = F1; q < NM; ++q) mma16(acc[q / RB][q % RB], cw[q / RB], ca[q % RB]);
  };
#pragma unroll
  for (int t = 0; t < NST - 1; ++t) issue(t);
  wait_stages(NST - 2);
  lds_barrier();
  Frag<f16_t> fa0[RB], fw0[kPCB], fa1[RB], fw1[kPCB];
  frags(0, fa0, fw0);
  for (int sg = 0; sg < ns - 2; sg += 2) {
    step(sg, fa0, fw0, fa1, fw1);
    step(sg + 1, fa1, fw1, fa0, fw0);
  }
  step(ns - 2, fa0, fw0, fa1, fw1);
#pragma unroll
  for (int j = 0; j < kPCB; ++j)
#pragma unroll
    for (int i = 0; i < RB; ++i) mma16(acc[j][i], fw1[j], fa1[i]);

  // Epilogue: RoPE per lane into an fp16 output tile [256 tokens][192
  // columns in run order], two row blocks at a time (their (cos, sin) rows
  // loaded together), then 16-byte stores by all waves.
  constexpr int OST = T::BN + 8;                     // fp16 elements per output row (pad: banks)
  constexpr int OT_BYTES = T::BM * OST * 2;
  static_assert(OT_BYTES + T::BM * 4 <= T::Smem, "epilogue fits the ring");
  _Float16 *otile = reinterpret_cast<_Float16 *>(smem);
  int *s_dst = reinterpret_cast<int *>(smem + OT_BYTES);
  const int nrot = (a.H + a.Hkv) * DH;
  bool range = true;
  vmcnt_wait<0>();
  lds_barrier();                                     // every wave is past its last ring reads
  auto rope_half = [&](auto HC) {
    constexpr int i0 = 2 * decltype(HC)::value;
    uint4 csv[kPCB][2];
#pragma unroll
    for (int j = 0; j < kPCB; ++j) {
      const int cb = min((n0 >> 4) + wn * kPCB + j, ncb - 1);
      const int hh = cb / cbh, p0 = (cb % cbh) * 8;
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int t = (wm * RB + i0 + ii) * 16 + r16;
        const int row = min(m0 + t, a.M - 1);
        csv[j][ii] = hh * DH < nrot ? *reinterpret_cast<const uint4 *>(a.cs + (size_t)row * (DH / 2) + p0 + 2 * g)
                                    : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < kPCB; ++j) {
      const int jb = wn * kPCB + j;
      const int cb = min((n0 >> 4) + jb, ncb - 1);
      const bool rot = cb / cbh * DH < nrot;
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int t = (wm * RB + i0 + ii) * 16 + r16;
        const f32x4_t y = acc[j][i0 + ii];
        float o0 = y[0], o1 = y[1], o2 = y[2], o3 = y[3];
        if (rot) {
          const uint4 c = csv[j][ii];
          const float c0 = __uint_as_float(c.x), s0 = __uint_as_float(c.y);
          const float c1 = __uint_as_float(c.z), s1 = __uint_as_float(c.w);
          o0 = y[0] * c0 - y[1] * s0;
          o1 = y[1] * c0 + y[0] * s0;
          o2 = y[2] * c1 - y[3] * s1;
          o3 = y[3] * c1 + y[2] * s1;
        }
        range = range && fabsf(o0) <= kF16Max && fabsf(o1) <= kF16Max && fabsf(o2) <= kF16Max && fabsf(o3) <= kF16Max;
        *reinterpret_cast<uint32_t *>(otile + t * OST + jb * 16 + 2 * g) = f16pair(o0, o2);
        *reinterpret_cast<uint32_t *>(otile + t * OST + jb * 16 + 8 + 2 * g) = f16pair(o1, o3);
      }
    }
  };
  rope_half(std::integral_constant<int, 0>{});
  rope_half(std::integral_constant<int, 1>{});
  if (tid < T::BM) s_dst[tid] = my_dst;
  if (!range) atomicOr(a.flags, 2u);
  lds_barrier();
  // 256 rows x 24 runs of 8 features per tile.
  const int qf = a.H * DH, kf = a.Hkv * DH;
  for (int t = tid; t < T::BM * (T::BN / 8); t += 64 * kGWaves) {
    const int row = t / (T::BN / 8), run = t % (T::BN / 8);
    const int m = m0 + row;
    const int cb = (n0 >> 4) + (run >> 1);
    if (m >= a.M || cb >= ncb) continue;
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    const int feat = hh * DH + ((run & 1) ? DH / 2 + p0 : p0);
    const int dst = s_dst[row];
    const uint4 val = *reinterpret_cast<const uint4 *>(otile + row * OST + run * 8);
    f16_t *out;
    if (feat < qf) out = static_cast<f16_t *>(a.q) + (size_t)dst * qf + feat;
    else if (feat < qf + kf) out = static_cast<f16_t *>(a.k) + (size_t)dst * kf + (feat - qf);
    else out = static_cast<f16_t *>(a.v) + (size_t)dst * kf + (feat - qf - kf);
    *reinterpret_cast<uint4 *>(out) = val;
  }
}

int gemm_rows_padded(int M) { return (M + kGBM - 1) / kGBM * kGBM; }

hipError_t launch_qkv_prep(const SeqArgs &sa, const PrepArgs &a, hipStream_t s, const LaunchEvents &ev) {
  if (a.M_pad <= 0) return hipSuccess;
  const dim3 grid((a.M_pad + 3) / 4);
  switch (a.D / 512) {
#define LC_PREP(NPV) \
  case NPV: lc_launch<qkv_prep_kernel<NPV>>(grid, dim3(256), 0, s, ev, sa, a); break;
    LC_PREP(1) LC_PREP(2) LC_PREP(3) LC_PREP(4) LC_PREP(5) LC_PREP(6) LC_PREP(7) LC_PREP(8)
    LC_PREP(9) LC_PREP(10) LC_PREP(11) LC_PREP(12) LC_PREP(13) LC_PREP(14) LC_PREP(15) LC_PREP(16)
#undef LC_PREP
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny GEMM (at most 64 tokens, packed weight): a workgroup of 8 waves owns
// 48 GEMM columns (column blocks 3q..3q+2 of packed tile n) and the TB
// 16-token blocks of the launch.  The waves split the contraction by
// 64-wide tiles (wave w takes tiles w, w+8, ..., NPW of them); every operand
// fragment is one contiguous KB (fragment-major tiles), loaded straight
// into registers three tiles ahead, so the weight streams at the load unit's
// full rate and no LDS staging is needed.  The 8 partial sums meet in LDS
// in a fixed order (results do not depend on the token count); the
// epilogue is the packed GEMM's: RoPE in-lane, fp16 cache write.
// ---------------------------------------------------------------------------
constexpr int kSkinnyMaxTokens = 64;
template <int TB> constexpr int skinny_smem() { return 8 * 3 * TB * 64 * 16; }

template <int I, int N> struct Unroll {
  template <class F> __device__ __forceinline__ static void run(F &f) {
    f(std::integral_constant<int, I>{});
    Unroll<I + 1, N>::run(f);
  }
};
template <int N> struct Unroll<N, N> {
  template <class F> __device__ __forceinline__ static void run(F &) {}
};

template <int DH, int TB, int NPW>
__global__ __launch_bounds__(512) void qkv_skinny_kernel(const GemmArgs a) {
  constexpr int NFB = 3, NBLK = NFB * TB;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int nk = 8 * NPW;                            // contraction tiles (D / 64)
  const int cbh = DH / 16, ncb = a.F / 16;
  const int n = blockIdx.x >> 2, fb0 = 3 * (blockIdx.x & 3);
  const char *wt = static_cast<const char *>(a.Wp) + (size_t)n * nk * kGStageW + frag_off(fb0, 0) + lane * 16;
  const char *at = static_cast<const char *>(a.A) + lane * 16;      // row tile 0: the launch's <= 64 tokens

  struct Tile {
    uint4 w[NFB][2];
    uint4 x[TB][2];
  };
  auto fetch = [&](Tile &t, int kt) {
    const char *wp = wt + (size_t)kt * kGStageW, *ap = at + (size_t)kt * kGStageA;
#pragma unroll
    for (int f = 0; f < NFB; ++f)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) t.w[f][ks] = *reinterpret_cast<const uint4 *>(wp + frag_off(f, ks));
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) t.x[b][ks] = *reinterpret_cast<const uint4 *>(ap + frag_off(b, ks));
    // Keep the loads here: the scheduler would otherwise sink them next to
    // their use and collapse the three-tile prefetch.
    __builtin_amdgcn_sched_barrier(0);
  };
  f32x4_t acc[NFB][TB];
#pragma unroll
  for (int f = 0; f < NFB; ++f)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[f][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Tile t0, t1, t2;
  fetch(t0, w);
  if (NPW > 1) fetch(t1, w + 8);
  if (NPW > 2) fetch(t2, w + 16);
  auto step = [&](auto IC) {
    constexpr int i = decltype(IC)::value;
    Tile &cur = i % 3 == 0 ? t0 : (i % 3 == 1 ? t1 : t2);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int f = 0; f < NFB; ++f)
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          Frag<f16_t> fw, fx;
          fw.v = __builtin_bit_cast(f16x8_t, cur.w[f][ks]);
          fx.v = __builtin_bit_cast(f16x8_t, cur.x[b][ks]);
          mma16(acc[f][b], fw, fx);
        }
    if (i + 3 < NPW) fetch(cur, w + 8 * (i + 3));
  };
  Unroll<0, NPW>::run(step);

  // Partial sums of the 8 waves, then wave w finishes blocks w, w + 8.
  f32x4_t *red = reinterpret_cast<f32x4_t *>(smem);
#pragma unroll
  for (int f = 0; f < NFB; ++f)
#pragma unroll
    for (int b = 0; b < TB; ++b) red[(w * NBLK + f * TB + b) * 64 + lane] = acc[f][b];
  __syncthreads();
  const int nrot = (a.H + a.Hkv) * DH, qf = a.H * DH, kf = a.Hkv * DH;
  bool range = true;
  for (int blk = w; blk < NBLK; blk += 8) {
    f32x4_t y = red[blk * 64 + lane];
#pragma unroll
    for (int ww = 1; ww < 8; ++ww) y += red[(ww * NBLK + blk) * 64 + lane];
    const int f = blk / TB, b = blk % TB;
    const int cb = n * (kGBN / 16) + fb0 + f;
    const int tok = b * 16 + r16;
    if (cb >= ncb || tok >= a.M) continue;
    const int hh = cb / cbh, p0 = (cb % cbh) * 8;
    float o0 = y[0], o1 = y[1], o2 = y[2], o3 = y[3];
    if (hh * DH < nrot) {
      const uint4 c = *reinterpret_cast<const uint4 *>(a.cs + (size_t)tok * (DH / 2) + p0 + 2 * g);
      const float c0 = __uint_as_float(c.x), s0 = __uint_as_float(c.y);
      const float c1 = __uint_as_float(c.z), s1 = __uint_as_float(c.w);
      o0 = y[0] * c0 - y[1] * s0;
      o1 = y[1] * c0 + y[0] * s0;
      o2 = y[2] * c1 - y[3] * s1;
      o3 = y[3] * c1 + y[2] * s1;
    }
    range = range && fabsf(o0) <= kF16Max && fabsf(o1) <= kF16Max && fabsf(o2) <= kF16Max && fabsf(o3) <= kF16Max;
    const int dst = a.map[tok].x;
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
template <int DH, int TB, int NPW>
__global__ __launch_bounds__(512) void qkv_skinny_fused_kernel(const SeqArgs sa, const PrepArgs p, const GemmArgs a) {
  constexpr int NFB = 3, NBLK = NFB * TB, D = 512 * NPW;
  constexpr int RED = 8 * NBLK * 64 * 16;                        // partial sums of the 8 waves
  extern __shared__ __align__(16) char smem[];
  float *s_gamma = reinterpret_cast<float *>(smem + RED);        // [D]
  float *s_ss = s_gamma + D;                                     // [8 waves][64 tokens]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int cbh = DH / 16, ncb = a.F / 16;
  const int n = blockIdx.x >> 2, fb0 = 3 * (blockIdx.x & 3);
  const char *wt = static_cast<const char *>(a.Wp) + (size_t)n * 8 * NPW * kGStageW + frag_off(fb0, 0) + lane * 16;

  struct Tile {
    uint4 w[NFB][2];
    uint4 x[TB][2];
  };
  auto fetch_w = [&](Tile &t, int kt) {
    const char *wp = wt + (size_t)kt * kGStageW;
#pragma unroll
    for (int f = 0; f < NFB; ++f)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) t.w[f][ks] = *reinterpret_cast<const uint4 *>(wp + frag_off(f, ks));
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
  if (bad_l && lane < p.M && blockIdx.x == 0 && w == 0) atomicOr(p.flags, 1u);

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
    for (int sl = blockIdx.x; sl < TB * 8 * NPW; sl += gridDim.x) {
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
    const int cb = n * (kGBN / 16) + fb0 + f;
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
bool skinny_fused_supported(int M, int D, int vocab) {
  return skinny_supported(M, D) && (uint64_t)vocab * (uint64_t)D * 2u < (1ull << 32);
}
template <int TB, int NPW> constexpr int skinny_fused_smem() { return 8 * 3 * TB * 64 * 16 + 512 * NPW * 4 + 8 * 64 * 4; }

hipError_t launch_qkv_skinny_fused(int dh, const SeqArgs &sa, const PrepArgs &p, const GemmArgs &a, hipStream_t s,
                                   const LaunchEvents &ev) {
  if (a.M <= 0) return hipSuccess;
  if (!skinny_fused_supported(a.M, a.D, p.vocab) || !a.Wp || a.M != p.M || a.D != p.D) return hipErrorInvalidValue;
  const dim3 grid(4 * ((a.F + kGBN - 1) / kGBN));
#define LC_SF(DHV, TBV, NPWV) \
  lc_launch<qkv_skinny_fused_kernel<DHV, TBV, NPWV>>(grid, dim3(512), skinny_fused_smem<TBV, NPWV>(), s, ev, sa, p, a)
#define LC_SF_NPW(DHV, TBV)                       \
  switch (a.D / 512) {                             \
    case 1: LC_SF(DHV, TBV, 1); break;             \
    case 2: LC_SF(DHV, TBV, 2); break;             \
    case 4: LC_SF(DHV, TBV, 4); break;             \
    case 8: LC_SF(DHV, TBV, 8); break;             \
    default: LC_SF(DHV, TBV, 16); break;           \
  }
  if (dh == 128) {
    if (a.M <= 32) { LC_SF_NPW(128, 2) } else { LC_SF_NPW(128, 4) }
  } else {
    if (a.M <= 32) { LC_SF_NPW(64, 2) } else { LC_SF_NPW(64, 4) }
  }
#undef LC_SF_NPW
#undef LC_SF
  return hipGetLastError();
}

int prep_rows(int M, int D, bool packed) {
  if (packed && skinny_supported(M, D)) return M <= 32 ? 32 : 64;   // the token blocks the skinny GEMM reads
  return gemm_rows_padded(M);
}

bool skinny_supported(int M, int D) {
  const int npw = D / 512;
  return M >= 1 && M <= kSkinnyMaxTokens && D % 512 == 0 && (npw == 1 || npw == 2 || npw == 4 || npw == 8 || npw == 16);
}

size_t packed_qkv_weight_bytes(int D, int F) { return (size_t)((F + kGBN - 1) / kGBN) * kGBN * D * 2; }

hipError_t launch_pack_qkv_weight(const void *W, void *Wp, int D, int F, int dh, hipStream_t s) {
  const size_t n = packed_qkv_weight_bytes(D, F) / 16;
  if (n == 0) return hipSuccess;
  pack_qkv_weight_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
      static_cast<const bf16_t *>(W), static_cast<uint4 *>(Wp), D, F, dh, n);
  return hipGetLastError();
}

hipError_t launch_qkv_gemm(int dh, const GemmArgs &a, int tile, hipStream_t s, const LaunchEvents &ev) {
  if (a.M <= 0) return hipSuccess;
  if (a.Wp && skinny_supported(a.M, a.D)) {
    const dim3 grid(4 * ((a.F + kGBN - 1) / kGBN));
#define LC_SK(DHV, TBV, NPWV) \
  lc_launch<qkv_skinny_kernel<DHV, TBV, NPWV>>(grid, dim3(512), skinny_smem<TBV>(), s, ev, a)
#define LC_SK_NPW(DHV, TBV)                       \
  switch (a.D / 512) {                             \
    case 1: LC_SK(DHV, TBV, 1); break;             \
    case 2: LC_SK(DHV, TBV, 2); break;             \
    case 4: LC_SK(DHV, TBV, 4); break;             \
    case 8: LC_SK(DHV, TBV, 8); break;             \
    default: LC_SK(DHV, TBV, 16); break;           \
  }
    if (dh == 128) {
      if (a.M <= 32) { LC_SK_NPW(128, 2) } else { LC_SK_NPW(128, 4) }
    } else {
      if (a.M <= 32) { LC_SK_NPW(64, 2) } else { LC_SK_NPW(64, 4) }
    }
#undef LC_SK_NPW
#undef LC_SK
    return hipGetLastError();
  }
  dim3 grid((a.F + kGBN - 1) / kGBN, (a.M + kGBM - 1) / kGBM);
  if (a.Wp) {
    const unsigned cus = (unsigned)device_cus();
    const dim3 wgrid(grid.x, (a.M + WideTile::BM - 1) / WideTile::BM);
    if (tile == kGemmTileAuto) {
      // Wide tiles for at least one full round of them; half-width ones when
      // whole ones would leave half of the chip idle.
      tile = wgrid.x * wgrid.y >= cus ? kGemmTileWide : 2 * grid.x * grid.y <= cus ? kGemmTileHalf : kGemmTileWhole;
    }
    if (tile == kGemmTileWide) {
      if (dh == 128) lc_launch<qkv_gemm_packed_wide_kernel<128>>(wgrid, dim3(64 * kGWaves), WideTile::Smem, s, ev, a);
      else lc_launch<qkv_gemm_packed_wide_kernel<64>>(wgrid, dim3(64 * kGWaves), WideTile::Smem, s, ev, a);
    } else if (tile == kGemmTileHalf) {
      grid.x = (a.F + PackedTile<1>::BN - 1) / PackedTile<1>::BN;
      if (dh == 128) lc_launch<qkv_gemm_packed_kernel<128, 1>>(grid, dim3(64 * kGWaves), PackedTile<1>::Smem, s, ev, a);
      else lc_launch<qkv_gemm_packed_kernel<64, 1>>(grid, dim3(64 * kGWaves), PackedTile<1>::Smem, s, ev, a);
    } else {
      if (dh == 128) lc_launch<qkv_gemm_packed_kernel<128, 2>>(grid, dim3(64 * kGWaves), PackedTile<2>::Smem, s, ev, a);
      else lc_launch<qkv_gemm_packed_kernel<64, 2>>(grid, dim3(64 * kGWaves), PackedTile<2>::Smem, s, ev, a);
    }
  } else {
    if (dh == 128) lc_launch<qkv_gemm_bf16_kernel<128>>(grid, dim3(64 * kGWaves), kGemmSmem, s, ev, a);
    else lc_launch<qkv_gemm_bf16_kernel<64>>(grid, dim3(64 * kGWaves), kGemmSmem, s, ev, a);
  }
  return hipGetLastError();
}

hipError_t setup_gemm_attributes() {
  const std::pair<const void *, int> kernels[] = {
      {reinterpret_cast<const void *>(qkv_gemm_bf16_kernel<128>), kGemmSmem},
      {reinterpret_cast<const void *>(qkv_gemm_bf16_kernel<64>), kGemmSmem},
      {reinterpret_cast<const void *>(qkv_gemm_packed_kernel<128, 2>), PackedTile<2>::Smem},
      {reinterpret_cast<const void *>(qkv_gemm_packed_kernel<64, 2>), PackedTile<2>::Smem},
      {reinterpret_cast<const void *>(qkv_gemm_packed_kernel<128, 1>), PackedTile<1>::Smem},
      {reinterpret_cast<const void *>(qkv_gemm_packed_kernel<64, 1>), PackedTile<1>::Smem},
      {reinterpret_cast<const void *>(qkv_gemm_packed_wide_kernel<128>), WideTile::Smem},
      {reinterpret_cast<const void *>(qkv_gemm_packed_wide_kernel<64>), WideTile::Smem}};
  for (const auto &k : kernels) {
    const hipError_t e = hipFuncSetAttribute(k.first, hipFuncAttributeMaxDynamicSharedMemorySize, k.second);
    if (e != hipSuccess) return e;
  }
#define LC_SKA(DHV, NPWV)                                                                                    \
  {                                                                                                          \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(qkv_skinny_kernel<DHV, 4, NPWV>),      \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, skinny_smem<4>());        \
    if (e != hipSuccess) return e;                                                                           \
  }
  LC_SKA(128, 1) LC_SKA(128, 2) LC_SKA(128, 4) LC_SKA(128, 8) LC_SKA(128, 16)
  LC_SKA(64, 1) LC_SKA(64, 2) LC_SKA(64, 4) LC_SKA(64, 8) LC_SKA(64, 16)
#undef LC_SKA
#define LC_SFA(DHV, TBV, NPWV)                                                                                   \
  {                                                                                                              \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(qkv_skinny_fused_kernel<DHV, TBV, NPWV>),  \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, skinny_fused_smem<TBV, NPWV>()); \
    if (e != hipSuccess) return e;                                                                               \
  }
#define LC_SFA_NPW(DHV, TBV) LC_SFA(DHV, TBV, 1) LC_SFA(DHV, TBV, 2) LC_SFA(DHV, TBV, 4) LC_SFA(DHV, TBV, 8) LC_SFA(DHV, TBV, 16)
  LC_SFA_NPW(128, 2) LC_SFA_NPW(128, 4) LC_SFA_NPW(64, 2) LC_SFA_NPW(64, 4)
#undef LC_SFA_NPW
#undef LC_SFA
  return hipSuccess;
}

}  // namespace lc
