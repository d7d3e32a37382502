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
// Tiling of the GEMM (128 tokens x 192 features per workgroup, 8 waves of
// 64 x 48, 64-wide contraction tiles): A (fp16) and W (bf16, as stored) are
// copied global -> LDS by the load unit (global_load_lds_dwordx4) into a
// 3-stage ring, 16-byte pieces XOR-swizzled by row so the operand reads hit
// distinct banks; each wave converts the W pieces it copied to fp16 in
// place, one tile ahead of their use (exact for weights in fp16's normal
// range).  One workgroup barrier per contraction tile.  GEMM column j of a 16-column block holds RoPE pairs as
// in the small-batch kernel (features p..p+7 and p+d_h/2..p+d_h/2+7), so a
// rotation partner is 8 lanes away.  Consecutive workgroups take consecutive
// column tiles, so the row tiles of one column tile land on one XCD and
// share its weight tile in that XCD's L2.
//
// Precision: one fp16 rounding of the normalised activation (11-bit
// significand, 8x finer than bf16) and fp32 accumulation; the small-batch
// kernel instead keeps gamma * E exact with a bf16 hi/lo split, which costs
// twice the matrix-core work - affordable only where the step is bound by
// streaming the weights.

#include "internal.h"

namespace lc {

typedef _Float16 gh2_t __attribute__((ext_vector_type(2)));

// Global -> LDS copy of 16 bytes per lane to LDS byte address lds + 16*lane
// (lds wave-uniform).  Written as an instruction the compiler does not see
// as an LDS store: it would otherwise wait for every copy in flight before
// each LDS read, including copies into other stages of the ring.  The kernel
// waits for its copies itself (vmcnt) before the barrier that publishes a
// stage; M0 is used by nothing else in the kernel.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char *)p);
}

__device__ __forceinline__ uint32_t f16pair(float a, float b) {
  const gh2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// prep: one wave per token row m of the launch (rows past M of the padded
// tile are written as zeros).  Each lane owns D/64 consecutive elements.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void qkv_prep_kernel(const SeqArgs sa, const PrepArgs a) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= a.M_pad) return;
  const int D = a.D;
  const int per = D / 64;                          // elements per lane (multiple of 4)
  _Float16 *arow = static_cast<_Float16 *>(a.A) + (size_t)m * D + lane * per;
  float2 *csrow = a.cs + (size_t)m * (a.dh / 2);
  if (m >= a.M) {
    for (int j = 0; j < per; j += 8) *reinterpret_cast<uint4 *>(arow + j) = make_uint4(0, 0, 0, 0);
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
  const bf16_t *erow = static_cast<const bf16_t *>(a.E) + (size_t)(bad ? 0 : id) * D + lane * per;
  const bf16_t *grow = static_cast<const bf16_t *>(a.gamma) + lane * per;
  bf16_t *hrow = static_cast<bf16_t *>(a.h) + (size_t)dst * D + lane * per;
  float ss = 0.f;
  for (int j = 0; j < per; j += 8) {
    const uint4 u = bad ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4 *>(erow + j);
    *reinterpret_cast<uint4 *>(hrow + j) = u;
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
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
  for (int j = 0; j < per; j += 8) {
    const uint4 u = bad ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4 *>(erow + j);
    const uint4 gv = *reinterpret_cast<const uint4 *>(grow + j);
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float y0 = __uint_as_float(wd[q] << 16) * __uint_as_float(gw[q] << 16) * r;
      const float y1 = __uint_as_float(wd[q] & 0xffff0000u) * __uint_as_float(gw[q] & 0xffff0000u) * r;
      range = range && fabsf(y0) <= kF16Max && fabsf(y1) <= kF16Max;
      o[q] = f16pair(y0, y1);
    }
    *reinterpret_cast<uint4 *>(arow + j) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (!range) atomicOr(a.flags, 2u);
  if (lane == 0) a.map[m] = make_int2(dst, pos);
  if (lane < a.dh / 2) csrow[lane] = a.rope[(size_t)pos * (a.dh / 2) + lane];
}

// ---------------------------------------------------------------------------
// gemm
// ---------------------------------------------------------------------------
#ifndef LC_GEMM_IL
#define LC_GEMM_IL 1
#endif
constexpr int kGBM = 128, kGBN = 192, kGBK = 64, kGStages = LC_GEMM_IL ? 4 : 3;
#ifndef LC_GEMM_WM
#define LC_GEMM_WM 2
#define LC_GEMM_WN 4
#endif
constexpr int kGWM = LC_GEMM_WM, kGWN = LC_GEMM_WN;   // wave grid (rows x columns of the tile)
constexpr int kGWaves = kGWM * kGWN;
constexpr int kGRB = kGBM / kGWM / 16, kGCB = kGBN / kGWN / 16;   // 16x16 blocks per wave
constexpr int kGStageA = kGBM * kGBK * 2;          // bytes: fp16 A tile
constexpr int kGStageW = kGBN * kGBK * 2;          // bytes: W tile (bf16 as copied, fp16 once converted)
constexpr int kGStage = kGStageA + kGStageW;
constexpr int kGemmSmem = kGStages * kGStage;
constexpr int kGCopyA = kGStageA / 1024 / kGWaves;  // copy instructions per wave per stage (1 KB each)
constexpr int kGCopyW = kGStageW / 1024 / kGWaves;
constexpr int kGCopies = kGCopyA + kGCopyW;
static_assert(kGCopyA * 1024 * kGWaves == kGStageA && kGCopyW * 1024 * kGWaves == kGStageW, "copy tiling");

// Tile rows are 128 bytes (64 contraction elements); 16-byte piece p of row r
// sits in slot p ^ ((r >> 1) & 7): the 16 consecutive rows of one operand
// read then cover all 64 banks once.
__device__ __forceinline__ int gslot(int r, int p) { return p ^ ((r >> 1) & 7); }
__device__ __forceinline__ int gswz(int r, int p) { return r * 128 + (gslot(r, p) << 4); }

template <int DH>
__global__ __launch_bounds__(64 * kGWaves) void qkv_gemm_kernel(const GemmArgs a) {
  extern __shared__ __align__(16) char smem[];    // kGStages x (A tile, W tile)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = w / kGWN, wn = w % kGWN;          // this wave: rows 16*kGRB*wm.., columns 16*kGCB*wn..
  const int n0 = blockIdx.x * kGBN, m0 = blockIdx.y * kGBM;
  const int D = a.D;
  const int cbh = DH / 16;
  const int ncb = a.F / 16;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));

  // Sources of this wave's copy instructions: instruction j fills LDS pieces
  // [(j*kGWaves + w)*64, +64) of the tile, 8 rows of 8 pieces; piece slot s
  // of row r receives global piece s ^ ((r >> 1) & 7).  W tile rows are GEMM
  // columns, mapped to weight rows (columns past F repeat the last block).
  const _Float16 *asrc[kGCopyA];
  int aoff[kGCopyA];
#pragma unroll
  for (int j = 0; j < kGCopyA; ++j) {
    const int base = (j * kGWaves + w) * 64, idx = base + lane;
    const int r = idx >> 3, slot = idx & 7;
    asrc[j] = static_cast<const _Float16 *>(a.A) + (size_t)(m0 + r) * D + (gslot(r, slot) << 3);
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
    for (int j = 0; j < kGCopyA; ++j) dma16(asrc[j] + k0, st + aoff[j]);
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

  const int nk = D / kGBK;
#if LC_GEMM_IL
  // 4-stage ring: tile kt+1 is converted during iteration kt, its conversion
  // arithmetic interleaved with the MFMAs of tile kt.
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
        af[ks][i].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(st + gswz((wm * kGRB + i) * 16 + r16, 4 * ks + g)));
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
#else
  issue(0);
  if (nk > 1) {
    issue(1);
    __builtin_amdgcn_s_waitcnt(0x0F70 | kGCopies);            // vmcnt(kGCopies): tile 0 landed
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  convert(0);
  for (int kt = 0; kt < nk; ++kt) {
    // After the barrier tile kt is converted and visible, and the stage read
    // in iteration kt-1 is free for tile kt+2.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (kt + 2 < nk) issue(kt + 2);
    const char *st = smem + (kt % kGStages) * kGStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Frag<f16_t> af[kGRB], wf[kGCB];
#pragma unroll
      for (int i = 0; i < kGRB; ++i) {
        const int r = (wm * kGRB + i) * 16 + r16;
        af[i].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(st + gswz(r, 4 * ks + g)));
      }
#pragma unroll
      for (int j = 0; j < kGCB; ++j) {
        const int c = (wn * kGCB + j) * 16 + r16;
        wf[j].v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4 *>(st + kGStageA + gswz(c, 4 * ks + g)));
      }
#pragma unroll
      for (int i = 0; i < kGRB; ++i)
#pragma unroll
        for (int j = 0; j < kGCB; ++j) mma16(acc[i][j], af[i], wf[j]);
    }
    if (kt + 1 < nk) {
      // Tile kt+1: this wave's copies landed (tile kt+2's may stay in flight).
      if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(0x0F70 | kGCopies);
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      convert(kt + 1);
    }
  }
#endif

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

int gemm_rows_padded(int M) { return (M + kGBM - 1) / kGBM * kGBM; }

hipError_t launch_qkv_prep(const SeqArgs &sa, const PrepArgs &a, hipStream_t s, const LaunchEvents &ev) {
  if (a.M_pad <= 0) return hipSuccess;
  lc_launch(qkv_prep_kernel, dim3((a.M_pad + 3) / 4), dim3(256), 0, s, ev, sa, a);
  return hipGetLastError();
}

hipError_t launch_qkv_gemm(int dh, const GemmArgs &a, hipStream_t s, const LaunchEvents &ev) {
  if (a.M <= 0) return hipSuccess;
  dim3 grid((a.F + kGBN - 1) / kGBN, (a.M + kGBM - 1) / kGBM);
  if (dh == 128) lc_launch(qkv_gemm_kernel<128>, grid, dim3(64 * kGWaves), kGemmSmem, s, ev, a);
  else lc_launch(qkv_gemm_kernel<64>, grid, dim3(64 * kGWaves), kGemmSmem, s, ev, a);
  return hipGetLastError();
}

hipError_t setup_gemm_attributes() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(qkv_gemm_kernel<128>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kGemmSmem);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(qkv_gemm_kernel<64>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kGemmSmem);
  return e;
}

}  // namespace lc
