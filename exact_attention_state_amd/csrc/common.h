// Device-side helpers shared by the gfx950 kernels: element types, 16-byte
// loads, bf16 conversion, the 16x16 MFMA fragment abstraction, wave
// reductions, and the per-launch block table passed by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lc {

typedef uint16_t bf16_t;                                      // bf16 storage
typedef _Float16 f16_t;                                       // fp16 storage
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kF16Max = 65504.0f;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Samples per launch whose block-table rows travel inside the kernel
// arguments (no host->device copy per call).  Larger batches are launched in
// slices of this many samples.
constexpr int kMaxInline = 64;

// Block table of one launch.  pre[j][i] are non-decreasing prefix sums over
// samples (meaning fixed by each launcher); pre[j][n] is the total.
struct SeqArgs {
  int n;
  int off[kMaxInline];
  int len[kMaxInline];
  int bs[kMaxInline];
  int be[kMaxInline];
  int pre[4][kMaxInline + 1];
};

// Largest b < n with pre[b] <= item (samples with no items are skipped).
__device__ __forceinline__ int find_sample(const int *pre, int n, int item) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf2f(v); }
template <> __device__ __forceinline__ float to_f32<f16_t>(f16_t v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float v) { return (f16_t)v; }

// ---------------------------------------------------------------------------
// 8 consecutive elements along the contraction index: the per-lane operand
// of one 16x16 MFMA step of 32 (bf16 / fp16: one v_mfma_f32_16x16x32_bf16 /
// _f16; fp32: eight v_mfma_f32_16x16x4_f32).  For both, lane l supplies row/col l%16 and
// its lane group g = l/16 supplies 8 contraction elements; the hardware pairs
// A's and B's elements of the same lane group and slot, so any assignment of
// contraction indices to (group, slot) is valid as long as A and B share it.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16_t> { bf16x8_t v; };
template <> struct Frag<f16_t> { f16x8_t v; };
template <> struct Frag<float> { float v[8]; };

template <typename T> __device__ __forceinline__ void frag_zero(Frag<T> &f);
template <> __device__ __forceinline__ void frag_zero<bf16_t>(Frag<bf16_t> &f) {
  f.v = bf16x8_t{};
}
template <> __device__ __forceinline__ void frag_zero<f16_t>(Frag<f16_t> &f) {
  f.v = f16x8_t{};
}
template <> __device__ __forceinline__ void frag_zero<float>(Frag<float> &f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = 0.f;
}

// Load 8 consecutive elements (16 B for bf16, 32 B for fp32) from global or LDS.
template <typename T> __device__ __forceinline__ void frag_load(Frag<T> &f, const T *p);
template <> __device__ __forceinline__ void frag_load<bf16_t>(Frag<bf16_t> &f, const bf16_t *p) {
  uint4 u = *reinterpret_cast<const uint4 *>(p);
  f.v = __builtin_bit_cast(bf16x8_t, u);
}
template <> __device__ __forceinline__ void frag_load<f16_t>(Frag<f16_t> &f, const f16_t *p) {
  uint4 u = *reinterpret_cast<const uint4 *>(p);
  f.v = __builtin_bit_cast(f16x8_t, u);
}
template <> __device__ __forceinline__ void frag_load<float>(Frag<float> &f, const float *p) {
  float4 a = reinterpret_cast<const float4 *>(p)[0];
  float4 b = reinterpret_cast<const float4 *>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// Element access as fp32 (for prologue arithmetic on loaded values).
template <typename T> __device__ __forceinline__ float frag_get(const Frag<T> &f, int i);
template <> __device__ __forceinline__ float frag_get<bf16_t>(const Frag<bf16_t> &f, int i) {
  return (float)f.v[i];
}
template <> __device__ __forceinline__ float frag_get<f16_t>(const Frag<f16_t> &f, int i) {
  return (float)f.v[i];
}
template <> __device__ __forceinline__ float frag_get<float>(const Frag<float> &f, int i) {
  return f.v[i];
}
template <typename T> __device__ __forceinline__ void frag_set(Frag<T> &f, int i, float x);
template <> __device__ __forceinline__ void frag_set<bf16_t>(Frag<bf16_t> &f, int i, float x) {
  f.v[i] = (__bf16)x;
}
template <> __device__ __forceinline__ void frag_set<f16_t>(Frag<f16_t> &f, int i, float x) {
  f.v[i] = (_Float16)x;
}
template <> __device__ __forceinline__ void frag_set<float>(Frag<float> &f, int i, float x) {
  f.v[i] = x;
}

// acc += A * B over one contraction step of 32.
__device__ __forceinline__ void mma16(f32x4_t &acc, const Frag<bf16_t> &a, const Frag<bf16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4_t &acc, const Frag<f16_t> &a, const Frag<f16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4_t &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

// Lane exchanges by the gfx950 lane-swap instructions (one VALU step, no LDS
// permute): swapping x with itself leaves in every lane l the values of lanes
// l & ~16 and l | 16 (swap16), or of l & ~32 and l | 32 (swap32), i.e. the
// lane's own value and that of its partner l ^ 16 (l ^ 32) in lane order.
__device__ __forceinline__ void swap16(float x, float &lo, float &hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float &lo, float &hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Reductions across the four lane groups (lanes l, l^16, l^32, l^48).  The
// sum adds the pair (x_l, x_{l^16}), then the pair across l^32: the same
// rounding in every lane of a group (addition is commutative).
__device__ __forceinline__ float group_max(float x) {
  float a, b;
  swap16(x, a, b);
  swap32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float group_sum(float x) {
  float a, b;
  swap16(x, a, b);
  swap32(a + b, a, b);
  return a + b;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Global -> LDS copies by the load unit: lane l moves 16 (dma16) or 4 (dma4)
// bytes from its own `src` to LDS byte address lds + 16 l (+ 4 l); `lds` is
// wave-uniform.  Written as instructions the compiler does not see as LDS
// stores: it would otherwise wait for every copy in flight before each LDS
// read.  Callers wait for their copies themselves (vmcnt_wait) before
// reading what they wrote; M0 is clobbered.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char *)p);
}

// s_waitcnt vmcnt(N), N in [0, 63] (a compile-time constant); other counters
// untouched.  Also a compiler memory barrier: LDS filled by dma16/dma4 must
// not be read before the wait.
template <int N> __device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" : : : "memory");
}

// Global -> LDS copies with a wave-uniform base address (scalar registers) and
// a per-lane 32-bit byte offset: lane l moves 16 (4) bytes from base + voff
// to LDS byte address lds + 16 l (4 l).  One offset register serves every
// copy of a stage.  Waited for by the caller (vmcnt_wait); M0 is clobbered.
__device__ __forceinline__ void dma16_s(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(base)
               : "memory", "m0");
}

// x << sh, recomputed where it is used: a loop holding every copy offset in
// its own register across the main loop runs out of registers.
__device__ __forceinline__ uint32_t lane_bytes(int x, int sh) {
  uint32_t r;
  asm volatile("v_lshlrev_b32 %0, %1, %2" : "=v"(r) : "i"(sh), "v"(x));
  return r;
}

// s_waitcnt vmcnt(n) for a runtime n in [0, N].
template <int N> __device__ __forceinline__ void vmcnt_wait_rt(int n) {   // n in [0, N]: runtime -> constant
  if constexpr (N == 0) {
    vmcnt_wait<0>();
  } else {
    if (n >= N) vmcnt_wait<N>();
    else vmcnt_wait_rt<N - 1>(n);
  }
}


// In-wave LDS ordering: this wave's LDS writes complete before its later reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" : : : "memory");
}

// Workgroup barrier that orders LDS traffic only: the waves meet, and LDS
// stores issued before it are visible after it, while global loads issued
// before it stay in flight (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace lc
