// Device-side helpers shared by the gfx950 kernels: element types, MFMA
// wrappers and fragment layouts, bf16 rounding, wave/block scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moelora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// bfloat16 is stored as its raw 16-bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even.  Inputs are finite here.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// four consecutive outputs in one store (8 bytes of bf16, 16 of fp32); dst
// 8- (bf16) or 16-byte (fp32) aligned
__device__ __forceinline__ void store4(bf16_t* dst, float a, float b, float c, float d) {
  const uint32_t lo = f32_to_bf16(a) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
  const uint32_t hi = f32_to_bf16(c) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
}
__device__ __forceinline__ void store4(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

// ---------------------------------------------------------------------------
// MFMA 32x32 tiles.
//
// For both element types one instruction computes a 32x32 fp32 block
// D += A (32 x KSTEP) * B (KSTEP x 32).  Lane l = 32*h + c supplies
//   A fragment: row c of A, k-elements [h*KPACK, (h+1)*KPACK) of the step
//   B fragment: column c of B, the same k-elements
// and receives D element (row 8*(i/4) + 4*h + i%4, column c) in acc[i].
//   bf16: v_mfma_f32_32x32x16_bf16, KSTEP 16, KPACK 8 (16 bytes per lane)
//   f32 : v_mfma_f32_32x32x2_f32,    KSTEP 2,  KPACK 1 (4 bytes per lane)
// Any mapping of the real k indices onto the step's k positions is valid as
// long as A and B fragments use the same one.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
  static constexpr int KSTEP = 16;
  static constexpr int KPACK = 8;
  typedef bf16x8_t frag_t;
  __device__ __forceinline__ static void run(f32x16_t& acc, frag_t a, frag_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static frag_t load(const bf16_t* p) {
    return __builtin_bit_cast(frag_t, *reinterpret_cast<const uint4*>(p));
  }
  __device__ __forceinline__ static frag_t zero() { return __builtin_bit_cast(frag_t, make_uint4(0, 0, 0, 0)); }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 2;
  static constexpr int KPACK = 1;
  typedef float frag_t;
  __device__ __forceinline__ static void run(f32x16_t& acc, frag_t a, frag_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static frag_t load(const float* p) { return *p; }
  __device__ __forceinline__ static frag_t zero() { return 0.0f; }
};

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles (weight-streaming kernels).
// Lane l = 16*g + c (g in 0..3) supplies A row c and B column c with the
// k-elements [g*KPACK, (g+1)*KPACK) of the step, and receives D element
// (row 4*g + i, column c) in acc[i], i in 0..3.
//   bf16: v_mfma_f32_16x16x32_bf16, KSTEP 32, KPACK 8
//   f32 : v_mfma_f32_16x16x4_f32,   KSTEP 4,  KPACK 1
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma16;

template <> struct Mfma16<bf16_t> {
  static constexpr int KSTEP = 32;
  static constexpr int KPACK = 8;
  typedef bf16x8_t frag_t;
  __device__ __forceinline__ static void run(f32x4_t& acc, frag_t a, frag_t b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static frag_t load(const bf16_t* p) { return Mfma<bf16_t>::load(p); }
  __device__ __forceinline__ static frag_t zero() { return Mfma<bf16_t>::zero(); }
};

template <> struct Mfma16<float> {
  static constexpr int KSTEP = 4;
  static constexpr int KPACK = 1;
  typedef float frag_t;
  __device__ __forceinline__ static void run(f32x4_t& acc, frag_t a, frag_t b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static frag_t load(const float* p) { return *p; }
  __device__ __forceinline__ static frag_t zero() { return 0.0f; }
};

// SiLU(v) = v / (1 + e^-v), with the device expf.
__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// Eight fp32 values as two bf16 fragments with v ~= hi + lo (about 16
// significant bits): a bf16 MFMA against hi and then lo keeps fp32-like
// precision for the small rank-r operand of the LoRA expand.
__device__ __forceinline__ void split_bf16x8(float4 a, float4 b, bf16x8_t& hi, bf16x8_t& lo) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16_t h0 = f32_to_bf16(v[2 * i]), h1 = f32_to_bf16(v[2 * i + 1]);
    const bf16_t l0 = f32_to_bf16(v[2 * i] - bf16_to_f32(h0));
    const bf16_t l1 = f32_to_bf16(v[2 * i + 1] - bf16_to_f32(h1));
    hw[i] = h0 | (static_cast<uint32_t>(h1) << 16);
    lw[i] = l0 | (static_cast<uint32_t>(l1) << 16);
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
}
__device__ __forceinline__ void split_bf16x8(const float* v8, bf16x8_t& hi, bf16x8_t& lo) {
  split_bf16x8(*reinterpret_cast<const float4*>(v8), *reinterpret_cast<const float4*>(v8 + 4), hi, lo);
}

// LDS address space, for the destination of global_load_lds (the direct
// global-memory-to-LDS load: lane i's bytes land at base + i * size).
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only vmcnt constrained (gfx9 encoding: expcnt and lgkmcnt at
// their maximum), and the same with lgkmcnt(0).  The direct-to-LDS loads count
// in vmcnt.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  constexpr int imm = (N & 15) | ((N >> 4) << 14) | 0x0F70;
  __builtin_amdgcn_s_waitcnt(imm);
}
template <int N> __device__ __forceinline__ void wait_vmcnt_lgkm0() {
  constexpr int imm = (N & 15) | ((N >> 4) << 14) | 0x0070;
  __builtin_amdgcn_s_waitcnt(imm);
}

// Workgroup barrier that orders LDS accesses only (no wait on global memory).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Row (within the 32x32 block) of accumulator element i held by a lane of half h.
__device__ __forceinline__ int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

__device__ __forceinline__ f32x16_t zero_acc() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Relaxed, device-scope fp32 atomic add (hardware global_atomic_add_f32, no return).
__device__ __forceinline__ void atomic_add_relaxed(float* p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive scan of one int across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive scan of one int per thread across the whole block (blockDim.x a
// multiple of 64, at most 1024).  wave_tmp must hold 16 ints of LDS.  Every
// thread of the block must call it.  *total receives the block-wide sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int x = wave_inclusive_scan(v);
  if (lane == kWave - 1) wave_tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    int s = lane < nw ? wave_tmp[lane] : 0;
    s = wave_inclusive_scan(s);
    if (lane < nw) wave_tmp[lane] = s;
  }
  __syncthreads();
  int prefix = w > 0 ? wave_tmp[w - 1] : 0;
  *total = wave_tmp[nw - 1];
  __syncthreads();
  return prefix + x - v;
}

}  // namespace moelora
