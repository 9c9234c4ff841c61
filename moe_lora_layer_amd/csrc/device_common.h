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

// Round to nearest, ties to even: gfx950's conversion instruction
// (v_cvt_pk_bf16_f32), one instruction instead of three integer ones.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
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

// SiLU(v) = v * sigma(v) = v / (1 + e^-v), from the hardware base-2
// exponential and reciprocal (each within about one fp32 ulp, so the result
// is good to a few fp32 ulps, far inside the bf16 rounding of an activation).
// Large negative v: e^-v overflows to inf and the reciprocal to 0, the limit
// of SiLU there.  The library expf and IEEE division cost about 35 vector
// instructions per value, which made SiLU a visible part of the gate_up
// epilogue at 64 values per lane.
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v));
}

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

// Workgroup barrier after this wave's LDS accesses have completed (lgkmcnt(0)),
// with no fence: outstanding global stores and loads are not waited for.  For
// points where no direct-to-LDS load is in flight.
__device__ __forceinline__ void lds_only_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
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

// ---------------------------------------------------------------------------
// Weights stored k-major ([K][N], N contiguous: the page's h_in x h_out
// orientation).  MFMA fragments take K-contiguous runs per lane, so a k-major
// operand is turned around on its way in:
//   - loaded through registers straight into MFMA fragments (the LoRA
//     kernels, and fp32 tiles on their way to LDS): each aligned group of 8
//     lanes (bf16) or 4 lanes (fp32) loads a square block, lane m holding
//     k-row m of 8 (4) consecutive columns; transpose8/transpose4 leave lane m
//     holding column m of 8 (4) consecutive k, i.e. exactly the 16-byte chunk
//     the K-contiguous layout would have given it;
//   - staged in LDS (direct-to-LDS copies, and bf16 GEMM tiles stored from
//     registers as loaded): the tile stays k-major in LDS and the fragments
//     are read with ds_read_b64_tr_b16 (kn_frag).
// Every lane of a group must execute the transposes (no divergence).
// ---------------------------------------------------------------------------
// v of lane ^ MASK (MASK 1, 2, 4), with DPP moves on the vector ALU: quad
// permutations for 1 and 2, and for 4 a row shift by 4 towards or away from
// lane 0 (lanes with bit 2 clear read lane + 4, the others lane - 4).
template <int MASK>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  static_assert(MASK == 1 || MASK == 2 || MASK == 4, "xor_lane: 1, 2 or 4");
  const int x = static_cast<int>(v);
  if (MASK == 1) return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
  if (MASK == 2) return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
  const int up = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, true);    // row_shl:4, lane + 4
  const int down = __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, true);  // row_shr:4, lane - 4
  return static_cast<uint32_t>((threadIdx.x & 4) ? down : up);
}

// 8 x 8 bf16 transpose across the aligned 8-lane group of this lane: on entry
// lane m holds row m (columns 0..7, two per dword, low half first); on exit it
// holds column m (rows 0..7).  Three exchange steps swap the row and column
// bits 2, 1, 0 of every element.
__device__ __forceinline__ uint4 transpose8(uint4 v) {
  const int m = threadIdx.x & 7;
  {  // bit 2: dwords {0,1} hold columns 0-3, {2,3} columns 4-7
    const bool hi = (m & 4) != 0;
    const uint32_t s0 = xor_lane<4>(hi ? v.x : v.z), s1 = xor_lane<4>(hi ? v.y : v.w);
    if (hi) { v.x = s0; v.y = s1; } else { v.z = s0; v.w = s1; }
  }
  {  // bit 1: dwords {0,2} hold columns with bit 1 clear, {1,3} set
    const bool hi = (m & 2) != 0;
    const uint32_t s0 = xor_lane<2>(hi ? v.x : v.y), s1 = xor_lane<2>(hi ? v.z : v.w);
    if (hi) { v.x = s0; v.z = s1; } else { v.y = s0; v.w = s1; }
  }
  {  // bit 0: the low half of each dword holds the even column, the high half the odd
    const bool hi = (m & 1) != 0;
    // send the halves the partner keeps: odd columns from an even lane, even from an odd one
    const uint32_t p0 = hi ? ((v.x & 0xffffu) | (v.y << 16)) : ((v.x >> 16) | (v.y & 0xffff0000u));
    const uint32_t p1 = hi ? ((v.z & 0xffffu) | (v.w << 16)) : ((v.z >> 16) | (v.w & 0xffff0000u));
    const uint32_t r0 = xor_lane<1>(p0), r1 = xor_lane<1>(p1);
    if (hi) {  // keep the high halves, take the partner's high halves (its odd columns) as low
      v.x = (v.x & 0xffff0000u) | (r0 & 0xffffu);
      v.y = (v.y & 0xffff0000u) | (r0 >> 16);
      v.z = (v.z & 0xffff0000u) | (r1 & 0xffffu);
      v.w = (v.w & 0xffff0000u) | (r1 >> 16);
    } else {   // keep the low halves, take the partner's low halves (its even columns) as high
      v.x = (v.x & 0xffffu) | (r0 << 16);
      v.y = (v.y & 0xffffu) | (r0 & 0xffff0000u);
      v.z = (v.z & 0xffffu) | (r1 << 16);
      v.w = (v.w & 0xffffu) | (r1 & 0xffff0000u);
    }
  }
  return v;
}

// 4 x 4 fp32 transpose across the aligned 4-lane group (lane m: row m on
// entry, column m on exit).
__device__ __forceinline__ uint4 transpose4(uint4 v) {
  const int m = threadIdx.x & 3;
  {  // bit 1: x, y hold columns 0-1, z, w columns 2-3
    const bool hi = (m & 2) != 0;
    const uint32_t s0 = xor_lane<2>(hi ? v.x : v.z), s1 = xor_lane<2>(hi ? v.y : v.w);
    if (hi) { v.x = s0; v.y = s1; } else { v.z = s0; v.w = s1; }
  }
  {  // bit 0: x, z even columns, y, w odd
    const bool hi = (m & 1) != 0;
    const uint32_t s0 = xor_lane<1>(hi ? v.x : v.y), s1 = xor_lane<1>(hi ? v.z : v.w);
    if (hi) { v.x = s0; v.z = s1; } else { v.y = s0; v.w = s1; }
  }
  return v;
}

// The transpose for the element type of a 16-byte chunk.
template <typename T> __device__ __forceinline__ uint4 transpose_chunk(uint4 v);
template <> __device__ __forceinline__ uint4 transpose_chunk<bf16_t>(uint4 v) { return transpose8(v); }
template <> __device__ __forceinline__ uint4 transpose_chunk<float>(uint4 v) { return transpose4(v); }

// ds_read_b64_tr_b16: within each aligned 16-lane group, lane i supplies the
// LDS address of 4 consecutive bf16 of a k-major tile, namely row kb + i/4,
// columns cb + 4 (i % 4) .. + 3; lane i receives column cb + i of rows
// kb .. kb + 3 (element j = row kb + j).
typedef short tr_v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ds_read_tr16(const unsigned char* lds_byte_addr) {
  typedef __attribute__((address_space(3))) tr_v4i16 lds_v4i16;
  const tr_v4i16 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const_cast<unsigned char*>(lds_byte_addr)));
  return __builtin_bit_cast(uint2, v);
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
