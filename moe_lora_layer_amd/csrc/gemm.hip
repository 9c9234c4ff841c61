// Base grouped GEMM of the MoE experts on the MFMA units, plus the tile
// planner that turns bucket_offsets into per-expert M-tiles.
//
// The vLLM blog page "Multi-LoRA" (vllm.com.cn/blog/multi-lora), section
// "Implementing Multi-LoRA inference for MoE models in vLLM", runs the expert
// projections as a grouped GEMM: one GEMM per expert over the tokens routed to
// it.  Here the rows of every expert are contiguous in the sorted order, so the
// grid is a flat list of (M-tile, N-tile) pairs with the M-tiles computed on
// the device; surplus workgroups exit at once.
//
// Tile: BM x BN outputs, K stepped by 128 bytes (64 bf16 / 32 fp32).  Both
// operands are K-contiguous in memory (x rows and W^T rows), staged from
// registers into LDS with a 16-byte-chunk XOR swizzle so that the MFMA
// fragment reads (consecutive rows, same chunk) hit all banks, double
// buffered: the next K-step's global loads are in flight while the MFMAs of
// the current one run.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace moelora {

// ------------------------------------------------------------------------- prep
constexpr int kPrepThreads = 1024;

// Writes tiles for items [i0, i1) whose lengths come from offsets at stride
// `step`; `first` is the index of the first tile of item i0.
// Tiles are only emitted below max_tiles and only for rows inside [0, S), so a
// malformed offsets array cannot make any later kernel read out of bounds.
__device__ void emit_tiles(const int32_t* offsets, int i0, int i1, int step, int rows, int first,
                           int S, int max_tiles, int4* tiles) {
  int t = first;
  for (int i = i0; i < i1; ++i) {
    const int r0 = max(0, offsets[i * step]);
    const int r1 = min(S, offsets[(i + 1) * step]);
    for (int r = r0; r < r1 && t < max_tiles; r += rows) tiles[t++] = make_int4(i, r, min(r1, r + rows), 0);
  }
}

__device__ int count_tiles(const int32_t* offsets, int i0, int i1, int step, int rows, int S) {
  int n = 0;
  for (int i = i0; i < i1; ++i) {
    const int r0 = max(0, offsets[i * step]);
    const int r1 = min(S, offsets[(i + 1) * step]);
    if (r1 > r0) n += (r1 - r0 + rows - 1) / rows;
  }
  return n;
}

__global__ void __launch_bounds__(kPrepThreads)
k_prep(const int32_t* __restrict__ sorted_slots, const int32_t* __restrict__ offsets, int S,
       int E, int L, int bm, int bml, int max_mt, int max_lt, int32_t* __restrict__ pos,
       int4* __restrict__ mtiles, int4* __restrict__ ltiles, int32_t* __restrict__ counts,
       int32_t* __restrict__ expert_tiles, float4* __restrict__ zero, int64_t zero_n4) {
  __shared__ int wave_tmp[16];
  const int tid = threadIdx.x;
  // every workgroup: its share of the inverse permutation (one pass per
  // thread for the batches here, instead of S / 1024 dependent round trips
  // in one workgroup)
  for (int p = blockIdx.x * kPrepThreads + tid; p < S; p += gridDim.x * kPrepThreads) {
    const int s = sorted_slots[p];
    if (s >= 0 && s < S) pos[s] = p;
  }
  if (blockIdx.x > 0) {  // the other workgroups clear the accumulator region
    const int64_t stride = static_cast<int64_t>(gridDim.x - 1) * kPrepThreads;
    for (int64_t i = (blockIdx.x - 1) * static_cast<int64_t>(kPrepThreads) + tid; i < zero_n4;
         i += stride)
      zero[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  // the work queues of the persistent GEMM launches start empty
  if (tid >= kQueueBase && tid < kQueueBase + 2 * kXcds) counts[tid] = 0;

  // M-tiles: one item per expert, rows [offsets[e*L], offsets[(e+1)*L]).
  {
    const int per = (E + kPrepThreads - 1) / kPrepThreads;
    const int i0 = min(E, tid * per), i1 = min(E, i0 + per);
    int total = 0;
    const int first =
        block_exclusive_scan(count_tiles(offsets, i0, i1, L, bm, S), wave_tmp, &total);
    emit_tiles(offsets, i0, i1, L, bm, first, S, max_mt, mtiles);
    // expert_tiles[e] = index of expert e's first M-tile; expert_tiles[E] = count
    int t = first;
    for (int i = i0; i < i1; ++i) {
      expert_tiles[i] = min(t, max_mt);
      t += count_tiles(offsets, i, i + 1, L, bm, S);
    }
    if (tid == 0) {
      counts[0] = min(total, max_mt);
      expert_tiles[E] = min(total, max_mt);
    }
  }
  // LoRA tiles: one item per (expert, adapter) bucket.
  {
    const int nb = E * L;
    const int per = (nb + kPrepThreads - 1) / kPrepThreads;
    const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
    int total = 0;
    const int first =
        block_exclusive_scan(count_tiles(offsets, i0, i1, 1, bml, S), wave_tmp, &total);
    emit_tiles(offsets, i0, i1, 1, bml, first, S, max_lt, ltiles);
    if (tid == 0) counts[1] = min(total, max_lt);
  }
}

hipError_t launch_prep(const int32_t* sorted_slots, const int32_t* offsets, int S, int E, int L,
                       const TilePlan& plan, int32_t* pos, int4* mtiles, int4* ltiles,
                       int32_t* counts, int32_t* expert_tiles, float* zero, int64_t zero_n,
                       hipStream_t stream) {
  const int64_t n4 = zero_n / 4;  // callers pass multiples of 4
  int64_t zblocks = (n4 + kPrepThreads - 1) / kPrepThreads;
  if (zblocks > 512) zblocks = 512;
  // at least one pass of the inverse permutation per thread
  zblocks = std::max<int64_t>(zblocks, (S + kPrepThreads - 1) / kPrepThreads - 1);
  hipLaunchKernelGGL(k_prep, dim3(static_cast<unsigned>(1 + zblocks)), dim3(kPrepThreads), 0,
                     stream, sorted_slots, offsets, S, E, L, plan.bm, plan.bml, plan.max_mt,
                     plan.max_lt, pos, mtiles, ltiles, counts, expert_tiles,
                     reinterpret_cast<float4*>(zero), n4);
  return hipGetLastError();
}

// ------------------------------------------------------------------------- zero
// A plain fill kernel (no hipMemsetAsync: the call must stay capture-friendly).
__global__ void __launch_bounds__(256) k_zero(float4* __restrict__ p, int64_t n4) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += gridDim.x * 256ll)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;  // callers pass multiples of 4
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

// ------------------------------------------------------------------- LDS gemm
// P = number of K-steps whose global loads are in flight ahead of the MFMAs
// (register ring of P stages); NT = weights are loaded with the nontemporal
// hint (each weight element is used by one M-tile only in decode batches).
template <bool NT>
__device__ __forceinline__ uint4 load16(const void* p) {
  if (NT) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  return *reinterpret_cast<const uint4*>(p);
}

// 16-byte chunk swizzle of the LDS tiles (rows of 128 bytes = 8 chunks).  A
// fragment read has 16 consecutive rows read the same logical chunk; with 64
// LDS banks those 16 x 16 bytes must cover all banks, i.e. rows r and r + 8 of
// equal parity must land on different chunks: chunk ^ ((row >> 1) & 7).
template <int SWZ>
__device__ __forceinline__ int swz(int row) { return SWZ == 0 ? (row & 7) : ((row >> 1) & 7); }

__device__ __forceinline__ uint4 masked(uint4 v, uint32_t m) {
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Epilogues of the grouped GEMMs.  EPI_STORE writes the fp32 tile to C
// (relaxed atomics under split K).  The two fused forms first add the LoRA
// expand of the tile's rows to the accumulators and then,
// EPI_GATE_UP, apply SiLU(gate) * up and write bf16 ACT, or, EPI_DOWN, write
// D.  The vLLM blog page "Multi-LoRA" (section "Implementing Multi-LoRA
// inference for MoE models in vLLM") names folding the LoRA add into the base
// GEMM's output as the next fusion step.
// EPI_GATE_UP_FOLD: EPI_GATE_UP plus the down projection's shrink folded in
// (an instantiation of its own, so that the other kernels carry none of it).
enum { EPI_STORE = 0, EPI_GATE_UP = 1, EPI_DOWN = 2, EPI_GATE_UP_FOLD = 3 };
__host__ __device__ constexpr bool is_gu(int epi) { return epi == EPI_GATE_UP || epi == EPI_GATE_UP_FOLD; }
__host__ __device__ constexpr int expand_form(int epi) { return is_gu(epi) ? EPI_GATE_UP : epi; }

// One lane's 16 bytes of a 1 KiB direct-to-LDS copy (lane i lands at dst + 16 i).
__device__ __forceinline__ void dma_piece(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
}

// Byte offset of (row, col) in a k-major LDS tile with rows of `pitch` bytes
// (at least 16 chunks of 16 bytes): the 64-byte groups of a row are XORed with
// row % 4, so that the four rows of a transposed read fall on different banks.
__device__ __forceinline__ int kn_lds_off(int row, int col, int pitch) {
  return row * pitch + ((((col >> 3) ^ ((row & 3) << 2))) << 4) + ((col & 7) << 1);
}

// The 32x32x16 bf16 B fragment of a k-major LDS tile (rows = k, `pitch` bytes
// per row, kn_lds_off layout) for the lane's column: two transposed reads of
// four k each.  cbase: the tile column of lane c32 & ~15 (the lane's column
// is cbase + (c32 & 15), consecutive over its 16-lane group); k0: the first of
// the fragment's 16 k (the lane takes k0 + 8h .. + 7).
__device__ __forceinline__ bf16x8_t kn_frag(const unsigned char* tile, int pitch, int cbase, int k0,
                                            int lane) {
  const int i = lane & 15, h = lane >> 5;
  const int col = cbase + 4 * (i & 3);
  const int r = k0 + 8 * h + (i >> 2);
  const uint2 a = ds_read_tr16(tile + kn_lds_off(r, col, pitch));
  const uint2 b = ds_read_tr16(tile + kn_lds_off(r + 4, col, pitch));
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}

// The fused LoRA expand of a tile with its operands staged in `lds_bytes` of
// LDS that the K loop has finished with (whole KiB).  z of the tile's rows
// (fp32, rows [row0, row_end), at most tm of them, resident for the whole
// epilogue) and, for a group of adapter buckets, the B^T rows of the tile's tn
// columns are copied with global_load_lds (1 KiB pieces spread over the
// workgroup's nwaves waves) in one round trip per group; then each wave with
// rows adds z . B^T of every bucket meeting its rows [rw0, rw1) (FM blocks of
// 32) to its accumulators on the MFMAs (z split into bf16 hi + lo, rows
// outside the bucket masked to zero).  Buckets [lb, ub) of expert e are those
// meeting the tile.  EPI_GATE_UP: the tile's columns are gate i in
// [n0, n0 + tn/2) and up I + i, staged as the tn/2 gate rows then the tn/2 up
// rows; EPI_DOWN: [n0, n0 + tn).  lrow[j]: the staged row of the lane's
// column in fragment j.  KN (k-major B, [r][columns]): a bucket's tile is
// staged as r rows of tn columns (kn_lds_off layout, the same bytes) and read
// with transposed reads.
template <int EPI, int FM, int FN, bool KN = false>
__device__ __forceinline__ void staged_lora_expand(f32x16_t (&acc)[FM][FN], const LoraEpilogue& lora,
                                                   unsigned char* lds, int lds_bytes, int nwaves,
                                                   int e, int lb, int ub, int row0, int row_end,
                                                   int tm, int tn, int64_t n0, int64_t N,
                                                   const int (&lrow)[FN], bool active, int rw0,
                                                   int rw1, int wave, int lane, int c32, int h) {
  const int rk = lora.rank, nks = rk / 16;
  const int zbytes = tm * rk * 4;
  const int bbytes = tn * rk * 2;
  // buckets per group, >= 2 for the tiles that call this (128 x 128 in
  // 64 KiB, 256 x 256 in 128 KiB) at every supported rank
  const int cap = (lds_bytes - zbytes) / bbytes;
  const int32_t* off = lora.offsets + static_cast<int64_t>(e) * lora.buckets;
  // [src, src + bytes) to LDS dst in 1 KiB pieces; the lanes past the end
  // reload the last 16 bytes (their LDS bytes stay inside the piece and are
  // never read)
  auto copy = [&](unsigned char* dst, const void* src, int bytes) {
    const unsigned char* s8 = static_cast<const unsigned char*>(src);
    for (int c = wave; c * 1024 < bytes; c += nwaves)
      dma_piece(s8 + min(c * 1024 + lane * 16, bytes - 16), dst + c * 1024);
  };
  // k-major B block Bb ([rk][b_rows]): staged row q holds the tile's tn
  // columns; each lane fetches the logical chunk that belongs at its LDS
  // position (columns past the end fetch the segment's first chunk: never read)
  const int64_t I = N / 2;
  const int pitch = tn * 2;
  const int valid_cols = static_cast<int>(EPI == EPI_GATE_UP ? min<int64_t>(tn / 2, I - n0)
                                                             : min<int64_t>(tn, N - n0));
  auto copy_kn = [&](unsigned char* dst, const bf16_t* Bb) {
    for (int c = wave; c * 1024 < bbytes; c += nwaves) {
      const int o = c * 1024 + lane * 16;
      const int q = o / pitch, lc = ((o % pitch) >> 4) ^ ((q & 3) << 2);
      int col = lc * 8;
      int64_t g;
      if (EPI == EPI_GATE_UP) {
        const int up = col >= tn / 2;
        const int ci = col - up * (tn / 2);
        g = up * I + n0 + (ci < valid_cols ? ci : 0);
      } else {
        g = n0 + (col < valid_cols ? col : 0);
      }
      dma_piece(Bb + static_cast<int64_t>(q) * lora.b_rows + g, dst + c * 1024);
    }
  };
  for (int g = lb; g < ub; g += cap) {  // uniform
    const int ng = min(cap, ub - g);
    lds_barrier();  // every wave is done with what the LDS held before
    if (g == lb) copy(lds, lora.z + static_cast<int64_t>(row0) * rk, (row_end - row0) * rk * 4);
    for (int b = 0; b < ng; ++b) {
      const bf16_t* Bb = lora.b + (static_cast<int64_t>(g + b) * lora.experts + e) * lora.b_rows * rk;
      unsigned char* dst = lds + zbytes + b * bbytes;
      if (KN) {
        copy_kn(dst, Bb);
      } else if (EPI == EPI_GATE_UP) {
        const int bytes = valid_cols * rk * 2;
        copy(dst, Bb + n0 * rk, bytes);
        copy(dst + bbytes / 2, Bb + (I + n0) * rk, bytes);
      } else {
        copy(dst, Bb + n0 * rk, valid_cols * rk * 2);
      }
    }
    wait_vmcnt<0>();
    lds_barrier();
    if (!active) continue;
    for (int b = 0; b < ng; ++b) {
      const int s0 = max(rw0, off[g + b]), s1 = min(rw1, off[g + b + 1]);
      if (s0 >= s1) continue;  // uniform: the bucket misses this wave's rows
      bf16x8_t bfr[FN][4];
      if (KN) {
        const unsigned char* bt = lds + zbytes + b * bbytes;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            bfr[j][q4] = kn_frag(bt, pitch, lrow[j] - (c32 & 15), 16 * min(q4, nks - 1), lane);
      } else {
        const unsigned char* bt = lds + zbytes + b * bbytes + 16 * h;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            if (q4 < nks)  // (rk is known at run time only: no reads for unused steps)
              bfr[j][q4] = *reinterpret_cast<const bf16x8_t*>(bt + lrow[j] * rk * 2 + 32 * q4);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int rb = rw0 + 32 * i;
        if (rb >= s1 || rb + 32 <= s0) continue;  // uniform: block outside the bucket
        const int p = rb + c32;
        const bool in = p >= s0 && p < s1;
        const float* zr =
            reinterpret_cast<const float*>(lds) + (min(max(p, s0), s1 - 1) - row0) * rk + 8 * h;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          if (q4 >= nks) break;
          bf16x8_t zh, zl;
          split_bf16x8(zr + 16 * q4, zh, zl);
          if (!in) zh = zl = Mfma<bf16_t>::zero();
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zh, bfr[j][q4], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zl, bfr[j][q4], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  }
}

// The down projection's LoRA shrink folded into the fused gate_up epilogue:
// once a tile has its activation a = SiLU(gate) * up (rounded to bf16, the
// values it stores), it adds its tn columns' share of z2[p] = a[p] . A_dn[l][e]
// (the sum over the intermediate columns, section "Implementing Multi-LoRA
// inference for MoE models in vLLM" of the Multi-LoRA page: the shrink of the
// down projection) for each of its rows, so that no pass re-reads ACT.
// acc[i][j][r], j < FG: the lane's activation values (accumulator layout:
// block i of 32 rows from rw0, element r at row acc_row(r, h), intermediate
// column col[j]; wr[j]: this lane owns that column, i.e. when a wave holds one
// 32-column fragment the lane holds the gate half; col_ok[j]: the column is
// below I).  The tile's rows [row0, row_end) (at most tm) x columns
// [it0, it0 + tn) go to LDS column-major (a column's tm rows contiguous, four
// rows per 8-byte write), the layout of a k-major operand, and are read back as
// MFMA row fragments with transposed reads; each wave takes (32-row block,
// 32-rank block) items and, per adapter bucket meeting a block, loads all of
// the bucket's A_dn fragments for the tile's columns, then multiplies (rows
// outside the bucket zero, K = tn) and adds the results to Z2 (atomics, or the
// N-tile's partial slot).
__device__ __forceinline__ int fold_off(int row, int col, int pitch) {
  // 64-byte groups of a row XORed so that four consecutive rows of a
  // transposed read sit on different banks
  const int x = pitch >= 256 ? (row & 3) << 2 : (pitch == 128 ? ((row >> 1) & 1) << 2 : 0);
  return row * pitch + (((col >> 3) ^ x) << 4) + ((col & 7) << 1);
}

template <int FM, int FN, int FG, bool KN>
__device__ __forceinline__ void folded_down_shrink(const f32x16_t (&acc)[FM][FN],
                                                   const int64_t (&col)[FN], const bool (&wr)[FN],
                                                   const bool (&col_ok)[FN], int rw0,
                                                   const LoraEpilogue& lora, unsigned char* lds,
                                                   int nwaves, int e, int row0, int row_end, int tm,
                                                   int tn, int64_t it0, int64_t I, int nt, int wave,
                                                   int lane) {
  const int c32 = lane & 31, h = lane >> 5;
  const int rk = lora.rank, pitch = tm * 2;
  lds_barrier();  // the epilogue before this one is done with the LDS
  // every (row < row_end, column) of the tile is written: past I with zeros
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jg = 0; jg < FG; ++jg) {
      if (!wr[jg]) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int p = rw0 + 32 * i + 8 * g + 4 * h;  // rows p .. p + 3
        if (p >= row_end) continue;
        const f32x16_t& a = acc[i][jg];
        const uint32_t lo = col_ok[jg] ? (f32_to_bf16(a[4 * g]) | (static_cast<uint32_t>(f32_to_bf16(a[4 * g + 1])) << 16)) : 0u;
        const uint32_t hi = col_ok[jg] ? (f32_to_bf16(a[4 * g + 2]) | (static_cast<uint32_t>(f32_to_bf16(a[4 * g + 3])) << 16)) : 0u;
        *reinterpret_cast<uint2*>(lds + fold_off(static_cast<int>(col[jg] - it0), p - row0, pitch)) =
            make_uint2(lo, hi);
      }
    }
  lds_barrier();
  const int32_t* off = lora.offsets + static_cast<int64_t>(e) * lora.buckets;
  const int nblk = (min(row_end - row0, tm) + 31) / 32;
  const int nqb = (rk + 31) / 32;
  const int nks = tn / 16;  // 4 or 8
  for (int b = wave; b < nblk * nqb; b += nwaves) {  // (row block, rank block) items
    const int rb = row0 + 32 * (b / nqb), qb = b % nqb;
    const int rb1 = min(row_end, rb + 32);
    f32x16_t z = zero_acc();
    bool any = false;
    // adapter buckets meeting rows [rb, rb1); a base-only bucket has no LoRA
    int l = 0, hi_l = lora.adapters - 1;
    while (l < hi_l) {
      const int mid = (l + hi_l + 1) >> 1;
      if (off[mid] <= rb) l = mid; else hi_l = mid - 1;
    }
    for (; l < lora.adapters && off[l] < rb1; ++l) {
      const int s0 = max(rb, off[l]), s1 = min(rb1, off[l + 1]);
      if (s0 >= s1) continue;  // uniform
      any = true;
      const bf16_t* A = lora.dn_a + (static_cast<int64_t>(l) * lora.experts + e) * rk * I;
      // all the bucket's A_dn fragments for the tile's columns first
      bf16x8_t fb[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks >= nks) break;
        const int64_t k = it0 + 16 * ks + 8 * h;  // this lane's 8 columns
        if (KN) {
          // A_dn [I][r]: the lane's aligned 8-lane group loads 8 columns (k-rows)
          // of 8 ranks and transposes them
          const int qc = 32 * qb + (c32 & 24);
          const bool ok = qc < rk && k < I;
          const uint4 v = transpose8(*reinterpret_cast<const uint4*>(
              A + (ok ? (k + (c32 & 7)) * rk + qc : 0)));
          fb[ks] = ok ? __builtin_bit_cast(bf16x8_t, v) : Mfma<bf16_t>::zero();
        } else {
          const int q = 32 * qb + c32;
          const bool ok = q < rk && k < I;
          fb[ks] = ok ? *reinterpret_cast<const bf16x8_t*>(A + static_cast<int64_t>(q) * I + k)
                      : Mfma<bf16_t>::zero();
        }
      }
      const int p = rb + c32;
      const bool in = p >= s0 && p < s1;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks >= nks) break;
        // rows rb .. rb + 31 (the lane's row c32), columns 16 ks + 8 h ..
        const int i = lane & 15;
        const int pl = rb - row0 + (c32 & 16) + 4 * (i & 3);
        const int cl = 16 * ks + 8 * h + (i >> 2);
        const uint2 u0 = ds_read_tr16(lds + fold_off(cl, pl, pitch));
        const uint2 u1 = ds_read_tr16(lds + fold_off(cl + 4, pl, pitch));
        bf16x8_t fa = __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
        if (!in) fa = Mfma<bf16_t>::zero();
        z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb[ks], z, 0, 0, 0);
      }
    }
    if (!any) continue;  // uniform
    const int q = 32 * qb + c32;
    if (q >= rk) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = rb + acc_row(r, h);
      if (p >= rb1) continue;
      const int64_t idx = static_cast<int64_t>(p) * rk + q;
      if (lora.dn_parts != nullptr)
        lora.dn_parts[nt * lora.dn_part_stride + idx] = z[r];
      else
        atomic_add_relaxed(lora.dn_z + idx, z[r]);
    }
  }
}

// Adapter buckets of expert e meeting rows [row0, row_end), as [lb, ub); a
// base-only bucket, if any, comes last in the expert and is left out.
// lb is the last bucket starting at or before row0 (0 if none), ub the first
// at or after lb starting at or after row_end.  Up to 64 adapters every lane
// of the wave loads one bucket start and two ballots give both ends in one
// memory round trip (the offsets are nondecreasing, so the buckets starting
// before row_end are a prefix); above that a binary search and a scan.
__device__ __forceinline__ void lora_buckets(const LoraEpilogue& lora, int e, int row0, int row_end,
                                             int& lb, int& ub) {
  const int32_t* off = lora.offsets + static_cast<int64_t>(e) * lora.buckets;
  const int nad = lora.adapters;
  if (nad <= kWave) {
    const int l = threadIdx.x & (kWave - 1);
    const int o = l < nad ? off[l] : 0;
    const uint64_t le = __ballot(l < nad && o <= row0);
    const uint64_t lt = __ballot(l < nad && o < row_end);
    lb = le == 0 ? 0 : 63 - __builtin_clzll(le);
    ub = max(lb, __popcll(lt));
    return;
  }
  lb = 0;
  int hb = nad - 1;
  while (lb < hb) {
    const int mid = (lb + hb + 1) >> 1;
    if (off[mid] <= row0) lb = mid; else hb = mid - 1;
  }
  ub = lb;
  while (ub < nad && off[ub] < row_end) ++ub;
}

// ksplit > 1: workgroup (tile, s) covers the s-th of ksplit K ranges and adds
// its partial tile to C with relaxed fp32 atomics (C must be zero before).
// PIPE: the LDS writes of K-step kt+1 and the global loads of K-step kt+2 are
// issued between the MFMAs of K-step kt (one barrier per K-step); requires P = 1.
// EPI: EPI_STORE, or a fused LoRA epilogue (bf16, unsplit K).  EPI_GATE_UP
// tiles cover BN/2 columns i of the intermediate width I = N/2 and load the
// weight rows so that gate i and up I + i meet in the same wave: with two or
// more 32-column fragments per wave, fragment j < FN/2 holds gate columns and
// j + FN/2 the matching up columns (same lane); with one, lanes c < 16 hold
// gate and lanes c + 16 the matching up columns.
// KN: the weights are k-major ([K][N]); each aligned group of VEC lanes loads
// VEC k-rows of VEC consecutive columns and transposes them in registers, so
// the LDS tile and the fragment reads are those of the K-contiguous layout.
template <typename T, int BM, int BN, int WM, int WN, int P, bool NT, bool GATHER, bool SCHED = false,
          int SWZ = 1, bool PIPE = false, int EPI = EPI_STORE, bool KN = false>
__global__ void __launch_bounds__(WM * WN * kWave)
k_gemm(const T* __restrict__ X, int x_rows, const int32_t* __restrict__ gather_slots, int gather_k,
       const T* __restrict__ Wt, int64_t N, int64_t K, float* __restrict__ C,
       const int4* __restrict__ mtiles, const int32_t* __restrict__ counts,
       const int32_t* __restrict__ expert_tiles, int n_ntiles, int ksplit, float* __restrict__ parts,
       int64_t part_stride, LoraEpilogue lora, int order) {
  typedef Mfma<T> M;
  constexpr int NT_ = WM * WN * kWave;
  constexpr int ROWB = 128;                    // bytes of K per LDS row
  constexpr int BK = ROWB / sizeof(T);
  constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int A_CH = BM * 8 / NT_;
  constexpr int B_CH = BN * 8 / NT_;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(A_CH >= 1 && B_CH >= 1 && BM * 8 % NT_ == 0 && BN * 8 % NT_ == 0, "tile/threads");
  static_assert(FM >= 1 && FN >= 1 && P >= 1, "wave tile");
  // k-major bf16 weights stay k-major in LDS (a K-step's 64 k-rows of BN
  // columns, the same bytes as BN rows of 128) and are read transposed
  constexpr bool KNL = KN && sizeof(T) == 2;
  static_assert(!KNL || BN >= 128, "kn_lds_off needs rows of 16 chunks");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2][(BM + BN) * ROWB];

  // Workgroup order.  The grid is sized from a host-side bound; the first
  // counts[0] * n_ntiles workgroups are the real ones.  Hardware hands
  // consecutive workgroup ids to the 8 XCDs in turn; ORDER_XCD remaps the real
  // ones so that consecutive logical ids run on the same XCD (each XCD gets
  // an equal share), then each expert's tiles are walked N-tile by N-tile with
  // its M-tiles innermost, so M-tiles sharing one weight tile run together on
  // one XCD (one L2).
  const int ks = static_cast<int>(blockIdx.x) % ksplit;
  const int pid = static_cast<int>(blockIdx.x) / ksplit;
  const int active = counts[0] * n_ntiles;
  if (pid >= active) return;
  const int xcd = pid % kXcds, q = active / kXcds, rem = active % kXcds;
  const bool xcd_grouped = order_xcd(order);
  const int bid = xcd_grouped ? xcd * q + min(xcd, rem) + pid / kXcds : pid;
  const int t0 = bid / n_ntiles;
  const int ex = mtiles[t0].x;
  const int ta = expert_tiles[ex], tb = expert_tiles[ex + 1];
  const int local = bid - ta * n_ntiles;
  const int nt = local / (tb - ta);
  const int m_local = local % (tb - ta);  // M-tile of the expert, from its first
  const int mt = ta + m_local;
  const int4 tile = mtiles[mt];
  const int e = tile.x, row0 = tile.y, row_end = tile.z;
  const int64_t n0 = static_cast<int64_t>(nt) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int c32 = lane & 31, h = lane >> 5;

  // global sources and LDS destinations of this thread's 16-byte chunks.
  // Rows outside the tile read a clamped valid row and store zeros instead
  // (a select, not a branch).
  const T* a_src[A_CH];
  uint32_t a_mask[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int q = tid + i * NT_, row = q >> 3, ch = q & 7;
    const int p = row0 + row;
    a_mask[i] = p < row_end ? 0xffffffffu : 0u;
    const int pc = p < row_end ? p : row_end - 1;
    const int r = GATHER ? gather_slots[pc] / gather_k : pc;
    a_src[i] = X + static_cast<int64_t>(min(max(r, 0), x_rows - 1)) * K + ch * VEC;
    a_dst[i] = row * ROWB + ((ch ^ swz<SWZ>(row)) << 4);
  }
  const T* b_src[B_CH];
  uint32_t b_mask[B_CH];
  int b_dst[B_CH];
  const T* We = Wt + static_cast<int64_t>(e) * N * K;
  const int64_t I = N / 2;                          // EPI_GATE_UP: intermediate width
  const int64_t it0 = static_cast<int64_t>(nt) * (BN / 2);
  // EPI_GATE_UP: the intermediate column i and gate (0) / up (1) half of
  // wave column group wg's fragment j, lane column c
  auto gu_col = [&](int wg, int j, int c, int& up) -> int64_t {
    if (FN >= 2) {
      up = j >= FN / 2;
      return it0 + wg * (WTN / 2) + (j % (FN / 2 > 0 ? FN / 2 : 1)) * 32 + c;
    }
    up = c >= 16;
    return it0 + wg * 16 + (c & 15);
  };
  // the weight column (gate_up: up * I + intermediate column) of tile row
  // `row`, clamped to a valid one when it is past the end (ok = false)
  auto w_col = [&](int row, bool& ok) -> int64_t {
    if (is_gu(EPI)) {
      int up;
      const int64_t ic = gu_col(row / WTN, (row % WTN) / 32, row & 31, up);
      ok = ic < I;
      return up * I + (ok ? ic : I - 1);
    }
    const int64_t n = n0 + row;
    ok = n < N;
    return ok ? n : N - 1;
  };
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int q = tid + i * NT_;
    bool ok;
    if (!KN) {
      const int row = q >> 3, ch = q & 7;
      b_src[i] = We + w_col(row, ok) * K + ch * VEC;
      b_dst[i] = BM * ROWB + row * ROWB + ((ch ^ swz<SWZ>(row)) << 4);
    } else {
      // block q / VEC: k-group kg (VEC k-rows) x column group cg (VEC tile
      // rows); lane m of the block loads k-row kg * VEC + m of the group's
      // columns.  bf16: the chunk is stored as loaded into a k-major LDS tile
      // (k-rows of BN columns, kn_lds_off layout) and the fragments are read
      // with transposed reads; fp32: the block is transposed across its lanes,
      // after which lane m holds tile row cg * VEC + m, chunk kg
      const int blk = q / VEC, m = q % VEC, ncg = BN / VEC;
      const int cg = blk % ncg, kg = blk / ncg;
      int64_t col0 = w_col(cg * VEC, ok);  // VEC consecutive columns, all valid or none
      if (!ok) col0 = 0;                   // masked: any VEC columns inside the row
      b_src[i] = We + static_cast<int64_t>(kg * VEC + m) * N + col0;
      const int row = cg * VEC + m;
      b_dst[i] = KNL ? BM * ROWB + kn_lds_off(kg * VEC + m, cg * VEC, BN * 2)
                     : BM * ROWB + row * ROWB + ((kg ^ swz<SWZ>(row)) << 4);
    }
    b_mask[i] = ok ? 0xffffffffu : 0u;
  }
  const int64_t b_kmul = KN ? N : 1;  // elements of B per unit of K

  // ORDER_ROTATED: every workgroup starts its K walk at a different step, so that
  // workgroups resident together do not all read the same K columns at once.
  // ORDER_XCD_STAGGERED: the M-tiles sharing a weight tile start kOrderStagger
  // steps apart (those sharing activation rows together), so that one of them
  // brings each weight step into L2 a little before the others read it
  const int nk_all = static_cast<int>(K / BK);
  const int nk_per = (nk_all + ksplit - 1) / ksplit;
  const int kbeg = min(nk_all, ks * nk_per);
  const int nk = min(nk_all, kbeg + nk_per) - kbeg;  // K-steps of this workgroup
  const bool rot = order == ORDER_ROTATED || order == ORDER_XCD_ROTATED;
  const int kstart =
      nk <= 0 ? 0
      : rot   ? static_cast<int>((static_cast<int64_t>(blockIdx.x) * 37) % nk)
      : order == ORDER_XCD_STAGGERED ? (kOrderStagger * m_local) % nk
              : 0;
  uint4 a_reg[P][A_CH], b_reg[P][B_CH];
  auto gload = [&](int slot, int kt) {
    int kk = kt + kstart;
    if (kk >= nk) kk -= nk;
    const int64_t ko = static_cast<int64_t>(kbeg + kk) * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) a_reg[slot][i] = load16<false>(a_src[i] + ko);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) b_reg[slot][i] = load16<NT>(b_src[i] + ko * b_kmul);
  };
  auto sstore = [&](int slot, int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      *reinterpret_cast<uint4*>(&smem[buf][a_dst[i]]) = masked(a_reg[slot][i], a_mask[i]);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const uint4 v = (KN && !KNL) ? transpose_chunk<T>(b_reg[slot][i]) : b_reg[slot][i];
      *reinterpret_cast<uint4*>(&smem[buf][b_dst[i]]) = masked(v, b_mask[i]);
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = zero_acc();

  // byte offset of lane's fragment inside an LDS row, for K-step ks
  auto frag_off = [&](int row, int ks) {
    const int byte = (ks * M::KSTEP + h * M::KPACK) * static_cast<int>(sizeof(T));
    return row * ROWB + ((((byte >> 4) ^ swz<SWZ>(row))) << 4) + (byte & 15);
  };
  // Fragments of K-step ks+1 are read from LDS while the MFMAs of step ks
  // run (two fragment sets); the scheduling hints interleave one LDS read with
  // every MFMA_PER_READ MFMAs of the step.
  constexpr int KSN = BK / M::KSTEP;
  constexpr int READS = FM + FN;
  constexpr int MFMAS = FM * FN;
  typedef typename M::frag_t frag_t;
  auto read = [&](frag_t (&af)[FM], frag_t (&bfr)[FN], const unsigned char* As,
                  const unsigned char* Bs, int ks) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[i] = M::load(reinterpret_cast<const T*>(As + frag_off(wm * WTM + i * 32 + c32, ks)));
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (KNL)
        bfr[j] = kn_frag(Bs, BN * 2, wn * WTN + j * 32 + (c32 & 16), ks * M::KSTEP, lane);
      else
        bfr[j] = M::load(reinterpret_cast<const T*>(Bs + frag_off(wn * WTN + j * 32 + c32, ks)));
    }
  };
  auto mma = [&](const frag_t (&af)[FM], const frag_t (&bfr)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) M::run(acc[i][j], af[i], bfr[j]);
    if (SCHED) {
#pragma unroll
      for (int r = 0; r < READS; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                            // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, (MFMAS + READS - 1) / READS, 0);  // MFMAs
      }
    }
  };
  // hook(step) runs between the MFMAs of K-steps step and step+1
  auto compute_h = [&](int buf, auto&& hook) {
    const unsigned char* As = smem[buf];
    const unsigned char* Bs = smem[buf] + BM * ROWB;
    frag_t a0[FM], b0[FN], a1[FM], b1[FN];
    read(a0, b0, As, Bs, 0);
#pragma unroll
    for (int ks = 0; ks < KSN; ks += 2) {
      if (ks + 1 < KSN) read(a1, b1, As, Bs, ks + 1);
      mma(a0, b0);
      hook(ks);
      if (ks + 2 < KSN) read(a0, b0, As, Bs, ks + 2);
      if (ks + 1 < KSN) {
        mma(a1, b1);
        hook(ks + 1);
      }
    }
  };
  auto compute = [&](int buf) { compute_h(buf, [](int) {}); };

  // K-step kt lives in register slot kt % P until it is copied to LDS buffer kt % 2
  if (nk <= 0) return;  // uniform: an empty K split (only for tiny K)
#pragma unroll
  for (int s = 0; s < P; ++s)
    if (s < nk) gload(s, s);
  sstore(0, 0);
  __syncthreads();
  if (PIPE) {
    static_assert(!PIPE || P == 1, "PIPE uses a single register stage");
    if (1 < nk) gload(0, 1);  // slot 0 now holds K-step 1
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      compute_h(buf, [&](int step) {
        if (step == 0 && kt + 1 < nk) sstore(0, buf ^ 1);
        if (step == 1 && kt + 2 < nk) gload(0, kt + 2);
      });
      __syncthreads();
    }
  } else {
  if (P < nk) gload(0, P);
  for (int kt0 = 0; kt0 < nk; kt0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int kt = kt0 + u;
      if (kt < nk) {
        compute(kt & 1);
        if (kt + 1 < nk) sstore((u + 1) % P, (kt + 1) & 1);
        __syncthreads();
        if (kt + 1 + P < nk) gload((u + 1) % P, kt + 1 + P);
      }
    }
  }
  }

  if (EPI != EPI_STORE) {
    static_assert(EPI == EPI_STORE || sizeof(T) == 2, "fused epilogues are bf16");
    // output column of fragment j held by this lane
    int64_t col[FN];
    bool col_ok[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (is_gu(EPI)) {
        int up;
        col[j] = gu_col(wn, j, c32, up);
        col_ok[j] = col[j] < I;
      } else {
        col[j] = n0 + wn * WTN + j * 32 + c32;
        col_ok[j] = col[j] < N;
      }
    }
    const int rw0 = row0 + wm * WTM;  // this wave's rows [rw0, rw1)
    const int rw1 = min(row_end, rw0 + WTM);
    static_assert(EPI == EPI_STORE || FM <= 2, "the staged expand keeps z of FM blocks");
    if constexpr (NT_ >= 512) {
      // eight-wave tiles (two waves per SIMD per workgroup): the operands are
      // copied straight into the idle LDS stages, which costs no registers
      int lrow[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (is_gu(EPI)) {
          int up;
          const int64_t ic = gu_col(wn, j, c32, up);
          lrow[j] = up * (BN / 2) + static_cast<int>(ic - it0);
        } else {
          lrow[j] = wn * WTN + j * 32 + c32;
        }
      }
      int lb, ub;
      lora_buckets(lora, e, row0, row_end, lb, ub);
      staged_lora_expand<expand_form(EPI), FM, FN, KN>(acc, lora, &smem[0][0], 2 * (BM + BN) * ROWB, NT_ / kWave, e, lb,
                                      ub, row0, row_end, BM, BN,
                                      is_gu(EPI) ? it0 : n0, N, lrow, rw0 < rw1, rw0, rw1,
                                      wave, lane, c32, h);
    } else {
      // The expand with the B^T rows staged in the (now idle) LDS stages, a
      // group of NBUF adapter buckets per round trip: the workgroup walks the
      // non-empty buckets meeting its rows; every thread loads its chunks of
      // the group's B^T tiles (the tile rows of the main loop's B operand,
      // r wide) and writes them to LDS with the main loop's swizzle; each wave
      // then multiplies z of its rows (loaded and split once, rows outside the
      // bucket zero) by the fragments of every bucket meeting its rows.
      constexpr int BUCKET_BYTES = BN * ROWB;
      constexpr int NBUF = (2 * (BM + BN) * ROWB) / BUCKET_BYTES;
      static_assert(NBUF >= 1, "LDS holds a bucket's B^T tile");
      unsigned char* lds = &smem[0][0];
      const int32_t* off = lora.offsets + static_cast<int64_t>(e) * lora.buckets;
      const int A = lora.adapters, rk = lora.rank, nks = rk / 16;
      bf16x8_t zh[FM][4], zl[FM][4];
      int prow[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        prow[i] = rw0 + 32 * i + c32;
        const float* zr = lora.z + static_cast<int64_t>(min(prow[i], row_end - 1)) * rk + 8 * h;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) split_bf16x8(zr + 16 * min(q4, nks - 1), zh[i][q4], zl[i][q4]);
      }
      // this thread's B^T chunks: tile row and LDS position as in the main loop
      // (k-major B: the block of rank rows x columns this lane's group loads,
      // stored k-major as in the main loop and read transposed)
      int64_t b_off[B_CH];
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int q = tid + i * NT_;
        bool ok;
        if (!KN) {
          const int row = q >> 3, ch = q & 7;
          // chunks past r reload the last chunk of the row (never read)
          b_off[i] = w_col(row, ok) * rk + 8 * min(ch, 2 * nks - 1);
        } else {
          const int blk = q / 8, m = q % 8, ncg = BN / 8;
          const int cg = blk % ncg, kg = blk / ncg;
          int64_t col0 = w_col(cg * 8, ok);
          if (!ok) col0 = 0;
          // rank groups past r reload the last group (never read)
          b_off[i] = static_cast<int64_t>(min(kg, 2 * nks - 1) * 8 + m) * lora.b_rows + col0;
        }
      }
      const bf16_t* Be = lora.b + static_cast<int64_t>(e) * lora.b_rows * rk;
      const int64_t bstride = static_cast<int64_t>(lora.experts) * lora.b_rows * rk;  // per adapter
      // the first non-empty bucket from l on that meets [row0, row_end), or A
      auto next = [&](int l) {
        for (; l < A && off[l] < row_end; ++l)
          if (off[l + 1] > max(off[l], row0)) return l;
        return A;
      };
      int lb = 0, ub = A - 1;  // last bucket starting at or before row0
      while (lb < ub) {
        const int mid = (lb + ub + 1) >> 1;
        if (off[mid] <= row0) lb = mid; else ub = mid - 1;
      }
      int l = next(lb);
      while (l < A) {  // uniform across the workgroup
        int grp[NBUF];
        int ng = 0;
#pragma unroll
        for (int g = 0; g < NBUF; ++g) {
          grp[g] = l;
          if (l < A) {
            ++ng;
            l = next(l + 1);
          }
        }
        uint4 bv[NBUF][B_CH];
#pragma unroll
        for (int g = 0; g < NBUF; ++g) {
          const bf16_t* Bl = Be + static_cast<int64_t>(grp[g] < A ? grp[g] : grp[0]) * bstride;
#pragma unroll
          for (int i = 0; i < B_CH; ++i) bv[g][i] = *reinterpret_cast<const uint4*>(Bl + b_off[i]);
        }
#pragma unroll
        for (int g = 0; g < NBUF; ++g)
#pragma unroll
          for (int i = 0; i < B_CH; ++i)
            *reinterpret_cast<uint4*>(lds + g * BUCKET_BYTES + b_dst[i] - BM * ROWB) = bv[g][i];
        __syncthreads();
        for (int g = 0; g < ng; ++g) {
          const int lg = grp[g];
          const int s0 = max(rw0, off[lg]), s1 = min(rw1, off[lg + 1]);
          if (s0 >= s1) continue;  // uniform per wave: the bucket misses its rows
          const unsigned char* Bs = lds + g * BUCKET_BYTES;
          bf16x8_t bfr[FN][4];
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              if constexpr (KNL)
                bfr[j][q4] = kn_frag(Bs, BN * 2, wn * WTN + j * 32 + (c32 & 16), 16 * min(q4, nks - 1), lane);
              else
                bfr[j][q4] = M::load(reinterpret_cast<const T*>(
                    Bs + frag_off(wn * WTN + j * 32 + c32, min(q4, nks - 1))));
            }
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int rb = rw0 + 32 * i;
            if (rb >= s1 || rb + 32 <= s0) continue;  // uniform: block outside the bucket
            const bool in = prow[i] >= s0 && prow[i] < s1;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              if (q4 >= nks) break;
              const bf16x8_t zha = in ? zh[i][q4] : Mfma<bf16_t>::zero();
              const bf16x8_t zla = in ? zl[i][q4] : Mfma<bf16_t>::zero();
#pragma unroll
              for (int j = 0; j < FN; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zha, bfr[j][q4], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zla, bfr[j][q4], acc[i][j], 0, 0, 0);
              }
            }
          }
        }
        __syncthreads();  // every wave is done with the group before the next one lands
      }
    }
    if (is_gu(EPI)) {
      constexpr int FG = FN >= 2 ? FN / 2 : 1;  // gate fragments
      bool wr[FN];  // the lane owns column col[j] (gate half of the wave's fragment)
#pragma unroll
      for (int j = 0; j < FN; ++j) wr[j] = j < FG && (FN >= 2 || c32 < 16);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FG; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // FN == 1: the up value sits 16 lanes over (every lane takes part)
            const float g = acc[i][j][r];
            const float u = FN >= 2 ? acc[i][FN >= 2 ? j + FG : 0][r] : __shfl_xor(g, 16);
            acc[i][j][r] = silu(g) * u;  // the activation, in place of gate
            const int p = rw0 + 32 * i + acc_row(r, h);
            if (wr[j] && col_ok[j] && p < row_end)
              lora.act[static_cast<int64_t>(p) * I + col[j]] = f32_to_bf16(acc[i][j][r]);
          }
      if constexpr (EPI == EPI_GATE_UP_FOLD)
        folded_down_shrink<FM, FN, FG, KN>(acc, col, wr, col_ok, rw0, lora, &smem[0][0], NT_ / kWave,
                                           e, row0, row_end, BM, BN / 2, it0, I, nt, wave, lane);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int p = rw0 + 32 * i + acc_row(r, h);
            if (p < row_end && col_ok[j]) C[static_cast<int64_t>(p) * N + col[j]] = acc[i][j][r];
          }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * WTN + j * 32 + c32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = row0 + wm * WTM + i * 32 + acc_row(r, h);
        if (p < row_end && n < N) {
          const int64_t idx = static_cast<int64_t>(p) * N + n;
          if (ksplit == 1)
            C[idx] = acc[i][j][r];
          else if (parts != nullptr)  // deterministic: this split's partial
            parts[ks * part_stride + idx] = acc[i][j][r];
          else
            atomic_add_relaxed(C + idx, acc[i][j][r]);
        }
      }
    }
}

struct GemmArgs {
  const void* X;
  int x_rows;
  const int32_t* gather_slots;
  int gather_k;
  const void* Wt;
  int64_t N, K;
  float* C;
  const int4* mtiles;
  const int32_t* counts;
  const int32_t* expert_tiles;
  int ksplit;
  float* parts;         // split-K partials, or nullptr
  int64_t part_stride;  // elements per partial (rows of C times N)
  int32_t* queue;       // kXcds tile-queue counters (zero) for a persistent launch, or nullptr
};

template <bool KN, typename T, int BM, int BN, int WM, int WN, int P, bool NT, bool GATHER,
          bool SCHED = false, int SWZ = 1, bool PIPE = false, int EPI = EPI_STORE>
static hipError_t lds_launch_epi(const TilePlan& plan, const GemmArgs& a, const LoraEpilogue& lora,
                                 hipStream_t stream) {
  const int64_t cols = is_gu(EPI) ? a.N / 2 : a.N;
  const int tn = is_gu(EPI) ? BN / 2 : BN;
  const int n_ntiles = static_cast<int>((cols + tn - 1) / tn);
  const int64_t grid = static_cast<int64_t>(plan.max_mt) * n_ntiles * a.ksplit;
  hipLaunchKernelGGL((k_gemm<T, BM, BN, WM, WN, P, NT, GATHER, SCHED, SWZ, PIPE, EPI, KN>),
                     dim3(static_cast<unsigned>(grid)), dim3(WM * WN * kWave), 0, stream,
                     static_cast<const T*>(a.X), a.x_rows, a.gather_slots, a.gather_k,
                     static_cast<const T*>(a.Wt), a.N, a.K, a.C, a.mtiles, a.counts,
                     a.expert_tiles, n_ntiles, a.ksplit, a.parts, a.part_stride, lora, plan.order);
  return hipGetLastError();
}

// the epilogue picked by lora: none (EPI_STORE), gate_up (act set) or down
template <bool KN, typename T, int BM, int BN, int WM, int WN, int P, bool NT, bool GATHER,
          bool SCHED = false, int SWZ = 1, bool PIPE = false>
static hipError_t lds_launch(const TilePlan& plan, const GemmArgs& a, const LoraEpilogue* lora,
                             hipStream_t stream) {
  if constexpr (sizeof(T) == 2 && BM <= 128) {  // bf16 256-row tiles run k_gemm_dma
    if (lora != nullptr && lora->act != nullptr && lora->dn_a != nullptr)
      return lds_launch_epi<KN, T, BM, BN, WM, WN, P, NT, GATHER, SCHED, SWZ, PIPE,
                            EPI_GATE_UP_FOLD>(plan, a, *lora, stream);
    if (lora != nullptr && lora->act != nullptr)
      return lds_launch_epi<KN, T, BM, BN, WM, WN, P, NT, GATHER, SCHED, SWZ, PIPE,
                            EPI_GATE_UP>(plan, a, *lora, stream);
    if (lora != nullptr)
      return lds_launch_epi<KN, T, BM, BN, WM, WN, P, NT, GATHER, SCHED, SWZ, PIPE,
                            EPI_DOWN>(plan, a, *lora, stream);
  }
  return lds_launch_epi<KN, T, BM, BN, WM, WN, P, NT, GATHER, SCHED, SWZ, PIPE>(
      plan, a, LoraEpilogue{}, stream);
}


// ------------------------------------------------------------- DMA gemm
// bf16 tiles of BM x 256 outputs whose operands go from global memory straight
// into LDS (global_load_lds_dwordx4, no register round trip, no LDS store
// instructions), K staged in steps of 64 (128-byte rows).  Eight waves (two
// per SIMD) of BM/2 x 64 outputs.  The LDS rows keep the 16-byte-chunk XOR
// swizzle of the register-staged kernel: a load instruction fills 8 whole
// rows, each lane fetching the global chunk that belongs at its LDS position.
//  * BM = 256 (prefill: many rows per expert, every weight tile reused by
//    several M-tiles, bound by the matrix cores): two stages of 64 KiB; step
//    kt+2 is requested as soon as every wave has read step kt, so one step of
//    loads is always in flight behind the MFMAs.
//  * BM = 128 (one M-tile per expert, e.g. a dense layer's 128 tokens: the
//    weights stream through once, bound by HBM): three stages of 48 KiB, so
//    that two steps of weight loads are in flight; 256 weight rows per tile
//    halve the activation re-reads per weight byte against 128-row tiles.

constexpr int kDmaTile = 256;                       // weight rows (BN) of a tile
constexpr int kDmaRowB = 128;                       // bytes of K per LDS row (64 bf16)
constexpr int kDmaThreads = 512;

template <int BM>
struct DmaShape {
  static_assert(BM == 128 || BM == 256, "DMA tiles have 128 or 256 activation rows");
  static constexpr int kStages = BM == 256 ? 2 : 3;
  static constexpr int kStage = (BM + kDmaTile) * kDmaRowB;  // A and B rows of one K-step
  static constexpr int kARows = BM / 8;                      // activation rows loaded per wave
  static constexpr int kAIns = kARows / 8;                   // ... in load instructions of 8 rows
  static constexpr int kLoads = kAIns + 4;                   // loads per wave per K-step
  static constexpr int kWaveRows = BM / 2;                   // a wave's output rows
  static constexpr int kFM = kWaveRows / 32;                 // ... in 32-row MFMA blocks
};

// The kAIns A and four B load instructions of one wave for the K-step at
// element offset ko into the stage at `st` (8 rows of 128 bytes each; KN,
// k-major weights: the B tile is 64 k-rows of 512 bytes, 2 rows per
// instruction, and the step advances the weight rows by ko * N).
template <int BM, bool KN>
__device__ __forceinline__ void dma_issue(unsigned char* st, int64_t ko, int64_t N,
                                          const bf16_t* const* a_src, const bf16_t* const* b_src,
                                          int wave) {
  typedef DmaShape<BM> S;
#pragma unroll
  for (int j = 0; j < S::kAIns; ++j)
    dma_piece(a_src[j] + ko, st + (S::kARows * wave + 8 * j) * kDmaRowB);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (KN)
      dma_piece(b_src[j] + ko * N, st + BM * kDmaRowB + (8 * wave + 2 * j) * (2 * kDmaTile));
    else
      dma_piece(b_src[j] + ko, st + (BM + 32 * wave + 8 * j) * kDmaRowB);
  }
}

// How a k_gemm_dma item writes its outputs: plain stores (the item covers the
// whole K range), relaxed fp32 atomics into C (zero beforehand), or the
// item's partial slot (deterministic split K).
enum { DMA_OUT_STORE = 0, DMA_OUT_ATOMIC = 1, DMA_OUT_PART = 2 };

// One item of k_gemm_dma: the K-steps [kbeg, kbeg + nk) of output tile
// (M-tile `tile`, N-tile nt), written as `out` says; with_lora adds the fused
// LoRA expand (exactly one item of a tile carries it).  Every wave of the
// workgroup calls it with the same arguments.
template <int BM, bool GATHER, int EPI, bool KN>
__device__ __forceinline__ void dma_item(unsigned char* smem, const bf16_t* __restrict__ X,
                                         int x_rows, const int32_t* __restrict__ gather_slots,
                                         int gather_k, const bf16_t* __restrict__ Wt, int64_t N,
                                         int64_t K, float* __restrict__ C, int4 tile, int nt,
                                         int kbeg, int nk, int out, bool with_lora,
                                         const LoraEpilogue& lora, float* __restrict__ part,
                                         int kstart, int32_t* qpop, int& qraw) {
  typedef DmaShape<BM> S;
  constexpr int FM = S::kFM, WR = S::kWaveRows;
  // every wave is done with what the LDS held for the previous item (its
  // direct-to-LDS loads were all waited for; a persistent workgroup's next
  // tile does not wait for the previous epilogue's global stores either)
  if (qpop != nullptr)
    lds_only_barrier();
  else
    lds_barrier();
  const int e = tile.x, row0 = tile.y, row_end = tile.z;
  // Output columns.  EPI_GATE_UP: the tile covers 128 columns i of the
  // intermediate width I = N/2; wave column group wn owns i in
  // [n0 + 32 wn, +32), as weight rows i (gate, fragment j = 0) and I + i
  // (up, j = 1), so gate and up of one output meet in the same lane.
  // Otherwise 256 columns n of N, wave wn owning [n0 + 64 wn, +64).
  const int64_t I = N / 2;
  const int64_t cols = is_gu(EPI) ? I : N;
  const int64_t n0 = static_cast<int64_t>(nt) * (is_gu(EPI) ? 128 : kDmaTile);

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int wm = wave >> 2, wn = wave & 3;
  const int c32 = lane & 31, h = lane >> 5;

  // Load instruction j of wave w fills A rows kARows w + 8j + lane/8 and B
  // rows 32w + 8j + lane/8; the lane's LDS chunk is lane%8, so it fetches
  // logical chunk (lane%8) ^ swz(row).  Rows past the tile's end (M) or past
  // N read a valid clamped row: they only feed outputs that are never stored.
  const bf16_t* a_src[S::kAIns];
  const bf16_t* b_src[4];
  const bf16_t* We = Wt + static_cast<int64_t>(e) * N * K;
#pragma unroll
  for (int j = 0; j < S::kAIns; ++j) {
    const int rt = S::kARows * wave + 8 * j + (lane >> 3);
    const int lch = (lane & 7) ^ swz<1>(rt);
    const int p = min(row0 + rt, row_end - 1);
    const int r = GATHER ? gather_slots[p] / gather_k : p;
    a_src[j] = X + static_cast<int64_t>(min(max(r, 0), x_rows - 1)) * K + lch * 8;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rt = 32 * wave + 8 * j + (lane >> 3);
    const int lch = (lane & 7) ^ swz<1>(rt);
    if (!KN) {
      int64_t wrow;
      if (is_gu(EPI)) {  // B tile row rt = 64 wn' + 32 half + c
        const int64_t i = min(n0 + 32 * (rt >> 6) + (rt & 31), I - 1);
        wrow = ((rt >> 5) & 1) * I + i;
      } else {
        wrow = min(n0 + rt, N - 1);
      }
      b_src[j] = We + wrow * K + lch * 8;
    } else {
      // k-row kr of the B tile, LDS chunk lane % 32 holding the logical
      // chunk (tile columns) of the kn_lds_off layout; columns past the end
      // fetch the first chunk of their half (never stored)
      const int kr = 8 * wave + 2 * j + (lane >> 5);
      const int t = 8 * ((lane & 31) ^ ((kr & 3) << 2));
      int64_t col;
      if (is_gu(EPI)) {
        const int64_t i = n0 + 32 * (t >> 6) + (t & 31);
        col = ((t >> 5) & 1) * I + (i < I ? i : 0);
      } else {
        col = n0 + t < N ? n0 + t : 0;
      }
      b_src[j] = We + static_cast<int64_t>(kr) * N + col;
    }
  }
  // adapter buckets of expert e meeting the tile, [lb, ub) (looked up before
  // the K loop so that the epilogue does not wait for it); a base-only
  // bucket, if any, comes last in the expert and is skipped
  int lb = 0, ub = 0;
  if (EPI != EPI_STORE && with_lora) lora_buckets(lora, e, row0, row_end, lb, ub);

  f32x16_t acc[FM][2];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero_acc();

  // fragment reads: substep s (16 of the 64 K) of row r = WR wm + 32 i + c32;
  // (r >> 1) & 7 depends on c32 only
  const int sw = swz<1>(c32);
  const int a_off = (wm * WR + c32) * kDmaRowB;
  const int b_off = (BM + wn * 64 + c32) * kDmaRowB;
  bf16x8_t fa[2][FM], fb[2][2];
  // Only the wave's 32-row blocks that hold rows of the tile are read and
  // multiplied (NB of the FM; an expert's last tile is often partly empty);
  // the K loop below is instantiated per NB.
  auto rd = [&](int f, const unsigned char* st, int s, auto nbc) {
    constexpr int NB = decltype(nbc)::value;
    const int ch = ((2 * s + h) ^ sw) << 4;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      fa[f][i] = *reinterpret_cast<const bf16x8_t*>(st + a_off + i * 32 * kDmaRowB + ch);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (KN)
        fb[f][j] = kn_frag(st + BM * kDmaRowB, 2 * kDmaTile, wn * 64 + 32 * j + (c32 & 16),
                           16 * s, lane);
      else
        fb[f][j] = *reinterpret_cast<const bf16x8_t*>(st + b_off + j * 32 * kDmaRowB + ch);
    }
  };
  // One substep's MFMAs, with the fragment reads of the next substep (issued
  // just before in program order) placed one after each MFMA: the reads then
  // overlap the MFMA pipe instead of queueing as a burst, and each fragment
  // still lands a whole substep before its use.
  auto mm = [&](int f, auto nbc) {
    constexpr int NB = decltype(nbc)::value, NR = NB + (KN ? 4 : 2), NM = 2 * NB;
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][i], fb[f][j], acc[i][j], 0, 0, 0);
    constexpr int PAIRS = NR < NM ? NR : NM;
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    if constexpr (NM > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NM - PAIRS, 0);
    if constexpr (NR > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NR - PAIRS, 0);
  };
  // workgroup barrier that orders LDS accesses only; the DMA is waited for
  // explicitly with vmcnt.  Two stages: the fenced barrier (its fence waits
  // for every LDS write in flight, the DMA included, which the two-stage loop
  // has waited for anyway).  Three stages: a bare s_barrier, so that the
  // step still in flight stays in flight (a compiler barrier for memory
  // accesses on both sides).
  constexpr int NS = S::kStages, LD = S::kLoads;
  auto bar = [&]() {
    if constexpr (NS == 2) {
      lds_barrier();
    } else {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto ko = [&](int kt) {
    const int kk = kt + kstart;
    return static_cast<int64_t>(kbeg + (kk >= nk ? kk - nk : kk)) * 64;
  };
  auto stage = [&](int q) { return smem + q * S::kStage; };

  // K-step kt lives in stage kt % NS.  The first NS steps are requested up
  // front; steps past the end repeat the last one (never read), which keeps
  // the vmcnt accounting the same in every iteration.
#pragma unroll
  for (int q = 0; q < NS; ++q)
    dma_issue<BM, KN>(stage(q), ko(min(q, nk - 1)), N, a_src, b_src, wave);
  wait_vmcnt<(NS - 1) * LD>();  // this wave's loads of step 0 are in LDS
  bar();                        // ... and every other wave's
  auto k_loop = [&](auto nbc) {
    rd(0, smem, 0, nbc);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): nothing scalar or LDS pending into the loop
    int cs = 0;                          // stage of step kt
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const int nx = cs + 1 == NS ? 0 : cs + 1;  // stage of step kt+1
      unsigned char* cur = stage(cs);
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        rd((s + 1) & 1, cur, s + 1, nbc);
        mm(s & 1, nbc);
        __builtin_amdgcn_sched_barrier(0);
      }
      // step kt+1 has landed (step kt+2 may still be in flight) and every
      // wave has finished reading step kt (lgkmcnt(0) before the barrier):
      // refill that stage with step kt+NS
      wait_vmcnt_lgkm0<(NS - 2) * LD>();
      bar();
      dma_issue<BM, KN>(cur, ko(min(kt + NS, nk - 1)), N, a_src, b_src, wave);
      rd(0, stage(nx), 0, nbc);
      mm(1, nbc);
      __builtin_amdgcn_sched_barrier(0);
      cs = nx;
    }
    const unsigned char* cur = stage(cs);
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      rd((s + 1) & 1, cur, s + 1, nbc);
      mm(s & 1, nbc);
      __builtin_amdgcn_sched_barrier(0);
    }
    mm(1, nbc);
    __builtin_amdgcn_sched_barrier(0);
  };
  // 32-row blocks of this wave that hold tile rows (every wave runs the same
  // number of K steps and barriers whatever its count; in a 256-row tile of
  // at most 128 rows, an expert's last, the second wave row has none and
  // leaves its SIMD's matrix core to the first)
  const int wave_rows = min(WR, row_end - row0 - WR * wm);
  switch (max(0, (wave_rows + 31) / 32)) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, (FM < 2 ? FM : 2)>{}); break;
    case 3: k_loop(std::integral_constant<int, (FM < 3 ? FM : 3)>{}); break;
    default: k_loop(std::integral_constant<int, FM>{}); break;
  }
  wait_vmcnt<0>();  // no LDS write of this item may outlive it
  // persistent workgroup: take the next tile now, so that the pop's round trip
  // overlaps the epilogue (a pop at the start of the tile instead let the
  // M-tiles sharing a weight tile drift apart)
  if (qpop != nullptr && threadIdx.x == 0) qraw = atomicAdd(qpop, 1);

  // output column of fragment j held by this lane
  int64_t col[2];
  bool col_ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    col[j] = is_gu(EPI) ? n0 + 32 * wn + c32 : n0 + 64 * wn + 32 * j + c32;
    col_ok[j] = col[j] < cols;
  }
  const int rw0 = row0 + WR * wm;                  // this wave's rows [rw0, rw1)
  const int rw1 = min(row_end, rw0 + WR);

  if (EPI != EPI_STORE && with_lora) {
    // operands staged in the idle K stages: up to 14, 6, 2 buckets per round
    // trip at rank 16, 32, 64
    int lrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      lrow[j] = is_gu(EPI) ? j * (kDmaTile / 2) + 32 * wn + c32 : 64 * wn + 32 * j + c32;
    staged_lora_expand<expand_form(EPI), FM, 2, KN>(acc, lora, smem, NS * S::kStage,
                                                    kDmaThreads / kWave, e, lb, ub, row0, row_end,
                                                    BM, kDmaTile, n0, N, lrow, rw0 < rw1, rw0,
                                                    rw1, wave, lane, c32, h);
  }

  if (is_gu(EPI)) {
    // Activation (block i, accumulator element r) of this lane lies at row
    // rw0 + 4h + ro(i, r) of its column: a lane base address plus a row
    // offset that is the same for every lane (a scalar product), rather than
    // a 64-bit product per element.  A wave's 32 columns are all inside or
    // all outside the output (I is a multiple of 64, tile columns start at
    // multiples of 128), so a block with all of its 32 rows in the tile
    // stores without per-element tests.
    auto ro = [](int i, int r) { return 32 * i + acc_row(r, 0); };
    bf16_t* const act_l = lora.act + static_cast<int64_t>(rw0 + 4 * h) * I + col[0];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[i][0][r] = silu(acc[i][0][r]) * acc[i][1][r];  // the activation, in place of gate
      if (col_ok[0] && rw0 + 32 * i + 32 <= row_end) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          act_l[static_cast<int64_t>(ro(i, r)) * I] = f32_to_bf16(acc[i][0][r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (col_ok[0] && rw0 + 4 * h + ro(i, r) < row_end)
            act_l[static_cast<int64_t>(ro(i, r)) * I] = f32_to_bf16(acc[i][0][r]);
      }
    }
    if constexpr (EPI == EPI_GATE_UP_FOLD) {
      const bool wr[2] = {true, false};
      folded_down_shrink<FM, 2, 1, KN>(acc, col, wr, col_ok, rw0, lora, smem, kDmaThreads / kWave,
                                       e, row0, row_end, BM, 128, n0, I, nt, wave, lane);
    }
    return;
  }
  auto store = [&](auto&& put) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int p = rw0 + 32 * i + acc_row(r, h);
          if (p < row_end && col_ok[j]) put(C + static_cast<int64_t>(p) * N + col[j], acc[i][j][r]);
        }
  };
  if (out == DMA_OUT_STORE)
    store([](float* dst, float v) { *dst = v; });
  else if (out == DMA_OUT_PART)  // deterministic split K: this split's partial, same index
    store([&](float* dst, float v) { part[dst - C] = v; });
  else
    store([](float* dst, float v) { atomic_add_relaxed(dst, v); });
}


// The M-tile and N-tile of tile index bid (expert-major, per expert N-tile by
// N-tile with its M-tiles innermost); m_local: the M-tile's index inside its
// expert.
__device__ __forceinline__ void dma_tile_of(int bid, int n_ntiles, const int4* __restrict__ mtiles,
                                            const int32_t* __restrict__ expert_tiles, int4& tile,
                                            int& nt, int& m_local) {
  const int t0 = bid / n_ntiles;
  const int ex = mtiles[t0].x;
  const int ta = expert_tiles[ex], tb = expert_tiles[ex + 1];
  const int local = bid - ta * n_ntiles;
  nt = local / (tb - ta);
  m_local = local % (tb - ta);
  tile = mtiles[ta + m_local];
}

// Tiles of the data-parallel part when the last, partial round of tiles is
// spread over `nwg` stream-K workgroups instead: whole rounds of nwg tiles,
// when there is at least one and the remainder leaves a fifth of the
// workgroups or more idle; else all tiles.
__device__ __forceinline__ int dma_dp_tiles(int tiles, int nwg) {
  const int r = tiles % nwg;
  return tiles >= nwg && r != 0 && 5 * r <= 4 * nwg ? tiles - r : tiles;
}

// sk_mode 0: every tile, split K over ksplit workgroups per tile.
// sk_mode 1: the data-parallel tiles only (ksplit 1), each workgroup of the
// first r also clearing the output of one stream-K tile.
// sk_mode 2 (grid nwg): the r = tiles - dp remaining tiles as r * nk K-steps
// cut into nwg equal contiguous ranges, one per workgroup; a range meets at
// most two tiles and adds each part with atomics, the part holding K-step 0
// carrying the LoRA expand.  Used for the down projection, whose few long
// tiles otherwise leave a last round with most CUs idle.
template <int BM, bool GATHER, int EPI, bool KN>
__global__ void __launch_bounds__(kDmaThreads)
k_gemm_dma(const bf16_t* __restrict__ X, int x_rows, const int32_t* __restrict__ gather_slots,
           int gather_k, const bf16_t* __restrict__ Wt, int64_t N, int64_t K, float* __restrict__ C,
           const int4* __restrict__ mtiles, const int32_t* __restrict__ counts,
           const int32_t* __restrict__ expert_tiles, int n_ntiles, int ksplit, LoraEpilogue lora,
           float* __restrict__ parts, int64_t part_stride, int sk_mode, int nwg, int order,
           int32_t* __restrict__ queue) {
  // the K stages, then 32 bytes for the next tile of a persistent workgroup:
  // its index and descriptor (inside the one LDS array: a second LDS object
  // made the compiler wait for every direct-to-LDS load before each fragment
  // read of the K loop)
  constexpr int kStagesBytes = DmaShape<BM>::kStages * DmaShape<BM>::kStage;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStagesBytes + 32];
  int* const s_next = reinterpret_cast<int*>(smem + kStagesBytes);
  const int tiles = counts[0] * n_ntiles;
  const int dp = sk_mode == 0 ? tiles : dma_dp_tiles(tiles, nwg);
  const int nk_all = static_cast<int>(K / 64);
  // Persistent workgroups (queue != nullptr; the gate_up forms' data-parallel
  // tiles without stream-K, unsplit K, XCD-grouped order): one workgroup per CU takes tile after tile from the
  // queue of its XCD (the XCD-grouped numbering: XCD y's tiles are the
  // contiguous run [y q + min(y, rem), + q + (y < rem))), then from the other
  // XCDs' queues once its own is empty.  No workgroup launch between tiles,
  // and the XCDs finish together.  queue[y] counts the pops of run y; it
  // starts at zero and may overshoot its run's length.
  // (compiled for the gate_up forms only: the others run stream-K for their
  // last round, and the persistent loop's code cost their K loop 1-2 %)
  const bool pers = is_gu(EPI) && queue != nullptr && sk_mode != 2;
  const int qq = dp / kXcds, qrem = dp % kXcds, qx = static_cast<int>(blockIdx.x) % kXcds;
  auto qlen = [&](int y) { return qq + (y < qrem ? 1 : 0); };
  auto pop = [&](int idx0) {  // thread 0; idx0 >= 0: a pop of run qx already made
    if (idx0 < 0) idx0 = atomicAdd(&queue[qx], 1);
    if (idx0 < qlen(qx)) return qx * qq + min(qx, qrem) + idx0;
    // the own run is done: read every run's counter at once, then pop from
    // those not yet exhausted
    int c[kXcds];
#pragma unroll
    for (int y = 0; y < kXcds; ++y)
      c[y] = __hip_atomic_load(&queue[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = 1; i < kXcds; ++i) {
      const int y = (qx + i) % kXcds;
      if (c[y] >= qlen(y)) continue;
      const int idx = atomicAdd(&queue[y], 1);
      if (idx < qlen(y)) return y * qq + min(y, qrem) + idx;
    }
    return -1;
  };
  // thread 0: the next tile and its descriptor to s_next ([0] tile index or
  // -1, [1..4] the M-tile, [5] N-tile, [6] M-tile within the expert), so that
  // the descriptor's three dependent loads overlap the other waves' epilogue
  // instead of following the barrier
  auto pop_next = [&](int idx0) {
    const int b = pop(idx0);
    s_next[0] = b;
    if (b >= 0) {
      int4 t;
      int n, m;
      dma_tile_of(b, n_ntiles, mtiles, expert_tiles, t, n, m);
      s_next[1] = t.x;
      s_next[2] = t.y;
      s_next[3] = t.z;
      s_next[4] = t.w;
      s_next[5] = n;
      s_next[6] = m;
    }
  };
  // the items of this workgroup: one (tile, K split) in modes 0 and 1 (tiles
  // until the queues are empty when persistent), the units [u, u1) in mode 2
  // (one call site of dma_item, so one inlined copy)
  int u = 0, u1 = 0;  // at most 255 tiles x 16384 K-steps
  int bid = 0, ks = 0;
  int raw = -1;  // thread 0: the pop of run qx made during the last epilogue
  if (sk_mode == 2) {
    const int64_t units = static_cast<int64_t>(tiles - dp) * nk_all;
    u = static_cast<int>(units * blockIdx.x / nwg);
    u1 = static_cast<int>(units * (blockIdx.x + 1) / nwg);
  } else if (pers) {
    if (threadIdx.x == 0) pop_next(-1);
    __syncthreads();
    bid = s_next[0];
    if (bid < 0) return;  // uniform
    u1 = 1;
  } else {
    // workgroup order: XCD remap over the real workgroups, then tile index
    ks = static_cast<int>(blockIdx.x) % ksplit;
    const int pid = static_cast<int>(blockIdx.x) / ksplit;
    if (pid >= dp) return;
    const int xcd = pid % kXcds, q = dp / kXcds, rem = dp % kXcds;
    bid = order_xcd(order) ? xcd * q + min(xcd, rem) + pid / kXcds : pid;
    if (sk_mode == 1 && bid < tiles - dp) {
      // clear the output of stream-K tile dp + bid (the next launch adds into it)
      int4 st;
      int snt, sml;
      dma_tile_of(dp + bid, n_ntiles, mtiles, expert_tiles, st, snt, sml);
      const int64_t c0 = static_cast<int64_t>(snt) * kDmaTile;
      const int nc4 = static_cast<int>(min<int64_t>(kDmaTile, N - c0)) / 4;
      for (int i = threadIdx.x; i < (st.z - st.y) * (kDmaTile / 4); i += kDmaThreads) {
        const int rr = i / (kDmaTile / 4), c4 = i % (kDmaTile / 4);
        if (c4 < nc4)
          *reinterpret_cast<float4*>(C + static_cast<int64_t>(st.y + rr) * N + c0 + 4 * c4) =
              make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    u1 = 1;
  }
  while (u < u1) {  // uniform
    int4 tile;
    int nt, m_local, kbeg, nk, out;
    bool with_lora;
    float* part = nullptr;
    if (sk_mode == 2) {
      const int t = u / nk_all;
      kbeg = u % nk_all;
      nk = min(nk_all - kbeg, u1 - u);
      dma_tile_of(dp + t, n_ntiles, mtiles, expert_tiles, tile, nt, m_local);
      out = DMA_OUT_ATOMIC;
      with_lora = kbeg == 0;
      u += nk;
    } else {
      if (pers) {
        tile = make_int4(s_next[1], s_next[2], s_next[3], s_next[4]);
        nt = s_next[5];
        m_local = s_next[6];
      } else {
        dma_tile_of(bid, n_ntiles, mtiles, expert_tiles, tile, nt, m_local);
      }
      const int nk_per = (nk_all + ksplit - 1) / ksplit;
      kbeg = min(nk_all, ks * nk_per);
      nk = min(nk_all, kbeg + nk_per) - kbeg;
      if (nk <= 0) return;  // uniform: an empty K split (only for tiny K)
      out = ksplit == 1 ? DMA_OUT_STORE : (parts != nullptr ? DMA_OUT_PART : DMA_OUT_ATOMIC);
      if (parts != nullptr) part = parts + ks * part_stride;
      with_lora = true;
      if (!pers) u = u1;
    }
    // rotated or staggered K walk (data-parallel items only, as in k_gemm):
    // this workgroup starts at step kstart
    int kstart = 0;
    if (sk_mode != 2 && nk > 0) {
      if (order == ORDER_ROTATED || order == ORDER_XCD_ROTATED)
        kstart = static_cast<int>((static_cast<int64_t>(blockIdx.x) * 37) % nk);
      else if (order == ORDER_XCD_STAGGERED)
        kstart = (kOrderStagger * m_local) % nk;
    }
    dma_item<BM, GATHER, EPI, KN>(smem, X, x_rows, gather_slots, gather_k, Wt, N, K, C, tile, nt,
                                  kbeg, nk, out, with_lora, lora, part, kstart,
                                  pers ? queue + qx : nullptr, raw);
    if (pers) {
      // every wave has read s_next (the item's barriers lie between)
      if (threadIdx.x == 0) pop_next(raw);
      lds_only_barrier();
      bid = s_next[0];
      if (bid < 0) u = u1;  // uniform
    }
  }
}

// Stream-K for the non-gate_up forms with unsplit K and no deterministic
// partials, when the tiles exceed one round: the data-parallel launch, then
// the stream-K launch over one workgroup per CU.
template <int BM, bool GATHER, int EPI, bool KN>
static hipError_t dma_launch(const TilePlan& plan, const GemmArgs& a, const LoraEpilogue& lora,
                             hipStream_t stream) {
  const int64_t cols = is_gu(EPI) ? a.N / 2 : a.N;
  const int tn = is_gu(EPI) ? 128 : kDmaTile;
  const int n_ntiles = static_cast<int>((cols + tn - 1) / tn);
  const int64_t grid = static_cast<int64_t>(plan.max_mt) * n_ntiles * a.ksplit;
  int nwg = 0;  // CUs: one stream-K workgroup each
  if (!is_gu(EPI) && a.ksplit == 1 && !plan.det) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&nwg, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
  }
  // the tiles' upper bound must reach a round for the device to pick stream-K
  const int mode = nwg > 0 && static_cast<int64_t>(plan.max_mt) * n_ntiles >= nwg ? 1 : 0;
  // persistent data-parallel launch: one workgroup per CU over the tile
  // queues, when the tiles may exceed one round (unsplit K, XCD-grouped order)
  int ncu = 0;
  // (not with stream-K, which already evens out the last round)
  const bool pers = is_gu(EPI) && a.queue != nullptr && a.ksplit == 1 && mode == 0 &&
                    (plan.order == ORDER_XCD || plan.order == ORDER_XCD_STAGGERED);
  if (pers) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
  }
  const bool use_q = pers && grid > ncu;
  hipLaunchKernelGGL((k_gemm_dma<BM, GATHER, EPI, KN>),
                     dim3(static_cast<unsigned>(use_q ? ncu : grid)), dim3(kDmaThreads), 0, stream,
                     static_cast<const bf16_t*>(a.X), a.x_rows, a.gather_slots, a.gather_k,
                     static_cast<const bf16_t*>(a.Wt), a.N, a.K, a.C, a.mtiles, a.counts,
                     a.expert_tiles, n_ntiles, a.ksplit, lora, a.parts, a.part_stride, mode, nwg,
                     plan.order, use_q ? a.queue : nullptr);
  if (mode == 0) return hipGetLastError();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_dma<BM, GATHER, EPI, KN>), dim3(static_cast<unsigned>(nwg)), dim3(kDmaThreads),
                     0, stream, static_cast<const bf16_t*>(a.X), a.x_rows, a.gather_slots, a.gather_k,
                     static_cast<const bf16_t*>(a.Wt), a.N, a.K, a.C, a.mtiles, a.counts,
                     a.expert_tiles, n_ntiles, 1, lora, a.parts, a.part_stride, 2, nwg, plan.order,
                     nullptr);
  return hipGetLastError();
}

// the DMA tiles' epilogue picked by lora, as in lds_launch
template <int BM, bool GATHER, bool KN>
static hipError_t dma_dispatch(const TilePlan& plan, const GemmArgs& a, const LoraEpilogue* lora,
                               hipStream_t stream) {
  if (lora == nullptr) return dma_launch<BM, GATHER, EPI_STORE, KN>(plan, a, LoraEpilogue{}, stream);
  if (lora->act != nullptr && lora->dn_a != nullptr)
    return dma_launch<BM, GATHER, EPI_GATE_UP_FOLD, KN>(plan, a, *lora, stream);
  if (lora->act != nullptr) return dma_launch<BM, GATHER, EPI_GATE_UP, KN>(plan, a, *lora, stream);
  return dma_launch<BM, GATHER, EPI_DOWN, KN>(plan, a, *lora, stream);
}

template <typename T, bool GATHER, bool KN>
static hipError_t gemm_dispatch(const TilePlan& plan, const GemmArgs& a, const LoraEpilogue* lora,
                                hipStream_t stream) {
  // decode-sized M-tiles stream the weights: nontemporal loads, rotated K walk
  switch (plan.bm) {
    case 32: return lds_launch<KN, T, 32, 128, 1, 4, 2, true, GATHER>(plan, a, lora, stream);
    case 64: return lds_launch<KN, T, 64, 128, 2, 2, 2, true, GATHER>(plan, a, lora, stream);
    case 128:
      if constexpr (sizeof(T) == 2) {
        if (plan.dma128)  // 128 x 256 DMA tiles, three stages
          return dma_dispatch<128, GATHER, KN>(plan, a, lora, stream);
      }
      if (plan.stream)  // eight waves of 64 x 32
        return lds_launch<KN, T, 128, 128, 2, 4, 2, true, GATHER>(plan, a, lora, stream);
      return lds_launch<KN, T, 128, 128, 2, 2, 1, false, GATHER, false, 1, true>(plan, a, lora, stream);
    case 256:  // prefill: 256x256 tiles, 8 waves of 128x64 (bf16: operands DMA'd into LDS)
      if constexpr (sizeof(T) == 2) {
        return dma_dispatch<256, GATHER, KN>(plan, a, lora, stream);
      } else {
        return lds_launch<KN, T, 256, 256, 2, 4, 1, false, GATHER, false, 1, true>(plan, a, nullptr, stream);
      }
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool KN>
static hipError_t gemm_dispatch_g(bool gather, const TilePlan& plan, const GemmArgs& a,
                                  const LoraEpilogue* lora, hipStream_t stream) {
  return gather ? gemm_dispatch<T, true, KN>(plan, a, lora, stream)
                : gemm_dispatch<T, false, KN>(plan, a, lora, stream);
}

hipError_t launch_gemm(int dtype, const TilePlan& plan, const void* X, int x_rows,
                       const int32_t* gather_slots, int gather_k, const void* Wt, int64_t N,
                       int64_t K, float* C, int64_t c_rows, const int4* mtiles,
                       const int32_t* counts, const int32_t* expert_tiles, int ksplit,
                       const LoraEpilogue* lora, float* parts, hipStream_t stream,
                       bool sum_parts, int32_t* queue) {
  ksplit = ksplit < 1 ? 1 : ksplit;
  float* pp = ksplit > 1 ? parts : nullptr;
  const GemmArgs a{X, x_rows, gather_slots, gather_k, Wt, N, K, C, mtiles, counts, expert_tiles,
                   ksplit, pp, c_rows * N, queue};
  const bool gather = gather_slots != nullptr;
  // the fused epilogues: bf16, unsplit K
  if (lora != nullptr && (dtype != DT_BF16 || a.ksplit != 1))
    return hipErrorInvalidValue;
  hipError_t e;
  if (dtype == DT_BF16)
    e = plan.kn ? gemm_dispatch_g<bf16_t, true>(gather, plan, a, lora, stream)
                : gemm_dispatch_g<bf16_t, false>(gather, plan, a, lora, stream);
  else
    e = plan.kn ? gemm_dispatch_g<float, true>(gather, plan, a, nullptr, stream)
                : gemm_dispatch_g<float, false>(gather, plan, a, nullptr, stream);
  if (e == hipSuccess && pp != nullptr && sum_parts)
    e = launch_reduce_parts(pp, ksplit, c_rows * N, C, stream);
  return e;
}

// ------------------------------------------------------------ partial sums
// Deterministic split-K: out = parts[0] + parts[1] + ... in that order.
__global__ void __launch_bounds__(256)
k_reduce_parts(const float4* __restrict__ parts, int nparts, int64_t n4, float4* __restrict__ out) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += gridDim.x * 256ll) {
    float4 s = parts[i];
    for (int q = 1; q < nparts; ++q) {
      const float4 v = parts[q * n4 + i];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    out[i] = s;
  }
}

hipError_t launch_reduce_parts(const float* parts, int nparts, int64_t n, float* out,
                               hipStream_t stream) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_reduce_parts, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(parts), nparts, n4, reinterpret_cast<float4*>(out));
  return hipGetLastError();
}

}  // namespace moelora
