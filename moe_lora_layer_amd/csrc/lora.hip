// LoRA shrink and expand kernels of the MoE layer, and the top-k combination.
//
// The vLLM blog page "Multi-LoRA" (vllm.com.cn/blog/multi-lora) defines the
// ops (section "Implementing Multi-LoRA inference for MoE models in vLLM"):
// shrink z = xA takes h_in down to the rank r, expand zB takes it back up to
// h_out, per (expert, adapter).  Its section "Kernel optimisation" gives the
// design points kept here: the shrink's long h_in sums are split over several
// workgroups whose partial sums meet in relaxed fp32 atomics, and the LoRA add
// is fused with the base add inside the expand kernel.
//
// Work unit of every kernel: a LoRA tile = consecutive sorted rows of one
// (expert, adapter) bucket.  Products run on MFMA 16x16 blocks; the rank r
// (16/32/64) is the M of the shrink and the K of the expand.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moelora {

constexpr int kLoraThreads = 256;
constexpr int kLoraWaves = kLoraThreads / kWave;

// Both LoRA products put the adapter weights on the MFMA A side (16 weight rows
// x KSTEP elements of the rank or hidden dimension per fragment) and up to 16
// activation rows of the tile on the B side; a LoRA tile is processed as
// consecutive 16-row blocks, so the number of rows costs no registers and the
// weights of a tile are read once.  16x16 MFMA output held by lane (g, c):
// element (weight row 4*g + i, activation row c), i = 0..3.

// Loads the 8 (bf16) or 1 (fp32) z values of a lane's activation fragment.
// bf16 MFMA inputs get z split into a high and a low bf16 part, so z keeps
// about 16 significant bits through the expand product; fp32 uses z as is.
template <typename T> struct ZFrag;
template <> struct ZFrag<bf16_t> {
  bf16x8_t hi, lo;
  __device__ __forceinline__ void load(const float* z) { split_bf16x8(z, hi, lo); }
  __device__ __forceinline__ void clear() { hi = Mfma16<bf16_t>::zero(); lo = hi; }
  __device__ __forceinline__ void mma(f32x4_t& acc, bf16x8_t a) const {
    Mfma16<bf16_t>::run(acc, a, hi);
    Mfma16<bf16_t>::run(acc, a, lo);
  }
};
template <> struct ZFrag<float> {
  float v;
  __device__ __forceinline__ void load(const float* z) { v = *z; }
  __device__ __forceinline__ void clear() { v = 0.0f; }
  __device__ __forceinline__ void mma(f32x4_t& acc, float a) const { Mfma16<float>::run(acc, a, v); }
};

// The MFMA 16x16 fragment (lane (g, c): row rb + c, the KPACK elements
// k0 + g * KPACK ..) of a k-major matrix M[k][row] with ld elements per k-row
// (LoRA weights stored h_in x r or r x h_out).  bf16: the lane's aligned
// 8-lane group loads 8 k-rows of 8 consecutive rows and transposes them;
// fp32: one element.  ok (uniform per group) false: zero, and row 0 of k-row 0
// is read instead (always in range).  Every lane of the wave must call it.
template <typename T> struct KnFrag;
template <> struct KnFrag<bf16_t> {
  __device__ __forceinline__ static bf16x8_t load(const bf16_t* M, int64_t ld, int64_t rb, int64_t k0,
                                                  bool ok) {
    const int lane = threadIdx.x & (kWave - 1), g = lane >> 4, c = lane & 15;
    const int64_t kk = ok ? k0 + 8 * g + (c & 7) : 0, rr = ok ? rb + (c & 8) : 0;
    const uint4 v = transpose8(*reinterpret_cast<const uint4*>(M + kk * ld + rr));
    return ok ? __builtin_bit_cast(bf16x8_t, v) : Mfma16<bf16_t>::zero();
  }
};
template <> struct KnFrag<float> {
  __device__ __forceinline__ static float load(const float* M, int64_t ld, int64_t rb, int64_t k0,
                                               bool ok) {
    const int lane = threadIdx.x & (kWave - 1), g = lane >> 4, c = lane & 15;
    return ok ? M[(k0 + g) * ld + rb + c] : 0.0f;
  }
};

// --------------------------------------------------------------------- shrink
// Workgroup (tile, split): four waves take consecutive K ranges of STEPS
// MFMA steps each.  For every 16-row block of the tile a wave issues all its
// loads (weights A^T and the gathered activation rows) up front, multiplies,
// and the four partial z blocks are summed through LDS; the sum goes to Z with
// one relaxed fp32 atomic per element.
template <typename T, int R, int STEPS, bool GATHER, bool KN>
__global__ void __launch_bounds__(kLoraThreads)
k_shrink(const T* __restrict__ X, int x_rows, const int32_t* __restrict__ gather_slots, int gather_k,
         const T* __restrict__ At, int E, int L, int nad, int64_t K, int nsplit,
         float* __restrict__ Z, const int4* __restrict__ ltiles, const int32_t* __restrict__ counts,
         float* __restrict__ parts, int64_t part_stride) {
  typedef Mfma16<T> M;
  typedef typename M::frag_t frag_t;
  constexpr int RB = R / 16;                 // 16-row blocks of A^T
  constexpr int KW = STEPS * M::KSTEP;       // K elements per wave
  __shared__ float red[kLoraWaves][RB * 4 * kWave];

  const int lt = blockIdx.x / nsplit;
  const int split = blockIdx.x % nsplit;
  if (lt >= counts[1]) return;
  const int4 tile = ltiles[lt];
  const int b = tile.x, row0 = tile.y, row_end = tile.z;
  const int e = b / L, l = b % L;
  if (l >= nad) return;  // base-only bucket: no LoRA term

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int64_t k0 = (static_cast<int64_t>(split) * kLoraWaves + wave) * KW;

  const T* Ab = At + (static_cast<int64_t>(l) * E + e) * R * K;
  for (int m0 = row0; m0 < row_end; m0 += 16) {
    const int p = m0 + c;
    const T* xp = nullptr;
    if (p < row_end) {
      const int r = GATHER ? gather_slots[p] / gather_k : p;
      xp = X + static_cast<int64_t>(min(max(r, 0), x_rows - 1)) * K + g * M::KPACK;
    }
    frag_t af[STEPS][RB], xf[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int64_t k = k0 + s * M::KSTEP;
      const bool in = k < K;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        if (KN)
          af[s][j] = KnFrag<T>::load(Ab, R, 16 * j, k, in);
        else
          af[s][j] = in ? M::load(Ab + static_cast<int64_t>(16 * j + c) * K + g * M::KPACK + k) : M::zero();
      }
      xf[s] = (in && xp) ? M::load(xp + k) : M::zero();
    }
    f32x4_t acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
      for (int j = 0; j < RB; ++j) M::run(acc[j], af[s][j], xf[s]);

#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][(j * 4 + i) * kWave + lane] = acc[j][i];
    __syncthreads();
    for (int idx = tid; idx < RB * 4 * kWave; idx += kLoraThreads) {
      const int ln = idx % kWave, ji = idx / kWave;
      const int pr = m0 + (ln & 15);
      if (pr < row_end) {
        float v = red[0][idx];
#pragma unroll
        for (int w = 1; w < kLoraWaves; ++w) v += red[w][idx];
        const int q = (ji >> 2) * 16 + 4 * (ln >> 4) + (ji & 3);
        const int64_t idx = static_cast<int64_t>(pr) * R + q;
        if (parts != nullptr)
          parts[split * part_stride + idx] = v;
        else
          atomic_add_relaxed(Z + idx, v);
      }
    }
    __syncthreads();
  }
}

// Tall tiles (many rows per bucket): each wave owns a 16-row block of the
// tile and walks the workgroup's whole K range, STEPS MFMA steps at a time
// with the next STEPS in flight; no cross-wave reduction is needed, and each
// wave adds its z block to Z with one relaxed atomic per element.
template <typename T, int R, int STEPS, bool GATHER, bool KN>
__global__ void __launch_bounds__(kLoraThreads)
k_shrink_tall(const T* __restrict__ X, int x_rows, const int32_t* __restrict__ gather_slots,
              int gather_k, const T* __restrict__ At, int E, int L, int nad, int64_t K, int64_t kwg,
              int nsplit, float* __restrict__ Z, const int4* __restrict__ ltiles,
              const int32_t* __restrict__ counts, float* __restrict__ parts,
              int64_t part_stride) {
  typedef Mfma16<T> M;
  typedef typename M::frag_t frag_t;
  constexpr int RB = R / 16;
  constexpr int KB = STEPS * M::KSTEP;
  const int lt = blockIdx.x / nsplit;
  const int split = blockIdx.x % nsplit;
  if (lt >= counts[1]) return;
  const int4 tile = ltiles[lt];
  const int b = tile.x, row0 = tile.y, row_end = tile.z;
  const int e = b / L, l = b % L;
  if (l >= nad) return;  // base-only bucket: no LoRA term
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int64_t kb0 = static_cast<int64_t>(split) * kwg;
  const int64_t kb1 = kb0 + kwg < K ? kb0 + kwg : K;
  const T* Ablk = At + (static_cast<int64_t>(l) * E + e) * R * K;
  const T* Ab = Ablk + g * M::KPACK;

  for (int m0 = row0 + 16 * wave; m0 < row_end; m0 += 16 * kLoraWaves) {
    const int p = m0 + c;
    const bool ok = p < row_end;
    const int pc = ok ? p : row_end - 1;
    const int r = GATHER ? gather_slots[pc] / gather_k : pc;
    const T* xp = X + static_cast<int64_t>(min(max(r, 0), x_rows - 1)) * K + g * M::KPACK;
    f32x4_t acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    frag_t a0[STEPS][RB], x0[STEPS], a1[STEPS][RB], x1[STEPS];
    auto load = [&](frag_t (&af)[STEPS][RB], frag_t (&xf)[STEPS], int64_t k0) {
#pragma unroll
      for (int s2 = 0; s2 < STEPS; ++s2) {
        const int64_t k = k0 + s2 * M::KSTEP;
        const bool in = k < kb1;
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          if (KN)
            af[s2][j] = KnFrag<T>::load(Ablk, R, 16 * j, k, in);
          else
            af[s2][j] = in ? M::load(Ab + static_cast<int64_t>(16 * j + c) * K + k) : M::zero();
        }
        xf[s2] = (in && ok) ? M::load(xp + k) : M::zero();
      }
    };
    auto mma = [&](const frag_t (&af)[STEPS][RB], const frag_t (&xf)[STEPS]) {
#pragma unroll
      for (int s2 = 0; s2 < STEPS; ++s2)
#pragma unroll
        for (int j = 0; j < RB; ++j) M::run(acc[j], af[s2][j], xf[s2]);
    };
    int64_t k0 = kb0;
    if (k0 < kb1) load(a0, x0, k0);
    while (k0 < kb1) {
      if (k0 + KB < kb1) load(a1, x1, k0 + KB);
      mma(a0, x0);
      k0 += KB;
      if (k0 >= kb1) break;
      if (k0 + KB < kb1) load(a0, x0, k0 + KB);
      mma(a1, x1);
      k0 += KB;
    }
    if (ok) {
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t idx = static_cast<int64_t>(p) * R + 16 * j + 4 * g + i;
          if (parts != nullptr)
            parts[split * part_stride + idx] = acc[j][i];
          else
            atomic_add_relaxed(Z + idx, acc[j][i]);
        }
    }
  }
}


// --------------------------------------------------------- tall shrink (bf16)
// LoRA tiles of many rows (prefill): one workgroup per (tile, K range) streams
// the tile's activation rows (at most 64) and the adapter's A^T rows through a
// four-stage LDS ring of 64-wide K steps, loaded with global_load_lds in whole
// 128-byte rows (swizzled 16-byte chunks, as in the base GEMM).  z = x A^T runs
// on 32x32x16 MFMAs, activation rows on the A side and rank rows on the B
// side.  Wave w takes rows 32 (w % 2) .. +32 and, for R <= 32, substeps
// 2 (w / 2) and 2 (w / 2) + 1 of each K step (R = 64: rank half w / 2, all
// substeps); it adds its 32 x 32 partial to Z with relaxed fp32 atomics, so Z
// must be zero beforehand (the split-K of the page's "Kernel optimisation"),
// or, deterministic, stores it as partial (split, substep pair).
constexpr int kShrinkStages = 4;

template <int R> struct ShrinkDma {
  static constexpr int RP = R < 32 ? 32 : R;        // rank rows staged (16 padded to 32)
  static constexpr int STAGE = (64 + RP) * 128;     // activation rows, then A^T rows
  static constexpr int XI = 2;                      // activation load instructions per wave
  static constexpr int AI = RP / 32;                // A^T load instructions per wave
  static constexpr int LPW = XI + AI;               // loads per wave per stage
};

// KN (k-major A, [K][R]): the A part of a stage holds the step's 64 k-rows of
// R ranks (R * 2 bytes each, 64-byte halves XORed with bit 1 of the row at
// R = 64), copied as R / 8 pieces of 1 KiB; with R = 16 the last two waves
// repeat the first two waves' pieces.
template <int R>
__device__ __forceinline__ int shrink_kn_piece(int wave, int j) {
  return min(ShrinkDma<R>::AI * wave + j, R / 8 - 1);
}
template <int R>
__device__ __forceinline__ int shrink_kn_off(int row, int col) {
  const int sw = R == 64 ? ((row >> 1) & 1) << 2 : 0;
  return row * (R * 2) + ((((col >> 3) ^ sw)) << 4) + ((col & 7) << 1);
}

template <int R, bool KN>
__device__ __forceinline__ void shrink_issue(unsigned char* smem, int slot, int64_t ko,
                                             const bf16_t* const* x_src, const bf16_t* const* a_src,
                                             int wave) {
  typedef ShrinkDma<R> S;
  unsigned char* st = smem + slot * S::STAGE;
#pragma unroll
  for (int j = 0; j < S::XI; ++j)
    __builtin_amdgcn_global_load_lds(x_src[j] + ko, (lds_void_t*)(st + (16 * wave + 8 * j) * 128),
                                     16, 0, 0);
#pragma unroll
  for (int j = 0; j < S::AI; ++j) {
    if (KN)
      __builtin_amdgcn_global_load_lds(a_src[j] + ko * R,
                                       (lds_void_t*)(st + 64 * 128 + shrink_kn_piece<R>(wave, j) * 1024),
                                       16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(a_src[j] + ko,
                                       (lds_void_t*)(st + (64 + 8 * (S::AI * wave + j)) * 128), 16, 0, 0);
  }
}

// One K range [kt0, kt0 + nk) (in 64-wide steps) of one tall LoRA tile through
// the ring; the wave's 32 x 32 partial is left in acc.  `tile` is the tile's
// (bucket, row0, row_end); the caller has checked that its bucket has an
// adapter.
template <int R, bool GATHER, bool KN>
__device__ __forceinline__ void shrink_dma_range(unsigned char* smem, const bf16_t* __restrict__ X,
                                                 int x_rows, const int32_t* __restrict__ gather_slots,
                                                 int gather_k, const bf16_t* __restrict__ At, int E,
                                                 int L, int64_t K, int4 tile, int kt0, int nk,
                                                 f32x16_t& acc) {
  typedef ShrinkDma<R> S;
  const int b = tile.x, row0 = tile.y, row_end = tile.z;
  const int e = b / L, l = b % L;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int c32 = lane & 31, h = lane >> 5;

  // load sources (rows past the tile or the rank read a clamped valid row)
  const bf16_t* x_src[S::XI];
  const bf16_t* a_src[S::AI];
#pragma unroll
  for (int j = 0; j < S::XI; ++j) {
    const int rt = 16 * wave + 8 * j + (lane >> 3);
    const int lch = (lane & 7) ^ ((rt >> 1) & 7);
    const int p = min(row0 + rt, row_end - 1);
    const int r = GATHER ? gather_slots[p] / gather_k : p;
    x_src[j] = X + static_cast<int64_t>(min(max(r, 0), x_rows - 1)) * K + kt0 * 64ll + lch * 8;
  }
  const bf16_t* Ab = At + (static_cast<int64_t>(l) * E + e) * R * K;
#pragma unroll
  for (int j = 0; j < S::AI; ++j) {
    if (KN) {
      // byte o of the step's A part: k-row o / (2R), the logical chunk that
      // belongs at its physical position
      const int o = shrink_kn_piece<R>(wave, j) * 1024 + lane * 16;
      const int kr = o / (2 * R);
      const int sw = R == 64 ? ((kr >> 1) & 1) << 2 : 0;
      const int lch = ((o % (2 * R)) >> 4) ^ sw;
      a_src[j] = Ab + (kt0 * 64ll + kr) * R + lch * 8;
    } else {
      const int rt = 8 * (S::AI * wave + j) + (lane >> 3);
      const int lch = (lane & 7) ^ ((rt >> 1) & 7);
      a_src[j] = Ab + static_cast<int64_t>(min(rt, R - 1)) * K + kt0 * 64ll + lch * 8;
    }
  }

  const int rh = wave & 1;
  const int sel = wave >> 1;                  // substep pair (R <= 32) or rank half (R = 64)
  const int q0 = R > 32 ? 32 * sel : 0;       // first rank column of this wave
  const int sw = (c32 >> 1) & 7;              // row swizzle of rows 32 rh + c32 and q0 + c32
  const int x_off = (32 * rh + c32) * 128;
  const int a_off = (64 + q0 + c32) * 128;

  for (int s = 0; s + 1 < kShrinkStages; ++s)
    shrink_issue<R, KN>(smem, s, static_cast<int64_t>(min(s, nk - 1)) * 64, x_src, a_src, wave);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt landed (two newer stages may still fly) and this wave's reads of
    // stage kt-1 are done; after the barrier its slot takes stage kt+3 (steps
    // past the end repeat the last one and are never read)
    wait_vmcnt_lgkm0<S::LPW * (kShrinkStages - 2)>();
    lds_barrier();
    shrink_issue<R, KN>(smem, (kt + kShrinkStages - 1) % kShrinkStages,
                        static_cast<int64_t>(min(kt + kShrinkStages - 1, nk - 1)) * 64, x_src, a_src,
                        wave);
    const unsigned char* st = smem + (kt % kShrinkStages) * S::STAGE;
#pragma unroll
    for (int u = 0; u < (R > 32 ? 4 : 2); ++u) {
      const int sub = R > 32 ? u : 2 * sel + u;
      const int ch = ((2 * sub + h) ^ sw) << 4;
      const bf16x8_t fx = *reinterpret_cast<const bf16x8_t*>(st + x_off + ch);
      bf16x8_t fa;
      if (KN) {
        // rank columns q0 + c32 (a 16-lane group past R = 16 repeats the first 16)
        const int i = lane & 15;
        const int cb = min(q0 + (c32 & 16), R - 16);
        const int col = cb + 4 * (i & 3), r = 16 * sub + 8 * h + (i >> 2);
        const unsigned char* ap = st + 64 * 128;
        const uint2 lo = ds_read_tr16(ap + shrink_kn_off<R>(r, col));
        const uint2 hi = ds_read_tr16(ap + shrink_kn_off<R>(r + 4, col));
        fa = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
      } else {
        fa = *reinterpret_cast<const bf16x8_t*>(st + a_off + ch);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx, fa, acc, 0, 0, 0);
    }
  }
  wait_vmcnt<0>();  // no LDS write of this workgroup may outlive the range
}

// The wave's 32 x 32 partial of a tall tile into partial slot `slot` (R > 32:
// the split; else split and substep pair); a separate pass sums the slots in
// order into Z.
template <int R>
__device__ __forceinline__ void shrink_dma_emit(const f32x16_t& acc, int4 tile,
                                                float* __restrict__ parts, int64_t part_stride,
                                                int slot) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int c32 = lane & 31, h = lane >> 5;
  const int rh = wave & 1, sel = wave >> 1;
  const int q = (R > 32 ? 32 * sel : 0) + c32;
  if (q >= R) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int p = tile.y + 32 * rh + acc_row(i, h);
    if (p >= tile.z) continue;
    parts[slot * part_stride + static_cast<int64_t>(p) * R + q] = acc[i];
  }
}

// Workgroup (tile, split): one K range of kwg_steps steps, written to the
// split's partial slots (every split owns at least one step, so every slot of
// every LoRA row is written).  Summing the slots in order beats relaxed fp32
// atomics into Z here, and is deterministic.
template <int R, bool GATHER, bool KN>
__global__ void __launch_bounds__(kLoraThreads)
k_shrink_dma(const bf16_t* __restrict__ X, int x_rows, const int32_t* __restrict__ gather_slots,
             int gather_k, const bf16_t* __restrict__ At, int E, int L, int nad, int64_t K, int kwg_steps,
             int nsplit, const int4* __restrict__ ltiles, const int32_t* __restrict__ counts,
             float* __restrict__ parts, int64_t part_stride) {
  typedef ShrinkDma<R> S;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kShrinkStages * S::STAGE];
  const int lt = blockIdx.x / nsplit;
  const int split = blockIdx.x % nsplit;
  if (lt >= counts[1]) return;
  const int4 tile = ltiles[lt];
  if (tile.x % L >= nad) return;  // base-only bucket: no LoRA term
  const int nk_all = static_cast<int>(K / 64);
  const int kt0 = split * kwg_steps;
  const int nk = min(nk_all, kt0 + kwg_steps) - kt0;
  if (nk <= 0) return;  // uniform
  f32x16_t acc = zero_acc();
  shrink_dma_range<R, GATHER, KN>(smem, X, x_rows, gather_slots, gather_k, At, E, L, K, tile, kt0, nk,
                                  acc);
  shrink_dma_emit<R>(acc, tile, parts, part_stride, R > 32 ? split : 2 * split + (threadIdx.x / kWave >> 1));
}

// ------------------------------------------------------------ streaming shrink
// LoRA tiles of at most 16 rows and many of them (large decode batches over
// many adapters): the adapter weights are nearly all of the bytes and each is
// used by a handful of rows, so the kernel is a weight stream.  The work is a
// flat list of items (LoRA tile, K chunk), tile-major; an item is 8 or 16
// MFMA fragments of A^T (R rows x KC columns) and the tile's activation rows
// over the same chunk.  Each wave of a persistent grid takes one contiguous
// run of items, so it walks along the rows of one A^T block after another
// (sequential DRAM pages), sums a tile's chunks in registers and adds them to
// Z with relaxed fp32 atomics only when its run leaves the tile (once or twice
// per tile and wave instead of once per chunk).  The next item is loaded while
// the current one is multiplied.  Every item is whole (the chunk width
// divides K), so the loop is straight-line code and the compiler's in-order
// vmcnt waits leave the prefetched item in flight.  Deterministic mode writes
// every item's partial to its own slot (parts[kc]) instead of using atomics.
template <int R> struct ShrinkStream {
  static constexpr int RB = R / 16;               // 16-row blocks of A^T
  static constexpr int ST = R == 64 ? 4 : 8;      // MFMA K steps per item (8 or 16 A^T fragments)
  // K steps per item for a given K: ST when its chunks divide K, else 2 (K is
  // a multiple of 64), so that every item is whole
  static int steps(int64_t K) { return (K / 32) % ST == 0 ? ST : 2; }
};
// persistent grid of the streaming shrink: two workgroups (eight waves) per CU
// of an MI355X, used when the host's bound of the item count gives every wave
// a run of at least four items
constexpr int kStreamWgs = 2 * 256;
constexpr int64_t kStreamMinItems = 4ll * kStreamWgs * kLoraWaves;

// Row of X read by lane c for the 16 sorted rows from m0 of a tile ending at
// row_end (clamped rows are computed but never stored).  m0 and row_end are
// wave-uniform, so the slot indices come from scalar loads.
template <bool GATHER>
__device__ __forceinline__ int64_t stream_x_row(const int32_t* __restrict__ gather_slots,
                                                int gather_k, int x_rows, int m0, int row_end,
                                                int c) {
  int v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = GATHER ? gather_slots[min(m0 + i, row_end - 1)] : m0 + i;
  int r = v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) r = c == i ? v[i] : r;
  if (GATHER) r /= gather_k;
  else r = min(r, row_end - 1);
  return min(max(r, 0), x_rows - 1);
}

template <int R, int ST, bool GATHER, bool DET, bool KN>
__global__ void __launch_bounds__(kLoraThreads, 2)
k_shrink_stream(const bf16_t* __restrict__ X, int x_rows, const int32_t* __restrict__ gather_slots,
                int gather_k, const bf16_t* __restrict__ At, int E, int L, int nad, int64_t K,
                float* __restrict__ Z, const int4* __restrict__ ltiles,
                const int32_t* __restrict__ counts, float* __restrict__ parts,
                int64_t part_stride) {
  typedef Mfma16<bf16_t> M;
  typedef M::frag_t frag_t;
  constexpr int RB = R / 16, KC = ST * M::KSTEP;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c = lane & 15, g = lane >> 4;
  const int nwaves = gridDim.x * kLoraWaves;
  const int wid = blockIdx.x * kLoraWaves + wave;
  const int nkc = static_cast<int>(K / KC);  // K chunks (KC divides K)

  struct Work {
    int row0, row_end;
    const bf16_t* ab;   // A^T block of the bucket, nullptr for a base-only bucket
    const bf16_t* xp;   // lane's activation row
  };
  auto describe = [&](int tl) {
    const int4 t = ltiles[tl];
    const int e = t.x / L, l = t.x % L;
    const int row_end = min(t.z, t.y + 16);
    const bf16_t* xr = X + stream_x_row<GATHER>(gather_slots, gather_k, x_rows, t.y, row_end, c) * K;
    return Work{t.y, row_end, l < nad ? At + (static_cast<int64_t>(l) * E + e) * R * K : nullptr, xr};
  };
  f32x4_t acc[RB];
  auto clear = [&]() {
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  // deterministic: the partial of K chunk kc into its own slot
  auto flush = [&](const Work& w, int kc) {
    const int p = w.row0 + c;
    if (w.ab != nullptr && p < w.row_end) {
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t idx = static_cast<int64_t>(p) * R + 16 * j + 4 * g + i;
          if (DET)
            parts[kc * part_stride + idx] = acc[j][i];
          else
            atomic_add_relaxed(Z + idx, acc[j][i]);
        }
    }
    clear();
  };
  // A base-only bucket's items read the A^T block of adapter 0 (in bounds;
  // their sum is never stored).
  auto load = [&](frag_t (&af)[ST][RB], frag_t (&xf)[ST], const Work& w, int kc) {
    const bf16_t* ab = w.ab != nullptr ? w.ab : At;
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      const int64_t k = static_cast<int64_t>(kc) * KC + s * M::KSTEP + g * M::KPACK;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        if (KN)
          af[s][j] = KnFrag<bf16_t>::load(ab, R, 16 * j, static_cast<int64_t>(kc) * KC + s * M::KSTEP,
                                          true);
        else
          af[s][j] = M::load(ab + static_cast<int64_t>(16 * j + c) * K + k);
      }
      xf[s] = M::load(w.xp + k);
    }
  };
  auto mma = [&](const frag_t (&af)[ST][RB], const frag_t (&xf)[ST]) {
#pragma unroll
    for (int s = 0; s < ST; ++s)
#pragma unroll
      for (int j = 0; j < RB; ++j) M::run(acc[j], af[s][j], xf[s]);
  };

  // this wave's contiguous run [i0, i1) of the item list, taken one tile at a
  // time: the chunks of a tile share its activation rows and A^T block, and
  // the pipelined inner loop has no stores (a store's registers would hold up
  // the next loads behind the waits of the one in-order counter)
  const int64_t n = static_cast<int64_t>(counts[1]) * nkc;
  const int64_t i0 = n * wid / nwaves, i1 = n * (wid + 1) / nwaves;
  clear();
  frag_t a0[ST][RB], x0[ST], a1[ST][RB], x1[ST];
  for (int64_t it = i0; it < i1;) {
    const int tl = static_cast<int>(it / nkc);
    const Work w = describe(tl);
    const int kc0 = static_cast<int>(it - static_cast<int64_t>(tl) * nkc);
    const int kc1 = static_cast<int>(min<int64_t>(nkc, kc0 + (i1 - it)));  // this run's chunks of the tile
    int kc = kc0;
    load(a0, x0, w, kc);
    for (;;) {
      // past the tile's last chunk the last one is loaded again (never used)
      load(a1, x1, w, min(kc + 1, kc1 - 1));
      __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads stay ahead of these MFMAs
      mma(a0, x0);
      if (DET) flush(w, kc);
      if (++kc >= kc1) break;
      load(a0, x0, w, min(kc + 1, kc1 - 1));
      __builtin_amdgcn_sched_barrier(0);
      mma(a1, x1);
      if (DET) flush(w, kc);
      if (++kc >= kc1) break;
    }
    if (!DET) flush(w, 0);
    it += kc1 - kc0;
  }
}

// --------------------------------------------------------------------- expand
// Each wave owns NB blocks of 16 output columns (and, for gate_up, the
// matching up columns I + n).  Its B^T fragments are loaded once and reused
// for every 16-row block of the tile.  The base values the epilogue adds to
// (G for gate_up, D for down) and the next block's z are loaded before the
// current block's MFMAs, so a wave never waits on two memory round trips in a
// row.
// GATE_UP: ACT[p][i] = SiLU(G[p][i] + z_p.B[i]) * (G[p][I+i] + z_p.B[I+i])
//          (ncols = I, B^T has 2I rows)
// down:    D[p][n] += z_p.B[n] (ncols = h)
// DB: double-buffer the row blocks (tiles of many rows); otherwise one block
// buffer, whose first fetch still overlaps the weight loads.
template <typename T, int R, int NB, bool GATE_UP, bool DB, bool KN>
__global__ void __launch_bounds__(kLoraThreads)
k_expand(const float* __restrict__ Z, const T* __restrict__ Bt, int E, int L, int nad,
         const float* __restrict__ G, T* __restrict__ ACT, float* __restrict__ D, int64_t ncols,
         const int4* __restrict__ ltiles, const int32_t* __restrict__ counts, int n_chunks) {
  typedef Mfma16<T> M;
  typedef typename M::frag_t frag_t;
  constexpr int KS = (R + M::KSTEP - 1) / M::KSTEP;
  constexpr int NH = GATE_UP ? 2 : 1;
  const int lt = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x % n_chunks;
  if (lt >= counts[1]) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int64_t c0 = (static_cast<int64_t>(chunk) * kLoraWaves + wave) * (16 * NB);
  if (c0 >= ncols) return;  // ncols is a multiple of 16: blocks are whole or absent
  const int4 tile = ltiles[lt];
  const int b = tile.x, row0 = tile.y, row_end = tile.z;
  const int e = b / L, l = b % L;
  // base-only bucket: no LoRA term; gate_up still produces ACT from G alone
  const bool lora = l < nad;
  if (!GATE_UP && !lora) return;

  const int64_t nfull = GATE_UP ? 2 * ncols : ncols;
  // (a base-only tile never loads B; its pointer still stays inside the array)
  const T* Bb = Bt + (static_cast<int64_t>(lora ? l : 0) * E + e) * nfull * R;
  bool nb_ok[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) nb_ok[j] = c0 + 16 * j < ncols;  // uniform per wave
  frag_t bf[NH][NB][KS];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int q = ks * M::KSTEP + g * M::KPACK;
        const int64_t n = hh * ncols + c0 + 16 * j + c;
        if (KN)  // B [R][nfull]: the rank is the k of the fragment
          bf[hh][j][ks] = KnFrag<T>::load(Bb, nfull, hh * ncols + c0 + 16 * j, ks * M::KSTEP,
                                          lora && q < R && nb_ok[j]);
        else
          bf[hh][j][ks] = (lora && q < R && nb_ok[j]) ? M::load(Bb + n * R + q) : M::zero();
      }

  // per 16-row block: z fragments and the four base values per column block
  struct Block {
    ZFrag<T> zf[KS];
    float4 base[NH][NB];
  };
  auto fetch = [&](Block& blk, int m0) {
    const int p = m0 + c;
    const bool ok = p < row_end;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int q = ks * M::KSTEP + g * M::KPACK;
      if (lora && ok && q < R)
        blk.zf[ks].load(Z + static_cast<int64_t>(p) * R + q);
      else
        blk.zf[ks].clear();
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int64_t n = hh * ncols + c0 + 16 * j + 4 * g;
        const float* src = GATE_UP ? G + static_cast<int64_t>(p) * nfull + n
                                   : D + static_cast<int64_t>(p) * ncols + n;
        blk.base[hh][j] = (ok && nb_ok[j]) ? *reinterpret_cast<const float4*>(src)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
      }
  };
  auto run = [&](const Block& blk, int m0) {
    f32x4_t acc[NH][NB];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        acc[hh][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) blk.zf[ks].mma(acc[hh][j], bf[hh][j][ks]);
      }
    const int p = m0 + c;
    if (p >= row_end) return;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (!nb_ok[j]) continue;
      const int64_t n = c0 + 16 * j + 4 * g;  // 4 consecutive output columns
      if (GATE_UP) {
        const float4 gg = blk.base[0][j], gu = blk.base[NH - 1][j];
        const float a0 = silu(gg.x + acc[0][j][0]) * (gu.x + acc[NH - 1][j][0]);
        const float a1 = silu(gg.y + acc[0][j][1]) * (gu.y + acc[NH - 1][j][1]);
        const float a2 = silu(gg.z + acc[0][j][2]) * (gu.z + acc[NH - 1][j][2]);
        const float a3 = silu(gg.w + acc[0][j][3]) * (gu.w + acc[NH - 1][j][3]);
        store4(ACT + static_cast<int64_t>(p) * ncols + n, a0, a1, a2, a3);
      } else {
        const float4 d = blk.base[0][j];
        *reinterpret_cast<float4*>(D + static_cast<int64_t>(p) * ncols + n) =
            make_float4(d.x + acc[0][j][0], d.y + acc[0][j][1], d.z + acc[0][j][2],
                        d.w + acc[0][j][3]);
      }
    }
  };

  if (DB) {
    Block cur, nxt;
    fetch(cur, row0);
    for (int m0 = row0; m0 < row_end; m0 += 32) {
      if (m0 + 16 < row_end) fetch(nxt, m0 + 16);
      run(cur, m0);
      if (m0 + 16 >= row_end) break;
      if (m0 + 32 < row_end) fetch(cur, m0 + 32);
      run(nxt, m0 + 16);
    }
  } else {
    Block blk;
    for (int m0 = row0; m0 < row_end; m0 += 16) {
      fetch(blk, m0);
      run(blk, m0);
    }
  }
}

// -------------------------------------------------------------------- combine
// D: nparts planes of [S][h] (pstride floats apart) whose sum, in plane order,
// is the down projection's output per slot (one plane unless its K range was
// split over workgroups that stored their partials).
template <typename T>
__global__ void __launch_bounds__(256)
k_combine(const float* __restrict__ D, int nparts, int64_t pstride, const int32_t* __restrict__ pos,
          const float* __restrict__ w, int k, int S, int64_t h, T* __restrict__ out) {
  const int t = blockIdx.x;
  const int64_t c = (static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x) * 4;
  if (c >= h) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int p = min(max(pos[t * k + j], 0), S - 1);
    const float wj = w != nullptr ? w[t * k + j] : 1.0f;
    const float* src = D + static_cast<int64_t>(p) * h + c;
    float4 d = *reinterpret_cast<const float4*>(src);
    // planes in order, four loads in flight at a time
    auto add = [&](const float4& v) {
      d.x += v.x;
      d.y += v.y;
      d.z += v.z;
      d.w += v.w;
    };
    int s = 1;
    for (; s + 3 < nparts; s += 4) {
      float4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const float4*>(src + (s + i) * pstride);
#pragma unroll
      for (int i = 0; i < 4; ++i) add(v[i]);
    }
    for (; s < nparts; ++s) add(*reinterpret_cast<const float4*>(src + s * pstride));
    acc.x += wj * d.x;
    acc.y += wj * d.y;
    acc.z += wj * d.z;
    acc.w += wj * d.w;
  }
  store4(out + static_cast<int64_t>(t) * h + c, acc.x, acc.y, acc.z, acc.w);
}

// -------------------------------------------------------------------- launchers
// 16-column blocks per wave: gate_up carries gate and up halves, so 4 blocks
// (64 + 64 columns); down takes 8 blocks for r <= 32
template <int R, bool GU> constexpr int expand_nb() { return (GU || R > 32) ? 4 : 8; }

// Split counts of the three shrink forms (shared by the launch and the host's
// count of deterministic partials).
struct ShrinkSplit {
  int nsplit, kwg_steps, parts;  // parts = partial slices in deterministic mode
  int64_t kwg;                   // K range per split (k_shrink_tall)
  bool stream;                   // k_shrink_stream (nsplit = K chunks per tile)
};

template <typename T, int R>
static ShrinkSplit shrink_split(const TilePlan& plan, int64_t K) {
  ShrinkSplit sp{1, 0, 1, K, false};
  const int64_t nkc = K / (32 * ShrinkStream<R>::steps(K));
  if (!plan.lora_db && sizeof(T) == 2 && plan.bml == 16 &&
      static_cast<int64_t>(plan.max_lt) * nkc >= kStreamMinItems) {
    // k_shrink_stream: one partial per K chunk
    sp.stream = true;
    sp.nsplit = sp.parts = static_cast<int>(nkc);
  } else if (plan.lora_db && sizeof(T) == 2) {  // k_shrink_dma
    const int nk_all = static_cast<int>(K / 64);
    int nsplit = (1024 + plan.max_lt - 1) / std::max(1, plan.max_lt);
    nsplit = std::max(1, std::min(nsplit, nk_all / 4));
    sp.kwg_steps = (nk_all + nsplit - 1) / nsplit;
    sp.nsplit = (nk_all + sp.kwg_steps - 1) / sp.kwg_steps;
    sp.parts = R > 32 ? sp.nsplit : 2 * sp.nsplit;
  } else if (plan.lora_db) {             // k_shrink_tall
    constexpr int STEPS = R > 32 ? 2 : 4;
    constexpr int64_t KB = STEPS * Mfma16<T>::KSTEP;
    int64_t nsplit = 1024 / std::max(1, plan.max_lt);
    nsplit = std::max<int64_t>(1, std::min<int64_t>(nsplit, K / (4 * KB)));
    int64_t kwg = (K + nsplit - 1) / nsplit;
    kwg = (kwg + KB - 1) / KB * KB;
    sp.kwg = kwg;
    sp.nsplit = sp.parts = static_cast<int>((K + kwg - 1) / kwg);
  } else {                               // k_shrink
    constexpr int STEPS = R <= 32 ? 8 : 4;
    constexpr int KW = STEPS * Mfma16<T>::KSTEP;
    sp.nsplit = sp.parts = static_cast<int>((K + kLoraWaves * KW - 1) / (kLoraWaves * KW));
  }
  return sp;
}

template <typename T, int R, bool GATHER, bool KN>
static hipError_t shrink_launch(const TilePlan& plan, const void* X, int x_rows,
                                const int32_t* gather_slots, int gather_k, const void* At, int E,
                                int L, int64_t K, float* Z, int S, const int4* ltiles,
                                const int32_t* counts, float* parts, hipStream_t stream) {
  const ShrinkSplit sp = shrink_split<T, R>(plan, K);
  const int64_t stride = static_cast<int64_t>(S) * R;
  const int64_t grid = static_cast<int64_t>(plan.max_lt) * sp.nsplit;
  if (plan.lora_db && sizeof(T) == 2 && parts == nullptr)
    return hipErrorInvalidValue;  // tall bf16 tiles always sum partials (plan.shrink_partials)
  if (sp.stream) {
    // many short tiles: persistent waves stream runs of (tile, K chunk) items
    constexpr int ST = ShrinkStream<R>::ST;
    const bool det = parts != nullptr;
    auto kern = ShrinkStream<R>::steps(K) == ST
                    ? (det ? k_shrink_stream<R, ST, GATHER, true, KN> : k_shrink_stream<R, ST, GATHER, false, KN>)
                    : (det ? k_shrink_stream<R, 2, GATHER, true, KN> : k_shrink_stream<R, 2, GATHER, false, KN>);
    hipLaunchKernelGGL(kern, dim3(kStreamWgs), dim3(kLoraThreads), 0, stream,
                       static_cast<const bf16_t*>(X), x_rows, gather_slots, gather_k,
                       static_cast<const bf16_t*>(At), E, L, plan.nad, K, Z, ltiles, counts,
                       parts, stride);
  } else if (plan.lora_db && sizeof(T) == 2) {
    // tall bf16 tiles: DMA ring, about 1024 workgroups of (tile, K range), partial slots
    hipLaunchKernelGGL((k_shrink_dma<R, GATHER, KN>), dim3(static_cast<unsigned>(grid)),
                       dim3(kLoraThreads), 0, stream, static_cast<const bf16_t*>(X), x_rows,
                       gather_slots, gather_k, static_cast<const bf16_t*>(At), E, L, plan.nad, K,
                       sp.kwg_steps, sp.nsplit, ltiles, counts, parts, stride);
  } else if (plan.lora_db) {
    // tall tiles: ~1024 workgroups, each wave a 16-row block over the split's K range
    constexpr int STEPS = R > 32 ? 2 : 4;
    hipLaunchKernelGGL((k_shrink_tall<T, R, STEPS, GATHER, KN>), dim3(static_cast<unsigned>(grid)),
                       dim3(kLoraThreads), 0, stream, static_cast<const T*>(X), x_rows,
                       gather_slots, gather_k, static_cast<const T*>(At), E, L, plan.nad, K, sp.kwg,
                       sp.nsplit, Z, ltiles, counts, parts, stride);
  } else {
    constexpr int STEPS = R <= 32 ? 8 : 4;
    hipLaunchKernelGGL((k_shrink<T, R, STEPS, GATHER, KN>), dim3(static_cast<unsigned>(grid)),
                       dim3(kLoraThreads), 0, stream, static_cast<const T*>(X), x_rows, gather_slots,
                       gather_k, static_cast<const T*>(At), E, L, plan.nad, K, sp.nsplit, Z, ltiles,
                       counts, parts, stride);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && parts != nullptr) e = launch_reduce_parts(parts, sp.parts, stride, Z, stream);
  return e;
}

template <typename T, bool GATHER, bool KN>
static hipError_t shrink_dispatch_kn(int rank, const TilePlan& plan, const void* X, int x_rows,
                                     const int32_t* gather_slots, int gather_k, const void* At, int E,
                                     int L, int64_t K, float* Z, int S, const int4* ltiles,
                                     const int32_t* counts, float* parts, hipStream_t stream) {
  switch (rank) {
    case 16: return shrink_launch<T, 16, GATHER, KN>(plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, S, ltiles, counts, parts, stream);
    case 32: return shrink_launch<T, 32, GATHER, KN>(plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, S, ltiles, counts, parts, stream);
    case 64: return shrink_launch<T, 64, GATHER, KN>(plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, S, ltiles, counts, parts, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool GATHER>
static hipError_t shrink_dispatch(int rank, const TilePlan& plan, const void* X, int x_rows,
                                  const int32_t* gather_slots, int gather_k, const void* At, int E,
                                  int L, int64_t K, float* Z, int S, const int4* ltiles,
                                  const int32_t* counts, float* parts, hipStream_t stream) {
  return plan.kn ? shrink_dispatch_kn<T, GATHER, true>(rank, plan, X, x_rows, gather_slots, gather_k, At,
                                                       E, L, K, Z, S, ltiles, counts, parts, stream)
                 : shrink_dispatch_kn<T, GATHER, false>(rank, plan, X, x_rows, gather_slots, gather_k,
                                                        At, E, L, K, Z, S, ltiles, counts, parts, stream);
}

hipError_t launch_shrink(int dtype, int rank, const TilePlan& plan, const void* X, int x_rows,
                         const int32_t* gather_slots, int gather_k, const void* At, int E, int L,
                         int64_t K, float* Z, int S, const int4* ltiles, const int32_t* counts,
                         float* parts, hipStream_t stream) {
  const bool gather = gather_slots != nullptr;
  if (dtype == DT_BF16)
    return gather ? shrink_dispatch<bf16_t, true>(rank, plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, S, ltiles, counts, parts, stream)
                  : shrink_dispatch<bf16_t, false>(rank, plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, S, ltiles, counts, parts, stream);
  return gather ? shrink_dispatch<float, true>(rank, plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, S, ltiles, counts, parts, stream)
                : shrink_dispatch<float, false>(rank, plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, S, ltiles, counts, parts, stream);
}

int shrink_parts(int dtype, int rank, const TilePlan& plan, int64_t K) {
  auto pick = [&](auto tag) {
    typedef decltype(tag) T;
    switch (rank) {
      case 16: return shrink_split<T, 16>(plan, K).parts;
      case 32: return shrink_split<T, 32>(plan, K).parts;
      default: return shrink_split<T, 64>(plan, K).parts;
    }
  };
  return dtype == DT_BF16 ? pick(bf16_t{}) : pick(float{});
}

template <typename T, int R, bool GU>
static hipError_t expand_launch(const TilePlan& plan, const float* Z, const void* Bt, int E, int L,
                                const float* G, void* ACT, float* D, int64_t ncols,
                                const int4* ltiles, const int32_t* counts, hipStream_t stream) {
  constexpr int NB = expand_nb<R, GU>();
  constexpr int COLS = kLoraWaves * 16 * NB;
  const int n_chunks = static_cast<int>((ncols + COLS - 1) / COLS);
  const int64_t grid = static_cast<int64_t>(plan.max_lt) * n_chunks;
  auto kern = plan.lora_db ? (plan.kn ? k_expand<T, R, NB, GU, true, true> : k_expand<T, R, NB, GU, true, false>)
                           : (plan.kn ? k_expand<T, R, NB, GU, false, true> : k_expand<T, R, NB, GU, false, false>);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kLoraThreads), 0, stream, Z,
                     static_cast<const T*>(Bt), E, L, plan.nad, G, static_cast<T*>(ACT), D, ncols,
                     ltiles, counts, n_chunks);
  return hipGetLastError();
}

template <typename T, bool GU>
static hipError_t expand_dispatch(int rank, const TilePlan& plan, const float* Z, const void* Bt,
                                  int E, int L, const float* G, void* ACT, float* D, int64_t ncols,
                                  const int4* ltiles, const int32_t* counts, hipStream_t stream) {
  switch (rank) {
    case 16: return expand_launch<T, 16, GU>(plan, Z, Bt, E, L, G, ACT, D, ncols, ltiles, counts, stream);
    case 32: return expand_launch<T, 32, GU>(plan, Z, Bt, E, L, G, ACT, D, ncols, ltiles, counts, stream);
    case 64: return expand_launch<T, 64, GU>(plan, Z, Bt, E, L, G, ACT, D, ncols, ltiles, counts, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_expand_gate_up(int dtype, int rank, const TilePlan& plan, const float* Z,
                                 const void* Bt, int E, int L, const float* G, void* ACT,
                                 int64_t I, const int4* ltiles, const int32_t* counts,
                                 hipStream_t stream) {
  if (dtype == DT_BF16)
    return expand_dispatch<bf16_t, true>(rank, plan, Z, Bt, E, L, G, ACT, nullptr, I, ltiles,
                                         counts, stream);
  return expand_dispatch<float, true>(rank, plan, Z, Bt, E, L, G, ACT, nullptr, I, ltiles, counts,
                                      stream);
}

hipError_t launch_expand_down(int dtype, int rank, const TilePlan& plan, const float* Z,
                              const void* Bt, int E, int L, float* D, int64_t h,
                              const int4* ltiles, const int32_t* counts, hipStream_t stream) {
  if (dtype == DT_BF16)
    return expand_dispatch<bf16_t, false>(rank, plan, Z, Bt, E, L, nullptr, nullptr, D, h, ltiles,
                                          counts, stream);
  return expand_dispatch<float, false>(rank, plan, Z, Bt, E, L, nullptr, nullptr, D, h, ltiles,
                                       counts, stream);
}

hipError_t launch_combine(int dtype, const float* D, const int32_t* pos, const float* w, int T,
                          int k, int64_t h, void* out, hipStream_t stream, int nparts) {
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>((h + 1023) / 1024));
  const int64_t pstride = static_cast<int64_t>(T) * k * h;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL((k_combine<bf16_t>), grid, dim3(256), 0, stream, D, nparts, pstride, pos, w,
                       k, T * k, h, static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL((k_combine<float>), grid, dim3(256), 0, stream, D, nparts, pstride, pos, w,
                       k, T * k, h, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace moelora
