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
// Work unit of every kernel: a LoRA tile = up to 64 consecutive sorted rows of
// one (expert, adapter) bucket.  Products run on MFMA 32x32 blocks; the rank r
// (16/32/64) is the N of the shrink and the K of the expand.
#include "device_common.h"
#include "launch.h"

namespace moelora {

constexpr int kLoraThreads = 256;
constexpr int kLoraRows = 64;          // rows per LoRA tile (two 32-row MFMA blocks)
constexpr int kLoraFM = kLoraRows / 32;
constexpr int kExpandCols = 128;       // output columns per expand workgroup (32 per wave)

// --------------------------------------------------------------------- shrink
// Workgroup (tile, split): K range [split*kc, split*kc + kc) cut into four
// wave ranges; every wave accumulates its partial z block in MFMA registers,
// the four partials are summed through LDS and the sum is added to Z with one
// relaxed atomic per element.
template <typename T, int R>
__global__ void __launch_bounds__(kLoraThreads)
k_shrink(const T* __restrict__ X, int x_rows, const int32_t* __restrict__ gather_slots, int gather_k,
         const T* __restrict__ At, int E, int L, int64_t K, int kc, int nsplit,
         float* __restrict__ Z, const int4* __restrict__ ltiles, const int32_t* __restrict__ counts) {
  typedef Mfma<T> M;
  constexpr int FQ = (R + 31) / 32;
  __shared__ float red[4][16 * kWave];

  const int lt = blockIdx.x / nsplit;
  const int split = blockIdx.x % nsplit;
  if (lt >= counts[1]) return;
  const int4 tile = ltiles[lt];
  const int b = tile.x, row0 = tile.y, row_end = tile.z;
  const int e = b / L, l = b % L;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c32 = lane & 31, h = lane >> 5;

  const int64_t kb = static_cast<int64_t>(split) * kc;
  const int64_t ke = kb + kc < K ? kb + kc : K;
  const int wlen = kc / 4;
  const int64_t kw0 = kb + static_cast<int64_t>(wave) * wlen;
  const int64_t kw1 = kw0 + wlen < ke ? kw0 + wlen : ke;

  const T* xrow[kLoraFM];
#pragma unroll
  for (int i = 0; i < kLoraFM; ++i) {
    const int p = row0 + i * 32 + c32;
    xrow[i] = nullptr;
    if (p < row_end) {
      const int r = gather_slots ? gather_slots[p] / gather_k : p;
      xrow[i] = X + static_cast<int64_t>(min(max(r, 0), x_rows - 1)) * K + h * M::KPACK;
    }
  }
  const T* Ab = At + (static_cast<int64_t>(l) * E + e) * R * K;
  const T* arow[FQ];
#pragma unroll
  for (int j = 0; j < FQ; ++j) {
    const int q = j * 32 + c32;
    arow[j] = q < R ? Ab + static_cast<int64_t>(q) * K + h * M::KPACK : nullptr;
  }

  f32x16_t acc[kLoraFM][FQ];
#pragma unroll
  for (int i = 0; i < kLoraFM; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j) acc[i][j] = zero_acc();

  const int nsteps = kw1 > kw0 ? static_cast<int>((kw1 - kw0) / M::KSTEP) : 0;

  for (int s = 0; s < nsteps; ++s) {
    const int64_t k = kw0 + static_cast<int64_t>(s) * M::KSTEP;
    typename M::frag_t af[kLoraFM], bfr[FQ];
#pragma unroll
    for (int i = 0; i < kLoraFM; ++i) af[i] = xrow[i] ? M::load(xrow[i] + k) : M::zero();
#pragma unroll
    for (int j = 0; j < FQ; ++j) bfr[j] = arow[j] ? M::load(arow[j] + k) : M::zero();
#pragma unroll
    for (int i = 0; i < kLoraFM; ++i)
#pragma unroll
      for (int j = 0; j < FQ; ++j) M::run(acc[i][j], af[i], bfr[j]);
  }

  // sum the four wave partials block by block, then one atomic per element
#pragma unroll
  for (int i = 0; i < kLoraFM; ++i) {
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      if (row0 + i * 32 >= row_end) continue;  // uniform across the workgroup
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave][r * kWave + lane] = acc[i][j][r];
      __syncthreads();
      for (int idx = tid; idx < 16 * kWave; idx += kLoraThreads) {
        const float v = red[0][idx] + red[1][idx] + red[2][idx] + red[3][idx];
        const int r = idx / kWave, ln = idx % kWave;
        const int p = row0 + i * 32 + acc_row(r, ln >> 5);
        const int q = j * 32 + (ln & 31);
        if (p < row_end && q < R) atomic_add_relaxed(Z + static_cast<int64_t>(p) * R + q, v);
      }
      __syncthreads();
    }
  }
}

// --------------------------------------------------------------------- expand
// Loads the 8 (bf16) or 1 (fp32) z values of a lane's A fragment.  bf16 MFMA
// inputs get z split into a high and a low bf16 part so that z keeps about 16
// significant bits; the fp32 path uses z as it is.
template <typename T> struct ZFrag;
template <> struct ZFrag<bf16_t> {
  bf16x8_t hi, lo;
  __device__ __forceinline__ void load(const float* z) {
    const float4 a = *reinterpret_cast<const float4*>(z);
    const float4 b = *reinterpret_cast<const float4*>(z + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint16_t hb[8], lb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hb[i] = f32_to_bf16(v[i]);
      lb[i] = f32_to_bf16(v[i] - bf16_to_f32(hb[i]));
    }
    uint4 hu = make_uint4(hb[0] | (uint32_t(hb[1]) << 16), hb[2] | (uint32_t(hb[3]) << 16),
                          hb[4] | (uint32_t(hb[5]) << 16), hb[6] | (uint32_t(hb[7]) << 16));
    uint4 lu = make_uint4(lb[0] | (uint32_t(lb[1]) << 16), lb[2] | (uint32_t(lb[3]) << 16),
                          lb[4] | (uint32_t(lb[5]) << 16), lb[6] | (uint32_t(lb[7]) << 16));
    hi = __builtin_bit_cast(bf16x8_t, hu);
    lo = __builtin_bit_cast(bf16x8_t, lu);
  }
  __device__ __forceinline__ void clear() { hi = Mfma<bf16_t>::zero(); lo = hi; }
  __device__ __forceinline__ void mma(f32x16_t& acc, bf16x8_t b) const {
    Mfma<bf16_t>::run(acc, hi, b);
    Mfma<bf16_t>::run(acc, lo, b);
  }
};
template <> struct ZFrag<float> {
  float v;
  __device__ __forceinline__ void load(const float* z) { v = *z; }
  __device__ __forceinline__ void clear() { v = 0.0f; }
  __device__ __forceinline__ void mma(f32x16_t& acc, float b) const { Mfma<float>::run(acc, v, b); }
};

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// GATE_UP: ACT[p][i] = SiLU(G[p][i] + z_p.B[i]) * (G[p][I+i] + z_p.B[I+i]) for
//          the 32 columns i of each wave (ncols = I, B has 2I rows).
// down:    D[p][n] += z_p.B[n] (ncols = h).
template <typename T, int R, bool GATE_UP>
__global__ void __launch_bounds__(kLoraThreads)
k_expand(const float* __restrict__ Z, const T* __restrict__ Bt, int E, int L,
         const float* __restrict__ G, T* __restrict__ ACT, float* __restrict__ D, int64_t ncols,
         const int4* __restrict__ ltiles, const int32_t* __restrict__ counts, int n_chunks) {
  typedef Mfma<T> M;
  const int lt = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x % n_chunks;
  if (lt >= counts[1]) return;
  const int4 tile = ltiles[lt];
  const int b = tile.x, row0 = tile.y, row_end = tile.z;
  const int e = b / L, l = b % L;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c32 = lane & 31, h = lane >> 5;
  const int64_t c0 = static_cast<int64_t>(chunk) * kExpandCols + wave * 32;
  if (c0 >= ncols) return;  // ncols is a multiple of 32: whole waves drop out
  const int64_t col = c0 + c32;

  const int64_t nfull = GATE_UP ? 2 * ncols : ncols;
  const T* Bb = Bt + (static_cast<int64_t>(l) * E + e) * nfull * R;
  const T* bg = Bb + col * R + h * M::KPACK;
  const T* bu = GATE_UP ? Bb + (ncols + col) * R + h * M::KPACK : nullptr;

  f32x16_t acc_g[kLoraFM], acc_u[kLoraFM];
#pragma unroll
  for (int i = 0; i < kLoraFM; ++i) {
    acc_g[i] = zero_acc();
    acc_u[i] = zero_acc();
  }
#pragma unroll
  for (int ks = 0; ks < R / M::KSTEP; ++ks) {
    const int ko = ks * M::KSTEP;
    const typename M::frag_t fg = M::load(bg + ko);
    typename M::frag_t fu = M::zero();
    if (GATE_UP) fu = M::load(bu + ko);
#pragma unroll
    for (int i = 0; i < kLoraFM; ++i) {
      if (row0 + i * 32 >= row_end) continue;  // uniform
      const int p = row0 + i * 32 + c32;
      ZFrag<T> zf;
      if (p < row_end)
        zf.load(Z + static_cast<int64_t>(p) * R + ko + h * M::KPACK);
      else
        zf.clear();
      zf.mma(acc_g[i], fg);
      if (GATE_UP) zf.mma(acc_u[i], fu);
    }
  }

#pragma unroll
  for (int i = 0; i < kLoraFM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = row0 + i * 32 + acc_row(r, h);
      if (p >= row_end) continue;
      if (GATE_UP) {
        const float* gr = G + static_cast<int64_t>(p) * nfull;
        const float g = gr[col] + acc_g[i][r];
        const float u = gr[ncols + col] + acc_u[i][r];
        ACT[static_cast<int64_t>(p) * ncols + col] = from_f32<T>(silu(g) * u);
      } else {
        float* dr = D + static_cast<int64_t>(p) * ncols + col;
        *dr = *dr + acc_g[i][r];
      }
    }
  }
}

// -------------------------------------------------------------------- combine
template <typename T>
__global__ void __launch_bounds__(256)
k_combine(const float* __restrict__ D, const int32_t* __restrict__ pos, const float* __restrict__ w,
          int k, int S, int64_t h, T* __restrict__ out) {
  const int t = blockIdx.x;
  const int64_t c = (static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x) * 4;
  if (c >= h) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int p = min(max(pos[t * k + j], 0), S - 1);
    const float wj = w[t * k + j];
    const float4 d = *reinterpret_cast<const float4*>(D + static_cast<int64_t>(p) * h + c);
    acc.x += wj * d.x;
    acc.y += wj * d.y;
    acc.z += wj * d.z;
    acc.w += wj * d.w;
  }
  T* o = out + static_cast<int64_t>(t) * h + c;
  o[0] = from_f32<T>(acc.x);
  o[1] = from_f32<T>(acc.y);
  o[2] = from_f32<T>(acc.z);
  o[3] = from_f32<T>(acc.w);
}

// -------------------------------------------------------------------- launchers
static int shrink_splits(const TilePlan& plan, int64_t K, int* kc_out) {
  // aim at ~2048 workgroups, at least 64 K-elements per split, kc a multiple of 64
  int64_t nsplit = 2048 / (plan.max_lt > 0 ? plan.max_lt : 1);
  const int64_t maxsplit = K / 64;
  if (nsplit > maxsplit) nsplit = maxsplit;
  if (nsplit < 1) nsplit = 1;
  int64_t kc = (K + nsplit - 1) / nsplit;
  kc = (kc + 63) / 64 * 64;
  *kc_out = static_cast<int>(kc);
  return static_cast<int>((K + kc - 1) / kc);
}

template <typename T, int R>
static hipError_t shrink_launch(const TilePlan& plan, const void* X, int x_rows, const int32_t* gather_slots,
                                int gather_k, const void* At, int E, int L, int64_t K, float* Z,
                                const int4* ltiles, const int32_t* counts, hipStream_t stream) {
  int kc = 0;
  const int nsplit = shrink_splits(plan, K, &kc);
  const int64_t grid = static_cast<int64_t>(plan.max_lt) * nsplit;
  hipLaunchKernelGGL((k_shrink<T, R>), dim3(static_cast<unsigned>(grid)), dim3(kLoraThreads), 0,
                     stream, static_cast<const T*>(X), x_rows, gather_slots, gather_k,
                     static_cast<const T*>(At), E, L, K, kc, nsplit, Z, ltiles, counts);
  return hipGetLastError();
}

template <typename T>
static hipError_t shrink_dispatch(int rank, const TilePlan& plan, const void* X, int x_rows,
                                  const int32_t* gather_slots, int gather_k, const void* At, int E,
                                  int L, int64_t K, float* Z, const int4* ltiles,
                                  const int32_t* counts, hipStream_t stream) {
  switch (rank) {
    case 16: return shrink_launch<T, 16>(plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, ltiles, counts, stream);
    case 32: return shrink_launch<T, 32>(plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, ltiles, counts, stream);
    case 64: return shrink_launch<T, 64>(plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, ltiles, counts, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shrink(int dtype, int rank, const TilePlan& plan, const void* X, int x_rows,
                         const int32_t* gather_slots, int gather_k, const void* At, int E, int L,
                         int64_t K, float* Z, const int4* ltiles, const int32_t* counts,
                         hipStream_t stream) {
  if (plan.bml != kLoraRows) return hipErrorInvalidValue;
  if (dtype == DT_BF16)
    return shrink_dispatch<bf16_t>(rank, plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, ltiles,
                                   counts, stream);
  return shrink_dispatch<float>(rank, plan, X, x_rows, gather_slots, gather_k, At, E, L, K, Z, ltiles,
                                counts, stream);
}

template <typename T, int R, bool GU>
static hipError_t expand_launch(const TilePlan& plan, const float* Z, const void* Bt, int E, int L,
                                const float* G, void* ACT, float* D, int64_t ncols,
                                const int4* ltiles, const int32_t* counts, hipStream_t stream) {
  const int n_chunks = static_cast<int>((ncols + kExpandCols - 1) / kExpandCols);
  const int64_t grid = static_cast<int64_t>(plan.max_lt) * n_chunks;
  hipLaunchKernelGGL((k_expand<T, R, GU>), dim3(static_cast<unsigned>(grid)), dim3(kLoraThreads),
                     0, stream, Z, static_cast<const T*>(Bt), E, L, G, static_cast<T*>(ACT), D,
                     ncols, ltiles, counts, n_chunks);
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
  if (plan.bml != kLoraRows) return hipErrorInvalidValue;
  if (dtype == DT_BF16)
    return expand_dispatch<bf16_t, true>(rank, plan, Z, Bt, E, L, G, ACT, nullptr, I, ltiles,
                                         counts, stream);
  return expand_dispatch<float, true>(rank, plan, Z, Bt, E, L, G, ACT, nullptr, I, ltiles, counts,
                                      stream);
}

hipError_t launch_expand_down(int dtype, int rank, const TilePlan& plan, const float* Z,
                              const void* Bt, int E, int L, float* D, int64_t h,
                              const int4* ltiles, const int32_t* counts, hipStream_t stream) {
  if (plan.bml != kLoraRows) return hipErrorInvalidValue;
  if (dtype == DT_BF16)
    return expand_dispatch<bf16_t, false>(rank, plan, Z, Bt, E, L, nullptr, nullptr, D, h, ltiles,
                                          counts, stream);
  return expand_dispatch<float, false>(rank, plan, Z, Bt, E, L, nullptr, nullptr, D, h, ltiles,
                                       counts, stream);
}

hipError_t launch_combine(int dtype, const float* D, const int32_t* pos, const float* w, int T,
                          int k, int64_t h, void* out, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>((h + 1023) / 1024));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL((k_combine<bf16_t>), grid, dim3(256), 0, stream, D, pos, w, k, T * k, h,
                       static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL((k_combine<float>), grid, dim3(256), 0, stream, D, pos, w, k, T * k, h,
                       static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace moelora
