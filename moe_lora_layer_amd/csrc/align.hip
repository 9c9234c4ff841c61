// Routing and the (expert, adapter)-bucketed slot permutation, one workgroup.
//
// Follows the vLLM blog page "Multi-LoRA" (vllm.com.cn/blog/multi-lora),
// section "Implementing Multi-LoRA inference for MoE models in vLLM": each
// token goes to its most relevant experts, and expert routing compounds with
// the per-request adapter choice, so slots are grouped by (expert, adapter).
//
// One workgroup of 1024 threads runs four phases separated by barriers:
//   1. route: per token, a k-deep insertion list over the E logits (ties keep
//      the lower id), softmax weights renormalised over the kept k; the slot
//      keys e*L + l go to the workspace;
//   2. chunk ranks: the S slots are cut into C contiguous chunks, one per wave.
//      A wave walks its chunk 64 slots at a time; lanes with equal keys find
//      each other with ballots, so every slot gets its rank among equal keys of
//      lower index inside the chunk, and the chunk's per-bucket counts live in
//      LDS (cnt[c][b]); keys and ranks stay in LDS too when the batch is small;
//   3. scan: bucket totals, a wavefront-level exclusive prefix scan over the
//      buckets gives bucket_offsets, and cnt[c][b] becomes the first output
//      position of chunk c's slots in bucket b;
//   4. scatter: sorted_slots[cnt[c][key] + rank] = s.
// ROUTE = false skips the routing of phase 1: the caller's topk_ids (its own
// router, e.g. a router GEMM and top-k just before this path) give the keys.
// device_status: 0 ok, 1 an adapter id outside [0, L), 2 internal
// inconsistency, 3 a given expert id outside [0, E) (the largest code wins).
// No step depends on atomic ordering, so the result is bit-exact and stable.
#include "device_common.h"
#include "launch.h"

namespace moelora {

constexpr int kAlignThreads = 1024;
constexpr int kMaxTopK = 8;

// KEYS_LDS: the per-slot keys and ranks live in LDS after the counters (small
// batches); otherwise in the workspace.
// KMAX: the routing list length compiled in, the smallest of 1, 2, 4, 8 that
// holds k (a longer list only adds compare-and-select steps).
template <bool KEYS_LDS, bool ROUTE, int KMAX>
__global__ void __launch_bounds__(kAlignThreads)
k_align(const float* __restrict__ logits, const int32_t* __restrict__ ids_in,
        const int32_t* __restrict__ adapter_ids, int T, int E,
        int k, int L, int Lb, int chunks, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
        int32_t* __restrict__ sorted_slots, int32_t* __restrict__ offsets,
        int32_t* __restrict__ status, int32_t* __restrict__ ws_key, int32_t* __restrict__ ws_rank) {
  extern __shared__ int cnt[];  // [chunks][nb], then (KEYS_LDS) key[S], rank[S]
  __shared__ int wave_tmp[16];
  __shared__ int bad;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nb = E * Lb;
  const int S = T * k;

  int* key_buf = KEYS_LDS ? cnt + chunks * nb : ws_key;
  int* rank_buf = KEYS_LDS ? cnt + chunks * nb + S : ws_rank;
  for (int i = tid; i < chunks * nb; i += kAlignThreads) cnt[i] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();

  // ---- 1. route --------------------------------------------------------------
  for (int t = tid; t < T; t += kAlignThreads) {
    int l = adapter_ids[t];
    if (l == -1 && Lb > L) {
      l = L;  // base-only token: the expert's last bucket
    } else if (l < 0 || l >= L) {
      atomicMax(&bad, 1);
      l = 0;
    }
    if (!ROUTE) {
      for (int q = 0; q < k; ++q) {
        const int s = t * k + q;
        int e = ids_in != nullptr ? ids_in[s] : 0;
        if (e < 0 || e >= E) {
          atomicMax(&bad, 3);
          e = 0;
        }
        key_buf[s] = e * Lb + l;
      }
      continue;
    }
    float val[KMAX];
    int id[KMAX];
#pragma unroll
    for (int q = 0; q < KMAX; ++q) {
      val[q] = -INFINITY;
      id[q] = 0x7fffffff;
    }
    const float* lg = logits + static_cast<int64_t>(t) * E;
    // logits in batches of 16 loads issued together (one memory latency per
    // batch, not per expert); past E the batch holds -inf candidates, which
    // never pass a real logit (E >= k real ones come first)
    constexpr int kBatch = 16;
    for (int e0 = 0; e0 < E; e0 += kBatch) {
      float lv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) lv[u] = lg[min(e0 + u, E - 1)];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) lv[u] = e0 + u < E ? lv[u] : -INFINITY;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        float cv = lv[u];
        int ci = e0 + u;
        // carry the candidate down the list: it passes every entry it beats
        // (selects, no branches)
#pragma unroll
        for (int q = 0; q < KMAX; ++q) {
          const bool before = (q < k) & ((cv > val[q]) | ((cv == val[q]) & (ci < id[q])));
          const float tv = val[q];
          const int ti = id[q];
          val[q] = before ? cv : tv;
          id[q] = before ? ci : ti;
          cv = before ? tv : cv;
          ci = before ? ti : ci;
        }
      }
    }
    float ex[KMAX];
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < KMAX; ++q) {
      if (q < k) {
        ex[q] = expf(val[q] - val[0]);
        sum += ex[q];
      }
    }
#pragma unroll
    for (int q = 0; q < KMAX; ++q) {
      if (q < k) {
        int s = t * k + q;
        topk_ids[s] = id[q];
        topk_w[s] = ex[q] / sum;
        key_buf[s] = id[q] * Lb + l;
      }
    }
  }
  __syncthreads();

  // ---- 2. ranks inside each chunk -------------------------------------------
  // 64 slots at a time: a bitonic sort of (key, lane) across the wave puts
  // equal keys next to each other in lane order; a lane's rank among equal
  // keys is its sorted position minus its key's first position, and goes
  // back to the slot's lane with a permute.  The last lane of each key adds
  // the key's count to the chunk's counter.  Cost: 21 exchange steps,
  // whatever the number of distinct keys.
  const int chunk_len = (S + chunks - 1) / chunks;
  if (wave < chunks) {
    const int c0 = wave * chunk_len;
    const int c1 = min(S, c0 + chunk_len);
    int* my_cnt = cnt + wave * nb;
    for (int base = c0; base < c1; base += kWave) {
      const int s = base + lane;
      const bool valid = s < c1;
      const int key = valid ? key_buf[s] : nb;  // invalid lanes sort last
      // packed (key, lane): keys < 2^24 / 64 by the bucket limit
      int v = (key << 6) | lane;
#pragma unroll
      for (int kk = 2; kk <= kWave; kk <<= 1) {
#pragma unroll
        for (int j = kk >> 1; j > 0; j >>= 1) {
          const int o = __shfl_xor(v, j, kWave);
          const bool up = (lane & kk) == 0;       // this pair sorts ascending
          const bool low = (lane & j) == 0;       // this lane keeps the smaller
          v = (low == up) ? min(v, o) : max(v, o);
        }
      }
      const int skey = v >> 6, src = v & 63;
      const int prev = __shfl_up(skey, 1, kWave);
      const int next = __shfl_down(skey, 1, kWave);
      const bool head = lane == 0 || prev != skey;
      const bool tail = lane == kWave - 1 || next != skey;
      // first sorted position of this lane's key: inclusive max-scan of head positions
      int first = head ? lane : 0;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(first, d, kWave);
        if (lane >= d) first = max(first, y);
      }
      const int rank = lane - first;
      const int before = skey < nb ? my_cnt[skey] : 0;
      // back to the slot's own lane
      const int r_src = __builtin_amdgcn_ds_permute(src << 2, before + rank);
      if (valid) rank_buf[s] = r_src;
      __builtin_amdgcn_wave_barrier();
      if (tail && skey < nb) my_cnt[skey] = before + rank + 1;
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();

  // ---- 3. bucket offsets (block-wide exclusive scan) -------------------------
  const int per = (nb + kAlignThreads - 1) / kAlignThreads;
  const int b0 = min(nb, tid * per);
  const int b1 = min(nb, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b)
    for (int c = 0; c < chunks; ++c) local += cnt[c * nb + b];
  int total = 0;
  int run = block_exclusive_scan(local, wave_tmp, &total);
  for (int b = b0; b < b1; ++b) {
    offsets[b] = run;
    for (int c = 0; c < chunks; ++c) {
      int v = cnt[c * nb + b];
      cnt[c * nb + b] = run;
      run += v;
    }
  }
  if (tid == 0) offsets[nb] = total;
  __syncthreads();

  // ---- 4. scatter --------------------------------------------------------------
  for (int s = tid; s < S; s += kAlignThreads) {
    const int c = s / chunk_len;
    const int dst = cnt[c * nb + key_buf[s]] + rank_buf[s];
    if (dst >= 0 && dst < S)
      sorted_slots[dst] = s;
    else
      atomicMax(&bad, 2);  // cannot happen for consistent counts; never write out of bounds
  }
  __syncthreads();
  if (tid == 0 && status != nullptr) *status = bad;
}

// Per-slot keys and ranks go to LDS when they fit beside at least one
// chunk of counters.
static bool keys_in_lds(int S, int nb) { return 2ll * S + nb <= kAlignLdsInts; }

int align_chunks(int nb, int S) {
  const int budget = keys_in_lds(S, nb) ? kAlignLdsInts - 2 * S : kAlignLdsInts;
  int c = budget / nb;
  if (c > 16) c = 16;
  if (c < 1) c = 1;
  return c;
}

hipError_t launch_align(const float* logits, const int32_t* ids_in, const int32_t* adapter_ids,
                        int T, int E, int k, int L, int Lb, int32_t* topk_ids, float* topk_w,
                        int32_t* sorted_slots, int32_t* offsets, int32_t* status, int32_t* ws_key,
                        int32_t* ws_rank, hipStream_t stream) {
  const int nb = E * Lb;
  const int S = T * k;
  const int chunks = align_chunks(nb, S);
  const bool in_lds = keys_in_lds(S, nb);
  const size_t lds = (static_cast<size_t>(chunks) * nb + (in_lds ? 2 * S : 0)) * sizeof(int);
#define MOELORA_ALIGN_LAUNCH(KL, RT, KM)                                                          \
  hipLaunchKernelGGL((k_align<KL, RT, KM>), dim3(1), dim3(kAlignThreads), lds, stream, logits,    \
                     ids_in, adapter_ids, T, E, k, L, Lb, chunks, topk_ids, topk_w, sorted_slots, \
                     offsets, status, ws_key, ws_rank)
#define MOELORA_ALIGN_ROUTE(KL)                                      \
  do {                                                               \
    if (k <= 1) MOELORA_ALIGN_LAUNCH(KL, true, 1);                   \
    else if (k <= 2) MOELORA_ALIGN_LAUNCH(KL, true, 2);              \
    else if (k <= 4) MOELORA_ALIGN_LAUNCH(KL, true, 4);              \
    else MOELORA_ALIGN_LAUNCH(KL, true, kMaxTopK);                   \
  } while (0)
  const bool route = logits != nullptr;
  if (in_lds) {
    if (route) MOELORA_ALIGN_ROUTE(true); else MOELORA_ALIGN_LAUNCH(true, false, 1);
  } else {
    if (route) MOELORA_ALIGN_ROUTE(false); else MOELORA_ALIGN_LAUNCH(false, false, 1);
  }
#undef MOELORA_ALIGN_ROUTE
#undef MOELORA_ALIGN_LAUNCH
  return hipGetLastError();
}

}  // namespace moelora
