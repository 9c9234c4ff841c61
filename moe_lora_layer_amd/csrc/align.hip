// Routing and the (expert, adapter)-bucketed slot permutation, one workgroup.
//
// Follows the vLLM blog page "Multi-LoRA" (vllm.com.cn/blog/multi-lora),
// section "Implementing Multi-LoRA inference for MoE models in vLLM": each
// token goes to its most relevant experts, and expert routing compounds with
// the per-request adapter choice, so slots are grouped by (expert, adapter).
//
// Routing runs first in its own launch over as many workgroups as the batch
// needs (k_route): per token, k rounds of an arg-max over the E logits across
// a segment of lanes (ties keep the lower id), softmax weights renormalised
// over the kept k; the slot keys e*Lb + l go to the workspace.  Then one workgroup of 1024
// threads runs four phases separated by barriers:
//   1. keys: read the routed keys (or, without routing, form them from the
//      caller's expert ids) into LDS when they fit;
//   2. chunk ranks: the S slots are cut into C contiguous chunks, one per wave.
//      A wave walks its chunk 64 slots at a time; a bitonic sort of (key, lane)
//      across the wave brings equal keys together, so every slot gets its rank
//      among equal keys of lower index inside the chunk, and the chunk's
//      per-bucket counts live in LDS (cnt[c][b]), or in the workspace when
//      there are very many buckets; keys and ranks stay in LDS when they fit;
//   3. scan: bucket totals, a wavefront-level exclusive prefix scan over the
//      buckets gives bucket_offsets, and cnt[c][b] becomes the first output
//      position of chunk c's slots in bucket b;
//   4. scatter: sorted_slots[cnt[c][key] + rank] = s.
// ROUTED = false: no k_route launch; the caller's topk_ids (its own router,
// e.g. a router GEMM and top-k just before this path) give the keys.
// device_status: 0 ok, 1 an adapter id outside [0, L), 2 internal
// inconsistency, 3 a given expert id outside [0, E) (the largest code wins).
// No step depends on atomic ordering, so the result is bit-exact and stable.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moelora {

constexpr int kAlignThreads = 1024;
constexpr int kMaxTopK = 8;
constexpr int kKeyBatch = 8;  // slot keys loaded per thread before any is used

// KEYS_LDS: the per-slot keys and ranks live in LDS after the counters (small
// batches); otherwise in the workspace.
// Set in a routed key whose token had an adapter id outside [0, L) (keys stay
// below 2^18 by the bucket limit).
constexpr int kKeyBadAdapter = 1 << 30;

// Routing.  A segment of W lanes (the smallest power of two >= E, at most 64)
// holds one token, lane i of it the experts i, i + W, ...; k rounds of a
// segmented arg-max (larger logit, ties to the lower expert id) across the
// segment pick the token's experts in order, each round skipping the ones
// already picked; the segment's first lane writes the token.  Each wave makes
// one pass over 64 / W tokens, so a batch spreads over T W / 256 workgroups
// of four waves.  KMAX: the routing list length compiled in, the smallest of
// 1, 2, 4, 8 that holds k.
constexpr int kRouteWaves = 4;
constexpr int kRouteCached = 4;  // logits per lane kept in registers (E <= 256)

template <int KMAX>
__global__ void __launch_bounds__(kRouteWaves * kWave)
k_route(const float* __restrict__ logits, const int32_t* __restrict__ adapter_ids, int T, int E,
        int k, int L, int Lb, int W, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
        int32_t* __restrict__ ws_key) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int seg = lane / W, sl = lane % W;
  const int t = (blockIdx.x * kRouteWaves + wave) * (kWave / W) + seg;
  const bool tok = t < T;
  const float* lg = logits + static_cast<int64_t>(tok ? t : 0) * E;
  // a NaN logit ranks as -infinity (below every number), so every token still
  // gets k distinct experts in range
  auto rank_value = [](float v) { return v != v ? -INFINITY : v; };
  float lv[kRouteCached];
#pragma unroll
  for (int j = 0; j < kRouteCached; ++j) {
    const int e = sl + W * j;
    lv[j] = (tok && e < E) ? rank_value(lg[e]) : -INFINITY;
  }
  float win_v[KMAX];
  int win_id[KMAX];
#pragma unroll
  for (int q = 0; q < KMAX; ++q) {
    win_v[q] = -INFINITY;
    win_id[q] = 0x7fffffff;
    if (q >= k) continue;  // uniform
    // this lane's best expert not picked yet
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    auto consider = [&](float v, int e) {
      bool taken = false;
#pragma unroll
      for (int p = 0; p < q; ++p) taken |= win_id[p] == e;
      const bool better = !taken & ((v > bv) | ((v == bv) & (e < bi)));
      bv = better ? v : bv;
      bi = better ? e : bi;
    };
#pragma unroll
    for (int j = 0; j < kRouteCached; ++j) {
      const int e = sl + W * j;
      if (e < E) consider(lv[j], e);
    }
    for (int e = sl + W * kRouteCached; tok && e < E; e += W) consider(rank_value(lg[e]), e);  // E > 256
    // segmented arg-max over aligned groups of W lanes
    for (int d = 1; d < W; d <<= 1) {
      const float ov = __shfl_xor(bv, d, kWave);
      const int oi = __shfl_xor(bi, d, kWave);
      const bool better = (ov > bv) | ((ov == bv) & (oi < bi));
      bv = better ? ov : bv;
      bi = better ? oi : bi;
    }
    win_v[q] = bv;
    win_id[q] = bi;
  }
  if (!tok || sl != 0) return;
  int l = adapter_ids[t];
  int flag = 0;
  if (l == -1 && Lb > L) {
    l = L;  // base-only token: the expert's last bucket
  } else if (l < 0 || l >= L) {
    flag = kKeyBadAdapter;
    l = 0;
  }
  float ex[KMAX];
  float sum = 0.0f;
#pragma unroll
  for (int q = 0; q < KMAX; ++q) {
    if (q < k) {
      ex[q] = expf(win_v[q] - win_v[0]);
      sum += ex[q];
    }
  }
#pragma unroll
  for (int q = 0; q < KMAX; ++q) {
    if (q < k) {
      const int s = t * k + q;
      topk_ids[s] = win_id[q];
      topk_w[s] = ex[q] / sum;
      ws_key[s] = (win_id[q] * Lb + l) | flag;
    }
  }
}

// CNT_LDS: the per-chunk bucket counters live in LDS (up to kAlignLdsInts of
// them); otherwise (very many buckets) in the workspace, updated with atomics.
template <bool KEYS_LDS, bool ROUTED, bool CNT_LDS>
__global__ void __launch_bounds__(kAlignThreads)
k_align(const int32_t* __restrict__ ids_in, const int32_t* __restrict__ adapter_ids, int T, int E,
        int k, int L, int Lb, int chunks, int32_t* __restrict__ sorted_slots,
        int32_t* __restrict__ offsets, int32_t* __restrict__ status, int32_t* __restrict__ ws_key,
        int32_t* __restrict__ ws_rank, int32_t* __restrict__ ws_cnt) {
  extern __shared__ int lds[];  // (CNT_LDS) cnt[chunks][nb], then (KEYS_LDS) key[S], rank[S]
  __shared__ int wave_tmp[16];
  __shared__ int bad;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nb = E * Lb;
  const int S = T * k;

  int* cnt = CNT_LDS ? lds : ws_cnt;
  int* const keys_base = CNT_LDS ? lds + chunks * nb : lds;
  int* key_buf = KEYS_LDS ? keys_base : ws_key;
  int* rank_buf = KEYS_LDS ? keys_base + S : ws_rank;
  for (int i = tid; i < chunks * nb; i += kAlignThreads) cnt[i] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();

  // ---- 1. keys -----------------------------------------------------------------
  if (ROUTED) {
    // keys from k_route; a flagged key marks a token whose adapter id was out of range.
    // kKeyBatch keys per thread are loaded before any is used, so their
    // latencies overlap (the loop would otherwise wait for each load in turn)
    for (int s0 = tid; s0 < S; s0 += kKeyBatch * kAlignThreads) {
      int kv[kKeyBatch];
#pragma unroll
      for (int u = 0; u < kKeyBatch; ++u) {
        const int s = s0 + u * kAlignThreads;
        kv[u] = s < S ? ws_key[s] : 0;
      }
#pragma unroll
      for (int u = 0; u < kKeyBatch; ++u) {
        const int s = s0 + u * kAlignThreads;
        if (s >= S) break;
        int key = kv[u];
        if (key & kKeyBadAdapter) {
          atomicMax(&bad, 1);
          key &= ~kKeyBadAdapter;
        }
        if (key < 0 || key >= nb) {  // cannot happen for routed keys; never index with it
          atomicMax(&bad, 2);
          key = 0;
        }
        key_buf[s] = key;
      }
    }
  } else {
    for (int t = tid; t < T; t += kAlignThreads) {
      int l = adapter_ids[t];
      if (l == -1 && Lb > L) {
        l = L;  // base-only token: the expert's last bucket
      } else if (l < 0 || l >= L) {
        atomicMax(&bad, 1);
        l = 0;
      }
      for (int q = 0; q < k; ++q) {
        const int s = t * k + q;
        int e = ids_in != nullptr ? ids_in[s] : 0;
        if (e < 0 || e >= E) {
          atomicMax(&bad, 3);
          e = 0;
        }
        key_buf[s] = e * Lb + l;
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
      // packed (key, lane): keys <= 2^18 by the bucket limit, far below 2^25
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
      int before;
      if (CNT_LDS) {
        before = skey < nb ? my_cnt[skey] : 0;
        __builtin_amdgcn_wave_barrier();
        if (tail && skey < nb) my_cnt[skey] = before + rank + 1;
        __builtin_amdgcn_wave_barrier();
      } else {
        // counters in global memory: the key's last lane adds the key's count
        // with one returning atomic, and every lane of the key takes the old
        // value from that lane (the nearest tail at or after it)
        int old = 0;
        if (tail && skey < nb) old = atomicAdd(my_cnt + skey, rank + 1);
        int last = tail ? lane : kWave;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
          const int y = __shfl_down(last, d, kWave);
          if (lane + d < kWave) last = min(last, y);
        }
        before = __shfl(old, last, kWave);
      }
      // back to the slot's own lane
      const int r_src = __builtin_amdgcn_ds_permute(src << 2, before + rank);
      if (valid) rank_buf[s] = r_src;
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

AlignLayout align_layout(int nb, int S) {
  AlignLayout a;
  a.cnt_lds = nb <= kAlignLdsInts;
  if (a.cnt_lds) {
    // keys and ranks go to LDS when they fit beside at least one chunk of counters
    a.keys_lds = 2ll * S + nb <= kAlignLdsInts;
    const int budget = a.keys_lds ? kAlignLdsInts - 2 * S : kAlignLdsInts;
    a.chunks = std::max(1, std::min(16, budget / nb));
    a.cnt_ints = 0;
  } else {
    // more buckets than LDS holds counters: counters in the workspace, one
    // chunk per 1024 slots (every chunk's counters are cleared by the kernel)
    a.keys_lds = 2ll * S <= kAlignLdsInts;
    a.chunks = std::max(1, std::min(16, S / 1024));
    a.cnt_ints = static_cast<int64_t>(a.chunks) * nb;
  }
  return a;
}

hipError_t launch_align(const float* logits, const int32_t* ids_in, const int32_t* adapter_ids,
                        int T, int E, int k, int L, int Lb, int32_t* topk_ids, float* topk_w,
                        int32_t* sorted_slots, int32_t* offsets, int32_t* status, int32_t* ws_key,
                        int32_t* ws_rank, int32_t* ws_cnt, hipStream_t stream) {
  const int nb = E * Lb;
  const int S = T * k;
  const AlignLayout al = align_layout(nb, S);
  const int chunks = al.chunks;
  const bool in_lds = al.keys_lds;
  const size_t lds =
      ((al.cnt_lds ? static_cast<size_t>(chunks) * nb : 0) + (in_lds ? 2 * S : 0)) * sizeof(int);
  const bool routed = logits != nullptr;
  if (routed && T > 0) {
    int W = 1;
    while (W < E && W < kWave) W <<= 1;
    const int per_wg = kRouteWaves * (kWave / W);  // tokens per workgroup
    const dim3 grid(static_cast<unsigned>((T + per_wg - 1) / per_wg));
#define MOELORA_ROUTE_LAUNCH(KM)                                                                 \
  hipLaunchKernelGGL((k_route<KM>), grid, dim3(kRouteWaves * kWave), 0, stream, logits,          \
                     adapter_ids, T, E, k, L, Lb, W, topk_ids, topk_w, ws_key)
    if (k <= 1) MOELORA_ROUTE_LAUNCH(1);
    else if (k <= 2) MOELORA_ROUTE_LAUNCH(2);
    else if (k <= 4) MOELORA_ROUTE_LAUNCH(4);
    else MOELORA_ROUTE_LAUNCH(kMaxTopK);
#undef MOELORA_ROUTE_LAUNCH
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define MOELORA_ALIGN_LAUNCH(KL, RT, CL)                                                           \
  hipLaunchKernelGGL((k_align<KL, RT, CL>), dim3(1), dim3(kAlignThreads), lds, stream, ids_in,    \
                     adapter_ids, T, E, k, L, Lb, chunks, sorted_slots, offsets, status, ws_key, \
                     ws_rank, ws_cnt)
#define MOELORA_ALIGN_LAUNCH2(KL, CL)                                                              \
  if (routed) MOELORA_ALIGN_LAUNCH(KL, true, CL); else MOELORA_ALIGN_LAUNCH(KL, false, CL)
  if (!al.cnt_lds && ws_cnt == nullptr) return hipErrorInvalidValue;
  if (al.cnt_lds) {
    if (in_lds) { MOELORA_ALIGN_LAUNCH2(true, true); } else { MOELORA_ALIGN_LAUNCH2(false, true); }
  } else {
    if (in_lds) { MOELORA_ALIGN_LAUNCH2(true, false); } else { MOELORA_ALIGN_LAUNCH2(false, false); }
  }
#undef MOELORA_ALIGN_LAUNCH2
#undef MOELORA_ALIGN_LAUNCH
  return hipGetLastError();
}

}  // namespace moelora
