// C ABI of the fused MoE multi-LoRA layer: argument checks, workspace layout,
// tile planning and the launch sequence.  Declarations and the meaning of
// every argument are in include/moelora.h.
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "launch.h"
#include "moelora.h"

// Device scratch of moelora_forward_noalloc: one copy per GPU the library runs
// on, held until the process ends.  Host code never passes the array's name to
// a kernel or a copy (on the host it is only a stand-in for the symbol): it
// uses the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MOELORA_NOALLOC_SCRATCH_BYTES];

using moelora::TilePlan;

namespace {

constexpr size_t kSectionAlign = 256;
constexpr int64_t kMaxExpertAdapters = 65536;  // E * L
constexpr int64_t kMaxGrid = (1ll << 31) - 1;

size_t round_up(size_t x) { return (x + kSectionAlign - 1) / kSectionAlign * kSectionAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// buckets per expert: the adapters, plus one for base-only tokens when enabled
int64_t buckets_per_expert(const moelora_dims* d) {
  return static_cast<int64_t>(d->adapters) + ((d->flags & MOELORA_FLAG_BASE_ONLY) ? 1 : 0);
}

// plan fields: 0 (automatic) or a value the kernels provide
int check_plan(const moelora_plan& o) {
  const int rows = o.gemm_rows;
  if (rows != 0 && rows != 32 && rows != 64 && rows != 128 && rows != 256)
    return MOELORA_ERR_UNSUPPORTED;
  if (o.gemm_form < 0 || o.gemm_form > 3) return MOELORA_ERR_UNSUPPORTED;
  if (o.gemm_form != 0 && (rows == 0 || (o.gemm_form == 1 && rows == 256) ||
                           (o.gemm_form == 2 && rows < 128) || (o.gemm_form == 3 && rows != 128)))
    return MOELORA_ERR_UNSUPPORTED;
  if (o.lora_rows != 0 && o.lora_rows != 16 && o.lora_rows != 64) return MOELORA_ERR_UNSUPPORTED;
  if (o.ksplit_gate_up < 0 || o.ksplit_gate_up > 1024 || o.ksplit_down < 0 || o.ksplit_down > 1024)
    return MOELORA_ERR_UNSUPPORTED;
  if (o.fuse < 0 || o.fuse > 3) return MOELORA_ERR_UNSUPPORTED;
  if (o.order < 0 || o.order > 5) return MOELORA_ERR_UNSUPPORTED;
  return MOELORA_OK;
}

int check_dims(const moelora_dims* d) {
  if (d == nullptr) return MOELORA_ERR_NULL;
  if (d->dtype != MOELORA_F32 && d->dtype != MOELORA_BF16) return MOELORA_ERR_UNSUPPORTED;
  if (d->rank != 16 && d->rank != 32 && d->rank != 64) return MOELORA_ERR_UNSUPPORTED;
  if ((d->flags & ~(MOELORA_FLAG_DETERMINISTIC | MOELORA_FLAG_BASE_ONLY | MOELORA_FLAG_UNFUSED |
                    MOELORA_FLAG_IN_OUT)) != 0)
    return MOELORA_ERR_UNSUPPORTED;
  if (d->tokens < 0 || d->hidden <= 0 || d->intermediate <= 0) return MOELORA_ERR_DIMS;
  if (d->hidden % 64 != 0 || d->intermediate % 64 != 0) return MOELORA_ERR_DIMS;
  if (d->hidden > (1 << 20) || d->intermediate > (1 << 20)) return MOELORA_ERR_DIMS;
  if (d->experts < 1 || d->adapters < 1 || d->top_k < 1 || d->top_k > 8 ||
      d->top_k > d->experts)
    return MOELORA_ERR_DIMS;
  // E * L <= 65536 adapters x experts (plus one base-only bucket per expert)
  if (static_cast<int64_t>(d->experts) * d->adapters > kMaxExpertAdapters ||
      static_cast<int64_t>(d->experts) * buckets_per_expert(d) > 2 * kMaxExpertAdapters)
    return MOELORA_ERR_DIMS;
  if (d->tokens * d->top_k >= (1ll << 31)) return MOELORA_ERR_DIMS;
  if (d->plan.gemm_form == 3 && d->dtype != MOELORA_BF16) return MOELORA_ERR_UNSUPPORTED;
  return check_plan(d->plan);
}

// The tile plan: the automatic choice for every field of d->plan that is 0,
// the caller's value for the others (split counts rounded so that no K range
// is empty).
TilePlan make_plan(const moelora_dims* d) {
  const moelora_plan& o = d->plan;
  const int64_t S = d->tokens * d->top_k;
  const int64_t E = d->experts, nb = E * buckets_per_expert(d);
  const int64_t avg = (S + E - 1) / E;  // mean rows per expert
  TilePlan p;
  // one M-tile per expert in the common case: mean rows per expert plus 25%
  const int64_t want = (avg * 5 + 3) / 4;
  // (bf16: 128-row tiles only up to 160 rows; above that one 256-row tile per
  // expert streams the weights once, 1536 tokens x 16 experts top-2: 1.31 ms
  // against 1.44 ms on 128-row DMA tiles and 1.74 ms on 128-row reuse tiles)
  const int64_t big = d->dtype == MOELORA_BF16 ? 160 : 256;
  p.bm = o.gemm_rows != 0 ? o.gemm_rows
                          : (want <= 32 ? 32 : (want <= 64 ? 64 : (want <= big ? 128 : 256)));
  // at most one 128-row M-tile per expert: nothing reuses a weight tile, so the
  // weights are streamed (nontemporal loads, rotated K walk)
  p.stream = o.gemm_form != 0 ? o.gemm_form == 1 || o.gemm_form == 3
                              : (p.bm < 128 || (p.bm == 128 && want <= 160));
  // bf16 weight-streaming 128-row M-tiles run on the DMA tiles of 256 weight
  // rows with three stages (dense 128 x 8192 -> 57344 gate_up 212 -> 197 us,
  // a 1024-token 16-expert layer 1.65 -> 1.42 ms)
  p.dma128 = d->dtype == MOELORA_BF16 && p.bm == 128 &&
             (o.gemm_form == 3 || (o.gemm_form == 0 && p.stream));
  // LoRA tiles: 64 rows when buckets average many rows (the tall-tile kernels),
  // else one 16-row MFMA block (the weight-streaming kernels)
  p.lora_db = o.lora_rows != 0 ? o.lora_rows == 64
                               : S / std::max<int64_t>(1, std::min<int64_t>(nb, S)) > 16;
  p.bml = p.lora_db ? 64 : 16;
  p.max_mt = static_cast<int>(S / p.bm + (E < S ? E : S) + 1);
  p.max_lt = static_cast<int>(S / p.bml + (nb < S ? nb : S) + 1);
  // Split K only when the real M x N tiles cannot give every CU a workgroup
  // (e.g. one expert and a narrow output): ~512 workgroups (two per CU;
  // more splits cost more in fp32 atomics than they gain), >= 8 K-steps per
  // split.
  const int64_t est_tiles = std::max<int64_t>((S + p.bm - 1) / p.bm, std::min<int64_t>(E, S));
  // The 128 x 256 DMA tiles hold a CU's LDS (one workgroup per CU): they
  // aim at about one round of 256 workgroups, and leave K whole from three
  // quarters of a round up.
  auto splits = [&](int64_t N, int64_t K, int64_t forced) {
    const int64_t tn = p.dma128 ? 256 : 128;
    const int64_t wgs = std::max<int64_t>(1, est_tiles * ((N + tn - 1) / tn));
    const int64_t steps = K / (d->dtype == MOELORA_BF16 ? 64 : 32);
    if (forced == 0 && wgs >= (p.dma128 ? 192 : 256)) return 1;
    const int64_t auto_want = p.dma128 ? (256 + wgs / 2) / wgs : (512 + wgs - 1) / wgs;
    const int64_t want =
        forced != 0 ? std::min<int64_t>(forced, steps)
                    : std::max<int64_t>(1, std::min<int64_t>(auto_want, steps / 8));
    // equal K ranges with none empty: every split then owns real work (and
    // writes its whole partial in deterministic mode)
    const int64_t per = (steps + want - 1) / want;
    return static_cast<int>((steps + per - 1) / per);
  };
  p.ksplit_gu = splits(2 * d->intermediate, d->hidden, o.ksplit_gate_up);
  p.ksplit_dn = splits(d->hidden, d->intermediate, o.ksplit_down);
  // bf16 GEMMs with unsplit K run the LoRA expand in their epilogue (every
  // tile family stages the expand's operands in its idle LDS, a group of
  // adapter buckets per memory round trip)
  const bool fusable = d->dtype == MOELORA_BF16 && (d->flags & MOELORA_FLAG_UNFUSED) == 0 &&
                       o.fuse != 2;
  p.fuse_gu = fusable && p.ksplit_gu == 1;
  p.fuse_dn = fusable && p.ksplit_dn == 1;
  // plan.fuse 3: the fused gate_up epilogue also adds its columns' share of
  // the down projection's shrink (no separate pass over ACT).  Not the
  // automatic choice: on MI355X the epilogue work (an LDS round trip of the
  // activation tile and a load round trip per adapter bucket, with the matrix
  // cores idle) costs more than the separate shrink's pass over ACT (prefill
  // gate_up GEMM +180 us against a 57 us shrink, decode +25 against 16 us).
  p.fold_dn = p.fuse_gu && o.fuse == 3;
  p.det = (d->flags & MOELORA_FLAG_DETERMINISTIC) != 0;
  // tall bf16 LoRA tiles: per-split partials and an ordered sum beat relaxed
  // fp32 atomics into Z (a few hundred split tiles each adding 64 x r values)
  p.shrink_partials = p.det || (p.lora_db && d->dtype == MOELORA_BF16);
  p.nad = d->adapters;
  p.kn = (d->flags & MOELORA_FLAG_IN_OUT) != 0;
  // workgroup order: tiles that reuse their weight tile (256 rows, 128-row
  // reuse) and the 128-row DMA tiles run each expert's tiles together per XCD
  // (one L2 holds the expert's activation rows: a 1024-token 16-expert layer
  // 1.28 ms against 1.48 ms rotated); the other weight-streaming tiles rotate
  // every workgroup's K walk, except over k-major weights, whose neighbouring
  // N-tiles read neighbouring pieces of the same k-rows
  const bool reuse = p.bm == 256 || (p.bm == 128 && !p.stream) || p.dma128;
  p.order = o.order != 0 ? o.order
                         : (reuse ? moelora::ORDER_XCD : (p.kn ? moelora::ORDER_LAUNCH : moelora::ORDER_ROTATED));
  return p;
}

// N-tiles of the gate_up GEMM (each covers 128 intermediate columns in the
// 256-row bf16 tiles, 64 in the others): the partial slots of the folded
// down shrink in deterministic mode.
int64_t gate_up_ntiles(const moelora_dims* d, const TilePlan& plan) {
  const int64_t tn = ((plan.bm == 256 && d->dtype == MOELORA_BF16) || plan.dma128) ? 128 : 64;
  return (d->intermediate + tn - 1) / tn;
}

struct ForwardLayout {
  size_t pos, counts, etiles, mtiles, ltiles, g, z1, z2, act, d, parts, total;
};

ForwardLayout forward_layout(const moelora_dims* d, const TilePlan& plan) {
  const size_t S = static_cast<size_t>(d->tokens * d->top_k);
  const size_t h = static_cast<size_t>(d->hidden), I = static_cast<size_t>(d->intermediate);
  const size_t r = static_cast<size_t>(d->rank);
  const size_t esz = d->dtype == MOELORA_BF16 ? 2 : 4;
  ForwardLayout L;
  size_t off = 0;
  L.pos = off;    off += round_up(S * 4);
  L.counts = off; off += round_up(moelora::kCountsInts * 4);
  L.etiles = off; off += round_up((static_cast<size_t>(d->experts) + 1) * 4);
  L.mtiles = off; off += round_up(static_cast<size_t>(plan.max_mt) * 16);
  L.ltiles = off; off += round_up(static_cast<size_t>(plan.max_lt) * 16);
  // G is written only when the gate_up expand runs as a kernel of its own
  L.g = off;      off += plan.fuse_gu ? 0 : round_up(S * 2 * I * 4);
  L.act = off;    off += round_up(S * I * esz);
  L.z1 = off;     // Z1, Z2 and D are adjacent: one fill clears Z1 and Z2, and D
  L.z2 = off + S * r * 4;  // too when the down GEMM accumulates with atomics
  L.d = off + 2 * S * r * 4;
  off += round_up(2 * S * r * 4 + S * h * 4);
  // one region for the partials of whichever split reduction runs (they run
  // one after another): the shrinks' (deterministic mode or tall tiles), the
  // split gate_up GEMM's (deterministic mode) and the split down GEMM's
  L.parts = off;
  if (plan.shrink_partials || (plan.det && plan.fold_dn) || plan.ksplit_dn > 1) {
    const int dt = d->dtype == MOELORA_BF16 ? moelora::DT_BF16 : moelora::DT_F32;
    size_t n = 0;
    n = std::max(n, static_cast<size_t>(moelora::shrink_parts(dt, d->rank, plan, d->hidden)) * S * r);
    n = std::max(n, static_cast<size_t>(moelora::shrink_parts(dt, d->rank, plan, d->intermediate)) * S * r);
    if (plan.det && plan.ksplit_gu > 1) n = std::max(n, static_cast<size_t>(plan.ksplit_gu) * S * 2 * I);
    if (plan.det && plan.fold_dn) n = std::max(n, static_cast<size_t>(gate_up_ntiles(d, plan)) * S * r);
    if (plan.ksplit_dn > 1) n = std::max(n, static_cast<size_t>(plan.ksplit_dn) * S * h);
    off += round_up(n * 4);
  }
  L.total = off;
  return L;
}

// The dense projection planned as the layer's down GEMM with one expert and
// k = 1: hidden = out_features (N), intermediate = in_features (K).
moelora_dims dense_as_layer(const moelora_dense_dims* d) {
  moelora_dims m{};
  m.tokens = d->tokens;
  m.hidden = d->out_features;
  m.intermediate = d->in_features;
  m.experts = 1;
  m.top_k = 1;
  m.adapters = d->adapters;
  m.rank = d->rank;
  m.dtype = d->dtype;
  m.flags = d->flags;
  m.plan = d->plan;
  return m;
}

// the dense dims as layer dims, checked (the projection is planned as the
// layer's down GEMM, so a gate_up split count is refused).  Automatic tiles of
// the projection: when its rows would get the 128-row weight-streaming tiles
// and those tiles fall short of one round of the MI355X's 256 CUs, bf16 takes
// the 128 x 256 DMA tiles and fp32 the four-wave weight-reuse tiles, split
// over K into about one round (q/k/v projection 128 x 8192 -> 10240: 61-64
// us per call with 6 splits of the DMA tiles, 71-72 with the reuse tiles in
// 3, 97-100 with unsplit streaming tiles), with at least 8 K-steps per split
// as in the layer's own rule.
int dense_check(const moelora_dense_dims* d, moelora_dims* m) {
  if (d == nullptr) return MOELORA_ERR_NULL;
  *m = dense_as_layer(d);
  if (d->plan.ksplit_gate_up != 0) return MOELORA_ERR_UNSUPPORTED;
  const int rc = check_dims(m);
  if (rc != MOELORA_OK) return rc;
  moelora_plan& p = m->plan;
  const int64_t want = (d->tokens * 5 + 3) / 4;  // the layer's automatic rule, one expert
  if (p.gemm_rows == 0 && p.gemm_form == 0 && p.ksplit_down == 0 && want > 64 && want <= 256) {
    const int64_t tiles = ((d->tokens + 127) / 128) * ((d->out_features + 127) / 128);
    if (tiles < 256) {
      const bool bf16 = d->dtype == MOELORA_BF16;
      // the DMA tiles are 256 outputs wide
      const int64_t wtiles = bf16 ? ((d->tokens + 127) / 128) * ((d->out_features + 255) / 256) : tiles;
      p.gemm_rows = 128;
      p.gemm_form = bf16 ? 3 : 2;
      const int64_t steps = d->in_features / (bf16 ? 64 : 32);
      p.ksplit_down = static_cast<int32_t>(std::max<int64_t>(
          1, std::min<int64_t>((256 + wtiles / 2) / wtiles, steps / 8)));
    }
  }
  return MOELORA_OK;
}

// the resolved plan in the ABI's terms
moelora_plan plan_out(const TilePlan& p) {
  moelora_plan o;
  o.gemm_rows = p.bm;
  o.gemm_form = p.dma128 ? 3 : (p.bm < 128 || (p.bm == 128 && p.stream) ? 1 : 2);
  o.lora_rows = p.bml;
  o.ksplit_gate_up = p.ksplit_gu;
  o.ksplit_down = p.ksplit_dn;
  o.fuse = p.fold_dn ? 3 : ((p.fuse_gu || p.fuse_dn) ? 1 : 2);
  o.order = p.order;
  return o;
}

struct DenseLayout {
  size_t key, rank, cnt, slots, offsets, pos, counts, etiles, mtiles, ltiles, z, d, parts, total;
};

DenseLayout dense_layout(const moelora_dims* m, const TilePlan& plan) {
  const size_t T = static_cast<size_t>(m->tokens), N = static_cast<size_t>(m->hidden);
  const size_t r = static_cast<size_t>(m->rank), Lb = static_cast<size_t>(buckets_per_expert(m));
  DenseLayout L;
  size_t off = 0;
  L.key = off;     off += round_up(T * 4);
  L.rank = off;    off += round_up(T * 4);
  L.cnt = off;
  off += round_up(static_cast<size_t>(moelora::align_layout(static_cast<int>(Lb), static_cast<int>(T)).cnt_ints) * 4);
  L.slots = off;   off += round_up(T * 4);
  L.offsets = off; off += round_up((Lb + 1) * 4);
  L.pos = off;     off += round_up(T * 4);
  L.counts = off;  off += round_up(moelora::kCountsInts * 4);
  L.etiles = off;  off += round_up(2 * 4);
  L.mtiles = off;  off += round_up(static_cast<size_t>(plan.max_mt) * 16);
  L.ltiles = off;  off += round_up(static_cast<size_t>(plan.max_lt) * 16);
  L.z = off;       // Z and D adjacent: the prep launch clears Z (and D under atomic split-K)
  L.d = off + T * r * 4;
  off += round_up(T * r * 4 + T * N * 4);
  L.parts = off;
  if (plan.shrink_partials || plan.ksplit_dn > 1) {
    const int dt = m->dtype == MOELORA_BF16 ? moelora::DT_BF16 : moelora::DT_F32;
    size_t n = plan.shrink_partials
                   ? static_cast<size_t>(moelora::shrink_parts(dt, m->rank, plan, m->intermediate)) * T * r
                   : 0;
    if (plan.ksplit_dn > 1) n = std::max(n, static_cast<size_t>(plan.ksplit_dn) * T * N);
    off += round_up(n * 4);
  }
  L.total = off;
  return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOELORA_OK : MOELORA_ERR_HIP; }

// Device address of `scratch` on the current device, looked up once per device
// (hipGetSymbolAddress with that device current) and kept for later calls.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Align workspace: per-slot keys and ranks, and the bucket counters when the
// buckets are too many for LDS.
struct AlignWs {
  size_t key, rank, cnt, total;
};

AlignWs align_ws_for(int64_t nb, int64_t S) {
  const moelora::AlignLayout al = moelora::align_layout(static_cast<int>(nb), static_cast<int>(S));
  AlignWs w;
  w.key = 0;
  w.rank = round_up(static_cast<size_t>(S) * 4);
  w.cnt = 2 * w.rank;
  w.total = w.cnt + round_up(static_cast<size_t>(al.cnt_ints) * 4);
  return w;
}

AlignWs align_ws(const moelora_dims* d) {
  return align_ws_for(static_cast<int64_t>(d->experts) * buckets_per_expert(d),
                      d->tokens * d->top_k);
}

}  // namespace

extern "C" {

int moelora_abi_version(void) { return MOELORA_ABI_VERSION; }

const char* moelora_status_string(int status) {
  switch (status) {
    case MOELORA_OK: return "moelora: ok";
    case MOELORA_ERR_NULL: return "moelora: a required pointer is NULL";
    case MOELORA_ERR_DIMS: return "moelora: dimensions out of range";
    case MOELORA_ERR_UNSUPPORTED: return "moelora: unsupported dtype or rank";
    case MOELORA_ERR_ALIGNMENT: return "moelora: a tensor pointer is not 16-byte aligned";
    case MOELORA_ERR_WORKSPACE: return "moelora: workspace missing or too small";
    case MOELORA_ERR_HIP: return "moelora: HIP launch error";
    case MOELORA_ERR_TOO_LARGE:
      return "moelora: the call needs more workspace than the static scratch of "
             "moelora_forward_noalloc holds";
    default: return "moelora: unknown status";
  }
}

int moelora_align_workspace_size(const moelora_dims* dims, size_t* bytes) {
  const int rc = check_dims(dims);
  if (rc != MOELORA_OK) return rc;
  if (bytes == nullptr) return MOELORA_ERR_NULL;
  *bytes = align_ws(dims).total;
  return MOELORA_OK;
}

int moelora_align(const moelora_dims* dims, const float* router_logits,
                  const int32_t* adapter_ids, int32_t* topk_ids, float* topk_weights,
                  int32_t* sorted_slots, int32_t* bucket_offsets, int32_t* device_status,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != MOELORA_OK) return rc;
  if (bucket_offsets == nullptr) return MOELORA_ERR_NULL;
  const int64_t T = dims->tokens;
  if (T > 0 && (router_logits == nullptr || adapter_ids == nullptr || topk_ids == nullptr ||
                topk_weights == nullptr || sorted_slots == nullptr))
    return MOELORA_ERR_NULL;
  size_t need = 0;
  moelora_align_workspace_size(dims, &need);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MOELORA_ERR_WORKSPACE;
  const void* ptrs[] = {router_logits, adapter_ids, topk_ids, topk_weights, sorted_slots,
                        bucket_offsets, workspace};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned16(p)) return MOELORA_ERR_ALIGNMENT;
  const AlignWs aw = align_ws(dims);
  char* ws = static_cast<char*>(workspace);
  return hip_status(moelora::launch_align(
      router_logits, nullptr, adapter_ids, static_cast<int>(T), dims->experts, dims->top_k,
      dims->adapters, static_cast<int>(buckets_per_expert(dims)), topk_ids, topk_weights,
      sorted_slots, bucket_offsets, device_status, reinterpret_cast<int32_t*>(ws + aw.key),
      reinterpret_cast<int32_t*>(ws + aw.rank), reinterpret_cast<int32_t*>(ws + aw.cnt),
      static_cast<hipStream_t>(stream)));
}

int moelora_align_topk(const moelora_dims* dims, const int32_t* topk_ids,
                       const int32_t* adapter_ids, int32_t* sorted_slots,
                       int32_t* bucket_offsets, int32_t* device_status, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != MOELORA_OK) return rc;
  if (bucket_offsets == nullptr) return MOELORA_ERR_NULL;
  const int64_t T = dims->tokens;
  if (T > 0 && (topk_ids == nullptr || adapter_ids == nullptr || sorted_slots == nullptr))
    return MOELORA_ERR_NULL;
  size_t need = 0;
  moelora_align_workspace_size(dims, &need);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MOELORA_ERR_WORKSPACE;
  const void* ptrs[] = {topk_ids, adapter_ids, sorted_slots, bucket_offsets, workspace};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned16(p)) return MOELORA_ERR_ALIGNMENT;
  const AlignWs aw = align_ws(dims);
  char* ws = static_cast<char*>(workspace);
  return hip_status(moelora::launch_align(
      nullptr, topk_ids, adapter_ids, static_cast<int>(T), dims->experts, dims->top_k,
      dims->adapters, static_cast<int>(buckets_per_expert(dims)), nullptr, nullptr, sorted_slots,
      bucket_offsets, device_status, reinterpret_cast<int32_t*>(ws + aw.key),
      reinterpret_cast<int32_t*>(ws + aw.rank), reinterpret_cast<int32_t*>(ws + aw.cnt),
      static_cast<hipStream_t>(stream)));
}

int moelora_forward_workspace_size(const moelora_dims* dims, size_t* bytes) {
  const int rc = check_dims(dims);
  if (rc != MOELORA_OK) return rc;
  if (bytes == nullptr) return MOELORA_ERR_NULL;
  *bytes = dims->tokens == 0 ? 0 : forward_layout(dims, make_plan(dims)).total;
  return MOELORA_OK;
}

int moelora_forward_workspace_layout(const moelora_dims* dims, size_t offsets[5]) {
  const int rc = check_dims(dims);
  if (rc != MOELORA_OK) return rc;
  if (offsets == nullptr) return MOELORA_ERR_NULL;
  const ForwardLayout L = forward_layout(dims, make_plan(dims));
  offsets[0] = L.g;
  offsets[1] = L.z1;
  offsets[2] = L.act;
  offsets[3] = L.z2;
  offsets[4] = L.d;
  return MOELORA_OK;
}

int moelora_forward_plan(const moelora_dims* dims, moelora_plan* plan) {
  if (plan == nullptr) return MOELORA_ERR_NULL;
  const int rc = check_dims(dims);
  if (rc != MOELORA_OK) return rc;
  *plan = plan_out(make_plan(dims));
  return MOELORA_OK;
}

int moelora_dense_forward_plan(const moelora_dense_dims* dims, moelora_plan* plan) {
  moelora_dims m;
  const int rc = dense_check(dims, &m);
  if (rc != MOELORA_OK) return rc;
  if (plan == nullptr) return MOELORA_ERR_NULL;
  const TilePlan tp = make_plan(&m);
  moelora_plan o = plan_out(tp);
  o.ksplit_gate_up = 0;
  o.fuse = tp.fuse_dn ? 1 : 2;
  *plan = o;
  return MOELORA_OK;
}

int moelora_forward_fusion(const moelora_dims* dims, int* flags) {
  if (flags == nullptr) return MOELORA_ERR_NULL;
  const int rc = check_dims(dims);
  if (rc != MOELORA_OK) return rc;
  const TilePlan plan = make_plan(dims);
  *flags = (plan.fuse_gu ? MOELORA_FUSED_GATE_UP : 0) | (plan.fuse_dn ? MOELORA_FUSED_DOWN : 0) |
           (plan.fold_dn ? MOELORA_FUSED_DOWN_SHRINK : 0);
  return MOELORA_OK;
}

int moelora_forward(const moelora_dims* dims, const void* x, const void* w_gate_up,
                    const void* w_down, const void* a_gate_up, const void* b_gate_up,
                    const void* a_down, const void* b_down, const int32_t* topk_ids,
                    const float* topk_weights, const int32_t* sorted_slots,
                    const int32_t* bucket_offsets, void* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return moelora_forward_profiled(dims, x, w_gate_up, w_down, a_gate_up, b_gate_up, a_down,
                                  b_down, topk_ids, topk_weights, sorted_slots, bucket_offsets,
                                  out, workspace, workspace_bytes, stream, nullptr);
}

int moelora_forward_noalloc(const moelora_dims* dims, const void* x, const void* w_gate_up,
                            const void* w_down, const void* a_gate_up, const void* b_gate_up,
                            const void* a_down, const void* b_down, const int32_t* topk_ids,
                            const float* topk_weights, const int32_t* sorted_slots,
                            const int32_t* bucket_offsets, void* out, void* stream) {
  size_t need = 0;
  const int rc = moelora_forward_workspace_size(dims, &need);
  if (rc != MOELORA_OK) return rc;
  if (dims->tokens == 0) return MOELORA_OK;
  if (need > MOELORA_NOALLOC_SCRATCH_BYTES) return MOELORA_ERR_TOO_LARGE;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return MOELORA_ERR_HIP;
  // the same launch sequence as moelora_forward; every accumulator it needs
  // cleared is cleared by its own kernels, so whatever the previous call left
  // in the scratch does not matter
  return moelora_forward_profiled(dims, x, w_gate_up, w_down, a_gate_up, b_gate_up, a_down,
                                  b_down, topk_ids, topk_weights, sorted_slots, bucket_offsets,
                                  out, ws, MOELORA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moelora_forward_profiled(const moelora_dims* dims, const void* x, const void* w_gate_up,
                             const void* w_down, const void* a_gate_up, const void* b_gate_up,
                             const void* a_down, const void* b_down, const int32_t* topk_ids,
                             const float* topk_weights, const int32_t* sorted_slots,
                             const int32_t* bucket_offsets, void* out, void* workspace,
                             size_t workspace_bytes, void* stream, void* const* stage_events) {
  // every sorted row's expert is that of its bucket: topk_ids is not read
  (void)topk_ids;
  int rc = check_dims(dims);
  if (rc != MOELORA_OK) return rc;
  const int64_t T = dims->tokens;
  if (T == 0) return MOELORA_OK;
  const void* ptrs[] = {x, w_gate_up, w_down, a_gate_up, b_gate_up, a_down, b_down,
                        topk_weights, sorted_slots, bucket_offsets, out};
  for (const void* p : ptrs)
    if (p == nullptr) return MOELORA_ERR_NULL;
  const TilePlan plan = make_plan(dims);
  const ForwardLayout L = forward_layout(dims, plan);
  if (workspace == nullptr || workspace_bytes < L.total) return MOELORA_ERR_WORKSPACE;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOELORA_ERR_ALIGNMENT;
  if (!aligned16(workspace)) return MOELORA_ERR_ALIGNMENT;

  // Lad: buckets per expert in bucket_offsets (adapters, + 1 for base-only tokens);
  // plan.nad: the adapters themselves
  const int k = dims->top_k, E = dims->experts, r = dims->rank;
  const int Lad = static_cast<int>(buckets_per_expert(dims));
  const int dt = dims->dtype == MOELORA_BF16 ? moelora::DT_BF16 : moelora::DT_F32;
  const int64_t h = dims->hidden, I = dims->intermediate;
  const int S = static_cast<int>(T * k);
  // grid sizes must fit the launch limits
  const int64_t ntiles_max = (2 * I + 31) / 32;
  if (static_cast<int64_t>(plan.max_mt) * ntiles_max * std::max(plan.ksplit_gu, plan.ksplit_dn) >
          kMaxGrid ||
      static_cast<int64_t>(plan.max_lt) * 2048 > kMaxGrid)
    return MOELORA_ERR_DIMS;

  char* ws = static_cast<char*>(workspace);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* etiles = reinterpret_cast<int32_t*>(ws + L.etiles);
  int4* mtiles = reinterpret_cast<int4*>(ws + L.mtiles);
  int4* ltiles = reinterpret_cast<int4*>(ws + L.ltiles);
  float* G = reinterpret_cast<float*>(ws + L.g);
  float* Z1 = reinterpret_cast<float*>(ws + L.z1);
  float* Z2 = reinterpret_cast<float*>(ws + L.z2);
  void* ACT = ws + L.act;
  float* D = reinterpret_cast<float*>(ws + L.d);
  hipStream_t st = static_cast<hipStream_t>(stream);

  // event i is recorded right before stage i, the last one after the last stage
  auto mark = [&](int i) -> hipError_t {
    if (stage_events == nullptr || stage_events[i] == nullptr) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), st);
  };
  // the prep launch also clears Z1 and Z2 (atomic shrinks)
  const int64_t nzero = plan.det ? 0 : 2ll * S * r;
  // one partials region: the shrinks' (deterministic mode or tall tiles), in
  // deterministic mode the split gate_up GEMM's, and the split down GEMM's
  // (they run one after another)
  float* sparts = plan.shrink_partials ? reinterpret_cast<float*>(ws + L.parts) : nullptr;
  float* parts = plan.det ? reinterpret_cast<float*>(ws + L.parts) : nullptr;
  float* dparts = plan.ksplit_dn > 1 ? reinterpret_cast<float*>(ws + L.parts) : nullptr;
  hipError_t e = mark(MOELORA_STAGE_PREP);
  if (e == hipSuccess)
    e = moelora::launch_prep(sorted_slots, bucket_offsets, S, E, Lad, plan, pos, mtiles, ltiles,
                             counts, etiles, Z1, nzero, st);
  if (e == hipSuccess) e = mark(MOELORA_STAGE_ZERO);
  if (e == hipSuccess && plan.ksplit_gu > 1 && !plan.det)
    e = moelora::launch_zero(G, static_cast<int64_t>(S) * 2 * I, st);
  // shrinks run before their GEMMs: a fused GEMM epilogue consumes Z
  if (e == hipSuccess) e = mark(MOELORA_STAGE_SHRINK_GATE_UP);
  if (e == hipSuccess)
    e = moelora::launch_shrink(dt, r, plan, x, static_cast<int>(T), sorted_slots, k, a_gate_up, E,
                               Lad, h, Z1, S, ltiles, counts, sparts, st);
  if (e == hipSuccess) e = mark(MOELORA_STAGE_GEMM_GATE_UP);
  if (e == hipSuccess) {
    // the folded down shrink adds into Z2 (cleared by prep), or, deterministic,
    // writes per-N-tile partials that the down-shrink stage sums in order
    const moelora::LoraEpilogue epi{Z1, static_cast<const uint16_t*>(b_gate_up), bucket_offsets,
                                    E, dims->adapters, r, Lad, 2 * I, static_cast<uint16_t*>(ACT),
                                    plan.fold_dn ? static_cast<const uint16_t*>(a_down) : nullptr,
                                    Z2, plan.fold_dn ? parts : nullptr,
                                    static_cast<int64_t>(S) * r};
    e = moelora::launch_gemm(dt, plan, x, static_cast<int>(T), sorted_slots, k, w_gate_up, 2 * I,
                             h, G, S, mtiles, counts, etiles, plan.ksplit_gu,
                             plan.fuse_gu ? &epi : nullptr, parts, st, true,
                             counts + moelora::kQueueBase);
  }
  if (e == hipSuccess) e = mark(MOELORA_STAGE_EXPAND_GATE_UP);
  if (e == hipSuccess && !plan.fuse_gu)
    e = moelora::launch_expand_gate_up(dt, r, plan, Z1, b_gate_up, E, Lad, G, ACT, I, ltiles,
                                       counts, st);
  if (e == hipSuccess) e = mark(MOELORA_STAGE_SHRINK_DOWN);
  if (e == hipSuccess && !plan.fold_dn)
    e = moelora::launch_shrink(dt, r, plan, ACT, S, nullptr, 1, a_down, E, Lad, I, Z2, S, ltiles,
                               counts, sparts, st);
  if (e == hipSuccess && plan.fold_dn && plan.det)
    e = moelora::launch_reduce_parts(parts, static_cast<int>(gate_up_ntiles(dims, plan)),
                                     static_cast<int64_t>(S) * r, Z2, st);
  if (e == hipSuccess) e = mark(MOELORA_STAGE_GEMM_DOWN);
  // split K: every split stores its partial plane (no atomics, no clearing),
  // the expand adds into plane 0 and the combine sums the planes in order
  float* Dn = plan.ksplit_dn > 1 ? dparts : D;
  if (e == hipSuccess) {
    const moelora::LoraEpilogue epi{Z2, static_cast<const uint16_t*>(b_down), bucket_offsets,
                                    E, dims->adapters, r, Lad, h, nullptr};
    e = moelora::launch_gemm(dt, plan, ACT, S, nullptr, 1, w_down, h, I, D, S, mtiles, counts,
                             etiles, plan.ksplit_dn, plan.fuse_dn ? &epi : nullptr, dparts, st,
                             false, counts + moelora::kQueueBase + moelora::kXcds);
  }
  if (e == hipSuccess) e = mark(MOELORA_STAGE_EXPAND_DOWN);
  if (e == hipSuccess && !plan.fuse_dn)
    e = moelora::launch_expand_down(dt, r, plan, Z2, b_down, E, Lad, Dn, h, ltiles, counts, st);
  if (e == hipSuccess) e = mark(MOELORA_STAGE_COMBINE);
  if (e == hipSuccess)
    e = moelora::launch_combine(dt, Dn, pos, topk_weights, static_cast<int>(T), k, h, out, st,
                                plan.ksplit_dn);
  if (e == hipSuccess) e = mark(MOELORA_NUM_STAGES);
  return hip_status(e);
}

int moelora_dense_workspace_size(const moelora_dense_dims* dims, size_t* bytes) {
  moelora_dims m;
  const int rc = dense_check(dims, &m);
  if (rc != MOELORA_OK) return rc;
  if (bytes == nullptr) return MOELORA_ERR_NULL;
  *bytes = m.tokens == 0 ? 0 : dense_layout(&m, make_plan(&m)).total;
  return MOELORA_OK;
}

int moelora_dense_forward(const moelora_dense_dims* dims, const void* x, const void* w,
                          const void* a, const void* b, const int32_t* adapter_ids, void* out,
                          int32_t* device_status, void* workspace, size_t workspace_bytes,
                          void* stream) {
  moelora_dims m;
  int rc = dense_check(dims, &m);
  if (rc != MOELORA_OK) return rc;
  const int64_t T = m.tokens;
  if (T == 0) return MOELORA_OK;
  const void* ptrs[] = {x, w, a, b, adapter_ids, out};
  for (const void* p : ptrs)
    if (p == nullptr) return MOELORA_ERR_NULL;
  const TilePlan plan = make_plan(&m);
  const DenseLayout L = dense_layout(&m, plan);
  if (workspace == nullptr || workspace_bytes < L.total) return MOELORA_ERR_WORKSPACE;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOELORA_ERR_ALIGNMENT;
  if (!aligned16(workspace)) return MOELORA_ERR_ALIGNMENT;
  const int64_t N = m.hidden, K = m.intermediate;
  const int r = m.rank, nad = m.adapters, Lb = static_cast<int>(buckets_per_expert(&m));
  const int dt = m.dtype == MOELORA_BF16 ? moelora::DT_BF16 : moelora::DT_F32;
  const int S = static_cast<int>(T);
  const int64_t ntiles_max = (N + 31) / 32;
  if (static_cast<int64_t>(plan.max_mt) * ntiles_max * plan.ksplit_dn > kMaxGrid ||
      static_cast<int64_t>(plan.max_lt) * 2048 > kMaxGrid)
    return MOELORA_ERR_DIMS;

  char* ws = static_cast<char*>(workspace);
  int32_t* ws_key = reinterpret_cast<int32_t*>(ws + L.key);
  int32_t* ws_rank = reinterpret_cast<int32_t*>(ws + L.rank);
  int32_t* ws_cnt = reinterpret_cast<int32_t*>(ws + L.cnt);
  int32_t* slots = reinterpret_cast<int32_t*>(ws + L.slots);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* etiles = reinterpret_cast<int32_t*>(ws + L.etiles);
  int4* mtiles = reinterpret_cast<int4*>(ws + L.mtiles);
  int4* ltiles = reinterpret_cast<int4*>(ws + L.ltiles);
  float* Z = reinterpret_cast<float*>(ws + L.z);
  float* D = reinterpret_cast<float*>(ws + L.d);
  float* sparts = plan.shrink_partials ? reinterpret_cast<float*>(ws + L.parts) : nullptr;
  float* dparts = plan.ksplit_dn > 1 ? reinterpret_cast<float*>(ws + L.parts) : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);

  // tokens bucketed by adapter (one expert, k = 1)
  hipError_t e = moelora::launch_align(nullptr, nullptr, adapter_ids, S, 1, 1, nad, Lb, nullptr,
                                       nullptr, slots, offsets, device_status, ws_key, ws_rank,
                                       ws_cnt, st);
  const int64_t nzero = plan.det ? 0 : static_cast<int64_t>(S) * r;
  if (e == hipSuccess)
    e = moelora::launch_prep(slots, offsets, S, 1, Lb, plan, pos, mtiles, ltiles, counts, etiles, Z,
                             nzero, st);
  if (e == hipSuccess)
    e = moelora::launch_shrink(dt, r, plan, x, S, slots, 1, a, 1, Lb, K, Z, S, ltiles, counts,
                               sparts, st);
  if (e == hipSuccess) {
    const moelora::LoraEpilogue epi{Z, static_cast<const uint16_t*>(b), offsets, 1, nad, r, Lb, N,
                                    nullptr};
    e = moelora::launch_gemm(dt, plan, x, S, slots, 1, w, N, K, D, S, mtiles, counts, etiles,
                             plan.ksplit_dn, plan.fuse_dn ? &epi : nullptr, dparts, st, false,
                             counts + moelora::kQueueBase + moelora::kXcds);
  }
  // split K: partial planes, the expand into plane 0, the ordered sum in the combine
  float* Dn = plan.ksplit_dn > 1 ? dparts : D;
  if (e == hipSuccess && !plan.fuse_dn)
    e = moelora::launch_expand_down(dt, r, plan, Z, b, 1, Lb, Dn, N, ltiles, counts, st);
  if (e == hipSuccess)
    e = moelora::launch_combine(dt, Dn, pos, nullptr, S, 1, N, out, st, plan.ksplit_dn);
  return hip_status(e);
}

}  // extern "C"
