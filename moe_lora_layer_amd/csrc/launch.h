// Internal launchers of the gfx950 kernels (host side).  Every launcher only
// enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moelora {

enum { DT_F32 = 0, DT_BF16 = 1 };

// LDS ints available to the align kernel's per-chunk bucket counters and,
// when they fit, the per-slot keys and ranks (144 KiB of the 160 KiB a gfx950
// workgroup may use).
constexpr int kAlignLdsInts = 36864;
// Where the align kernel keeps its per-chunk bucket counters and per-slot
// keys and ranks for nb buckets and S slots; cnt_ints = counters it needs in
// the workspace (0 when they live in LDS).
struct AlignLayout {
  bool cnt_lds, keys_lds;
  int chunks;
  int64_t cnt_ints;
};
AlignLayout align_layout(int nb, int S);

// logits == nullptr: the expert ids come from ids_in (no routing, topk_ids and
// topk_w untouched); ids_in == nullptr too: every slot goes to expert 0.
// L adapters; Lb buckets per expert (L, or L + 1 when adapter id -1 marks a
// base-only token, keyed to bucket L of its expert).
// ws_key and ws_rank hold S ints each; ws_cnt align_layout(E * Lb, T * k).cnt_ints
// (may be nullptr when that is 0).
hipError_t launch_align(const float* logits, const int32_t* ids_in, const int32_t* adapter_ids,
                        int T, int E, int k, int L, int Lb, int32_t* topk_ids, float* topk_w,
                        int32_t* sorted_slots, int32_t* offsets, int32_t* status, int32_t* ws_key,
                        int32_t* ws_rank, int32_t* ws_cnt, hipStream_t stream);

constexpr int kXcds = 8;  // XCDs of an MI355X
// counts[] in the forward workspace: [0] M-tiles, [1] LoRA tiles, then from
// kQueueBase the tile-queue counters of the persistent GEMM launches (kXcds
// for gate_up, kXcds for down), cleared by the prep launch
constexpr int kQueueBase = 4;
constexpr int kCountsInts = kQueueBase + 2 * kXcds;

// Workgroup order of the base GEMMs (moelora_plan.order): launch order, the
// expert's tiles grouped per XCD, every workgroup's K walk rotated, or both.
enum { ORDER_LAUNCH = 1, ORDER_XCD = 2, ORDER_ROTATED = 3, ORDER_XCD_ROTATED = 4, ORDER_XCD_STAGGERED = 5 };
// ORDER_XCD_STAGGERED: M-tile m of an expert (counted from the expert's first)
// starts its K walk kOrderStagger * m steps in
constexpr int kOrderStagger = 2;
__host__ __device__ constexpr bool order_xcd(int order) {
  return order == ORDER_XCD || order == ORDER_XCD_ROTATED || order == ORDER_XCD_STAGGERED;
}

// Tile descriptor: x = expert (M-tiles) or bucket (LoRA tiles), y = first
// sorted row, z = end row (exclusive), w unused.
struct TilePlan {
  int bm;        // rows per M-tile of the base GEMMs
  int bml;       // rows per LoRA tile
  int max_mt;    // upper bound of M-tiles, known on the host
  int max_lt;    // upper bound of LoRA tiles
  bool stream;   // weight tiles are used by one M-tile only: stream them
  bool dma128;   // bf16, bm 128: the 128 x 256 DMA tiles (three LDS stages)
  int ksplit_gu; // K splits of the gate_up GEMM (1 = none)
  int ksplit_dn; // K splits of the down GEMM (1 = none)
  bool lora_db;  // LoRA tiles average many rows: double-buffer their row blocks
  bool fuse_gu;  // gate_up GEMM applies the LoRA expand and SiLU-mul in its epilogue
  bool fuse_dn;  // down GEMM applies the LoRA expand in its epilogue
  bool det;      // split-K reductions go through ordered partial sums, not atomics
  bool shrink_partials;  // the shrinks sum per-split partials in order (det, or tall bf16 tiles)
  int nad;       // adapters; bucket index nad of an expert (base-only tokens) has no LoRA
  bool kn;       // every weight is k-major ([K][N], the h_in x h_out orientation)
  bool fold_dn;  // the down shrink runs in the fused gate_up GEMM's epilogue
  int order;     // ORDER_*: workgroup order of the base GEMMs
};

// Operands of the LoRA expand fused into a base GEMM's epilogue:
// acc[p][n] += z[p] . b[l][e][n] for the rows p of bucket (e, l).
// act == nullptr: down form (the GEMM writes D); otherwise gate_up form
// (the GEMM writes act[p][i] = SiLU(g) * u in bf16, intermediate width N/2).
struct LoraEpilogue {
  const float* z;           // [S][rank] fp32, sorted order
  const uint16_t* b;        // [L][E][b_rows][rank] bf16
  const int32_t* offsets;   // bucket_offsets [E*buckets + 1]
  int experts, adapters, rank;
  int buckets;              // buckets per expert (adapters, + 1 with base-only tokens)
  int64_t b_rows;           // rows of each B block (2I for gate_up, h for down)
  uint16_t* act;            // bf16 [S][I] output of the gate_up form, else nullptr
  // gate_up form only: the down projection's shrink z2 = act . A_dn folded
  // into the epilogue (dn_a == nullptr: not folded).  Each tile adds its
  // columns' share of z2 to dn_z with relaxed fp32 atomics (dn_z zero
  // beforehand), or, dn_parts != nullptr (deterministic), writes it to
  // partial slot nt (its N-tile) at dn_parts + nt * dn_part_stride.
  const uint16_t* dn_a;     // A_dn [L][E][r][I] bf16 (k-major: [L][E][I][r])
  float* dn_z;              // [S][rank] fp32
  float* dn_parts;
  int64_t dn_part_stride;
};

// Inverse permutation pos[slot] = sorted position, the M-tile list (tiles of
// plan.bm rows per expert, in expert order) with expert_tiles[e] = first tile
// of expert e (expert_tiles[E] = tile count), and the LoRA tile list; the same
// launch clears zero[0, zero_n) (a multiple of 4 floats).
hipError_t launch_prep(const int32_t* sorted_slots, const int32_t* offsets, int S, int E, int L,
                       const TilePlan& plan, int32_t* pos, int4* mtiles, int4* ltiles,
                       int32_t* counts, int32_t* expert_tiles, float* zero, int64_t zero_n,
                       hipStream_t stream);

hipError_t launch_zero(float* p, int64_t n, hipStream_t stream);

// C[p][n] = sum_k X[row(p)][k] * Wt[e][n][k] over the M-tiles of `mtiles`;
// row(p) = gather_slots[p] / gather_k when gather_slots != nullptr, else p,
// clamped to [0, x_rows).  ksplit > 1 splits K over workgroups that add into
// C with fp32 atomics (C must be zero beforehand).  lora != nullptr fuses the
// LoRA expand (and for gate_up the SiLU-mul) into the epilogue; only the bf16
// 256-row plan with ksplit == 1 has it (hipErrorInvalidValue otherwise).
// parts != nullptr (ksplit > 1): split s writes its partial tile to
// parts + s * c_rows * N with plain stores and, when sum_parts, a second launch
// sums them into C in split order (C needs no clearing then); without
// sum_parts the caller consumes the partials.  queue != nullptr: kXcds
// counters, zero beforehand, for the 256- and 128-row bf16 tiles' persistent
// launch (one workgroup per CU taking tiles from per-XCD queues).
hipError_t launch_gemm(int dtype, const TilePlan& plan, const void* X, int x_rows,
                       const int32_t* gather_slots, int gather_k, const void* Wt, int64_t N,
                       int64_t K, float* C, int64_t c_rows, const int4* mtiles,
                       const int32_t* counts, const int32_t* expert_tiles, int ksplit,
                       const LoraEpilogue* lora, float* parts, hipStream_t stream,
                       bool sum_parts = true, int32_t* queue = nullptr);

// out[i] = sum over p < nparts, in order, of parts[p * n + i] (n a multiple of 4).
hipError_t launch_reduce_parts(const float* parts, int nparts, int64_t n, float* out,
                               hipStream_t stream);

// Z[p][q] += sum_k X[row(p)][k] * At[l][e][q][k] over the LoRA tiles (split-K,
// fp32 atomics; Z must be zero beforehand).  parts != nullptr (deterministic
// mode): every split writes its partial to parts + s * S * rank and a second
// launch sums them into Z in split order (Z needs no clearing then);
// shrink_parts() is the number of partials, known on the host.
hipError_t launch_shrink(int dtype, int rank, const TilePlan& plan, const void* X, int x_rows,
                         const int32_t* gather_slots, int gather_k, const void* At, int E, int L,
                         int64_t K, float* Z, int S, const int4* ltiles, const int32_t* counts,
                         float* parts, hipStream_t stream);
int shrink_parts(int dtype, int rank, const TilePlan& plan, int64_t K);

// gate_up expand + base add + SiLU-mul:
// ACT[p][i] = SiLU(G[p][i] + Z[p].Bt[i]) * (G[p][I+i] + Z[p].Bt[I+i]).
hipError_t launch_expand_gate_up(int dtype, int rank, const TilePlan& plan, const float* Z,
                                 const void* Bt, int E, int L, const float* G, void* ACT,
                                 int64_t I, const int4* ltiles, const int32_t* counts,
                                 hipStream_t stream);

// down expand added in place: D[p][n] += Z[p].Bt[n].
hipError_t launch_expand_down(int dtype, int rank, const TilePlan& plan, const float* Z,
                              const void* Bt, int E, int L, float* D, int64_t h,
                              const int4* ltiles, const int32_t* counts, hipStream_t stream);

// out[t] = sum_j w[t][j] * D[pos[t*k + j]] in j order (w == nullptr: weights 1),
// D[p] being the sum, in order, of nparts planes of [T*k][h] (the partials of
// a split down GEMM).
hipError_t launch_combine(int dtype, const float* D, const int32_t* pos, const float* w, int T,
                          int k, int64_t h, void* out, hipStream_t stream, int nparts = 1);

}  // namespace moelora