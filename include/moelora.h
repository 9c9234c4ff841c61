/*
 * moelora.h -- C ABI of the fused MoE multi-LoRA layer for AMD MI355X (gfx950).
 *
 * The layer is the one described on the vLLM blog page "Multi-LoRA"
 * (vllm.com.cn/blog/multi-lora), section "Implementing Multi-LoRA inference for
 * MoE models in vLLM" and Fig. 1:
 *   - a router sends each token to its top-k experts and the expert outputs are
 *     combined with the routing weights;
 *   - each expert runs a gate_up projection (h -> 2I) and a down projection
 *     (I -> h) with SiLU(gate) * up in between;
 *   - every projection with frozen weight W (h_in x h_out) carries the LoRA
 *     adapter of the token's request, A (h_in x r) and B (r x h_out), and
 *     computes y = xW + (xA)B: a shrink z = xA and an expand zB;
 *   - LoRA weights exist per (adapter, expert), so each expert runs four LoRA
 *     ops and two sparsities compound: expert routing and adapter choice.
 *
 * Two calls make one layer step:
 *   moelora_align   routing + the (expert, adapter)-bucketed slot permutation
 *   moelora_forward base grouped GEMMs, LoRA shrink/expand, SiLU-mul, combine
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers (hipMalloc / torch allocations on the
 *     current device), row-major, contiguous, 16-byte aligned.
 *   - Weights are K-contiguous by default: each array holds its matrix
 *     TRANSPOSED, i.e. row n of the array is column n of the page's h_in x h_out
 *     matrix.  With MOELORA_FLAG_IN_OUT they are h_in x h_out as the page writes
 *     them (see there).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it: no host synchronisation, no allocation, no host reads of
 *     device memory.  The caller keeps every buffer alive until the stream has
 *     executed the work.  Calls are reentrant; concurrent calls need distinct
 *     outputs and workspaces.
 *   - Inputs are never written.  The library keeps no state between calls,
 *     except the static scratch of moelora_forward_noalloc (see there).
 *   - Errors are returned as a moelora_status code before anything is
 *     enqueued (argument errors) or right after the launches (MOELORA_ERR_HIP).
 *     No C++ exception crosses this boundary.
 */
#ifndef MOELORA_H
#define MOELORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOELORA_ABI_VERSION 8

typedef enum moelora_status {
  MOELORA_OK = 0,
  MOELORA_ERR_NULL = 1,         /* a required pointer is NULL                            */
  MOELORA_ERR_DIMS = 2,         /* a dimension is out of range                           */
  MOELORA_ERR_UNSUPPORTED = 3,  /* dtype or rank not supported                           */
  MOELORA_ERR_ALIGNMENT = 4,    /* a tensor pointer is not 16-byte aligned               */
  MOELORA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than *_workspace_size       */
  MOELORA_ERR_HIP = 6,          /* the HIP runtime reported an error at launch           */
  MOELORA_ERR_TOO_LARGE = 7     /* moelora_forward_noalloc: the call needs more than its
                                   static scratch (MOELORA_NOALLOC_SCRATCH_BYTES)         */
} moelora_status;

typedef enum moelora_dtype {
  MOELORA_F32 = 0,   /* x, weights and out in float32                                    */
  MOELORA_BF16 = 1   /* x, weights and out in bfloat16; accumulation is always float32   */
} moelora_dtype;

/*
 * Tile plan of moelora_forward and moelora_dense_forward: the per-shape
 * kernel configuration (tile sizes, split-K) that the vLLM blog page
 * "Multi-LoRA" (section "Kernel configuration tuning for Amazon SageMaker AI
 * and Amazon Bedrock") tunes offline and lets users load from their own
 * tuned configuration files; moe_lora_layer_amd.tune writes such a table for
 * this library.  Every field 0
 * means the library's automatic choice for that field; the result is the same
 * within the layer's tolerance for any valid plan, only the speed differs.
 *   gemm_rows       rows per M-tile of the base grouped GEMMs: 32, 64, 128, 256
 *   gemm_form       1 weight-streaming tiles (32, 64 or 128 rows: nontemporal
 *                   weight loads, rotated K walk), 2 weight-reuse tiles (128 or
 *                   256 rows), 3 (bf16, 128 rows) weight-streaming tiles of
 *                   128 x 256 outputs whose operands go straight into three LDS
 *                   stages; needs gemm_rows set
 *                   (MOELORA_ERR_UNSUPPORTED otherwise, and for 3 with fp32)
 *   lora_rows       rows per LoRA tile: 16 (one MFMA block, for buckets of few
 *                   rows) or 64 (tall tiles)
 *   ksplit_gate_up  K splits of the gate_up GEMM (fp32 atomics, or ordered
 *                   partials with MOELORA_FLAG_DETERMINISTIC), 1..1024; rounded
 *                   down to a count whose K ranges are all non-empty
 *   ksplit_down     the same for the down GEMM (the dense projection's GEMM),
 *                   whose splits always store partials that the combine pass
 *                   sums in split order (deterministic with or without the flag)
 *   fuse            1: every projection whose GEMM can (bf16, unsplit K) runs
 *                   its LoRA expand in the GEMM epilogue; 2: none does; 3: as
 *                   1, and the fused gate_up epilogue also computes the down
 *                   projection's LoRA shrink (MOELORA_FUSED_DOWN_SHRINK; never
 *                   the automatic choice: slower on MI355X at every shape
 *                   measured, kept for callers whose ACT re-read costs more)
 *   order           workgroup order of the base GEMMs (the page's CTA
 *                   swizzling for L2 reuse, section "Kernel optimisation"):
 *                   1 launch order; 2 each expert's tiles N-tile by N-tile,
 *                   M-tiles innermost, remapped so that every XCD (one L2)
 *                   runs a contiguous run of them; 3 launch order with every
 *                   workgroup's K walk starting at its own step (rotated), so
 *                   that resident workgroups stream different K columns; 4 both;
 *                   5 as 2, with the M-tiles of an expert starting their K walks
 *                   2 steps apart per M-tile (the tiles sharing a weight tile
 *                   then read each weight step from L2 after the first)
 *                   (automatic: 2 for the weight-reuse tiles and form 3, 3
 *                   for the other weight-streaming ones, 1 for those over
 *                   MOELORA_FLAG_IN_OUT weights)
 * The K step of every GEMM tile is fixed at 64 bf16 / 32 fp32 elements (one
 * 128-byte LDS row); it is not a plan field.
 * Out-of-range values make every call that takes the dims return
 * MOELORA_ERR_UNSUPPORTED.
 */
typedef struct moelora_plan {
  int32_t gemm_rows;
  int32_t gemm_form;
  int32_t lora_rows;
  int32_t ksplit_gate_up;
  int32_t ksplit_down;
  int32_t fuse;
  int32_t order;
} moelora_plan;

/*
 * Layer dimensions.  Limits (checked, MOELORA_ERR_DIMS / _UNSUPPORTED otherwise):
 *   tokens T >= 0 (T == 0 is a no-op), T * top_k < 2^31
 *   hidden h and intermediate I: positive multiples of 64
 *   experts E >= 1, 1 <= top_k <= min(E, 8), adapters L >= 1, E * L <= 65536
 *   rank r in {16, 32, 64}
 */
typedef struct moelora_dims {
  int64_t tokens;        /* T                                                       */
  int64_t hidden;        /* h: gate_up input width, down output width               */
  int64_t intermediate;  /* I: gate_up produces 2I columns, [gate | up]             */
  int32_t experts;       /* E                                                       */
  int32_t top_k;         /* k                                                       */
  int32_t adapters;      /* L: adapters resident at once                            */
  int32_t rank;          /* r                                                       */
  int32_t dtype;         /* moelora_dtype                                           */
  int32_t flags;         /* 0, or any of MOELORA_FLAG_*                              */
  moelora_plan plan;     /* all 0: automatic                                        */
} moelora_dims;

/*
 * MOELORA_FLAG_DETERMINISTIC: every split-K reduction (the LoRA shrinks, and
 * the gate_up GEMM when its K is split because the output is narrow) writes
 * one fp32 partial per split to the forward workspace and a separate pass sums
 * the partials in split order, instead of relaxed fp32 atomics (a split down
 * GEMM does so in every mode, its partials summed by the combine pass); and the
 * 256-row down GEMM gives up its stream-K pass (the last, partial round of
 * tiles cut into K ranges whose parts are added with atomics).  The output is
 * then bit-identical from run to run for the same inputs and dims (without the
 * flag the atomics' order varies, within the layer's tolerance).  The forward
 * workspace grows by the partials (moelora_forward_workspace_size accounts for
 * it).
 */
#define MOELORA_FLAG_DETERMINISTIC 1

/*
 * MOELORA_FLAG_BASE_ONLY: a token may carry adapter id -1, meaning the base
 * model without any adapter (the Multi-LoRA page does not cover it; the
 * reading taken is that such a token has no LoRA term in either projection,
 * exactly as if its B were zero).  Every expert then has Lb = L + 1 buckets,
 * its base-only slots in the last one: bucket_offsets has E * (L + 1) + 1
 * entries (E * L + 1 without the flag); E * L <= 65536 still holds.
 */
#define MOELORA_FLAG_BASE_ONLY 2

/*
 * MOELORA_FLAG_UNFUSED: moelora_forward runs every LoRA expand as a kernel of
 * its own after the base GEMM instead of inside the GEMM's epilogue, so that
 * the base output G is left in the workspace for layer-by-layer reconciliation
 * (moelora_forward_workspace_layout).  The result is the same within the
 * layer's tolerance; the fused form is faster.  Ignored by moelora_align.
 */
#define MOELORA_FLAG_UNFUSED 4

/*
 * MOELORA_FLAG_IN_OUT: every weight is stored as the Multi-LoRA page writes it
 * (section "Implementing Multi-LoRA inference for MoE models in vLLM": W is
 * h_in x h_out, A is h_in x r, B is r x h_out), row-major:
 *   moelora_forward:        w_gate_up [E][h][2I]   w_down [E][I][h]
 *                           a_gate_up [L][E][h][r] b_gate_up [L][E][r][2I]
 *                           a_down    [L][E][I][r] b_down    [L][E][r][h]
 *   moelora_dense_forward:  w [K][N], a [L][K][r], b [L][r][N]
 * instead of the default K-contiguous (transposed) arrays.  Same result within
 * the layer's tolerance.  The kernels read these arrays as they are: bf16
 * operands that pass through LDS (copied straight in, or stored from
 * registers as loaded) stay k-major there and are read with the transposing
 * LDS loads of gfx950; operands loaded straight into MFMA fragments (the LoRA
 * shrink and expand kernels) and fp32 tiles are transposed across lanes in
 * registers.  The default layout is the faster one for weight-streaming
 * (decode-sized) batches.
 */
#define MOELORA_FLAG_IN_OUT 8

int moelora_abi_version(void);

/* Static string for a status code (never NULL). */
const char* moelora_status_string(int status);

/* Bytes of device workspace moelora_align needs for these dimensions. */
int moelora_align_workspace_size(const moelora_dims* dims, size_t* bytes);

/*
 * moelora_align -- routing and the (expert, adapter)-bucketed permutation.
 *
 * Routing (same page, section "Implementing Multi-LoRA inference for MoE
 * models in vLLM": the router picks the most relevant experts per token): for
 * each token t, the k experts with the largest logits in descending logit order
 * (exact float comparison, ties to the lower expert id), and weights equal to
 * the softmax over all E logits restricted to those k and renormalised to sum
 * to one (computed as exp(l_j - l_max) / sum over the kept j, in float32).
 *
 * Permutation (the compound sparsity of expert routing and adapter choice,
 * same section): slot s = t*k + j has key topk_ids[s] * L + adapter_ids[t].
 * sorted_slots is the stable sort of all slots by key; bucket_offsets[b] is the
 * number of slots with key < b.  Both are deterministic and bit-exact.
 *
 *   router_logits  in  float [T][E]
 *   adapter_ids    in  int32 [T], each in [0, L) (or -1 with MOELORA_FLAG_BASE_ONLY)
 *   topk_ids       out int32 [T][k]
 *   topk_weights   out float [T][k]
 *   sorted_slots   out int32 [T*k]
 *   bucket_offsets out int32 [E*Lb + 1]  (Lb = L, or L + 1 with MOELORA_FLAG_BASE_ONLY;
 *                  bucket_offsets[E*Lb] = T*k; a base-only token's key is
 *                  topk_ids[s] * Lb + L)
 *   device_status  out int32 [1] or NULL: 0 = ok, 1 = an adapter id was outside
 *                  [0, L) (it was treated as 0; the outputs are then unspecified).
 *                  Read it after the stream has executed the call.
 *   workspace      device scratch of at least moelora_align_workspace_size bytes
 */
int moelora_align(const moelora_dims* dims, const float* router_logits,
                  const int32_t* adapter_ids, int32_t* topk_ids, float* topk_weights,
                  int32_t* sorted_slots, int32_t* bucket_offsets, int32_t* device_status,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * moelora_align_topk -- the permutation of moelora_align for a caller that
 * routes itself (its router GEMM and top-k run just before this path):
 * topk_ids is an input and no routing weight is computed (the caller passes
 * its own to moelora_forward).  Keys, sorted_slots and bucket_offsets are
 * exactly those of moelora_align for the same ids; repeated ids within a token
 * are allowed (each slot is an independent row).
 *
 *   topk_ids       in  int32 [T][k], each in [0, E)
 *   adapter_ids    in  int32 [T], each in [0, L)
 *   sorted_slots, bucket_offsets, workspace: as moelora_align
 *   device_status  out int32 [1] or NULL: 0 = ok, 1 = an adapter id outside
 *                  [0, L), 3 = an expert id outside [0, E) (either treated as 0,
 *                  the outputs then unspecified; the larger code is reported).
 */
int moelora_align_topk(const moelora_dims* dims, const int32_t* topk_ids,
                       const int32_t* adapter_ids, int32_t* sorted_slots,
                       int32_t* bucket_offsets, int32_t* device_status, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Bytes of device workspace moelora_forward needs for these dimensions. */
int moelora_forward_workspace_size(const moelora_dims* dims, size_t* bytes);

/*
 * moelora_forward -- the layer for every slot, then the weighted combination.
 *
 * For each slot s (token t, expert e = its bucket's expert, adapter l = its
 * bucket's adapter), following the page's section "Implementing Multi-LoRA
 * inference for MoE models in vLLM" (the expert MLP, y = xW + xAB, shrink and
 * expand, four LoRA ops per expert) and section "Kernel optimisation" (split-K
 * shrink with relaxed atomics, the LoRA add fused with the base add):
 *   g = x_t W_gu[e] + (x_t A_gu[l][e]) B_gu[l][e]          (2I columns)
 *   a = SiLU(g[0:I]) * g[I:2I],  SiLU(v) = v / (1 + exp(-v))
 *   d = a W_dn[e] + (a A_dn[l][e]) B_dn[l][e]              (h columns)
 *   out[t] = sum_{j<k} topk_weights[t][j] * d(slot t*k+j), summed in j order
 * The activation a is rounded to the layer dtype before the down projection;
 * every sum is accumulated in float32.  Split-K atomics make the low bits of
 * out vary from run to run.
 *
 *   x          in  [T][h]
 *   w_gate_up  in  [E][2I][h]      (W_gu^T; rows [0,I) gate, [I,2I) up)
 *   w_down     in  [E][h][I]       (W_dn^T)
 *   a_gate_up  in  [L][E][r][h]    (A_gu^T)
 *   b_gate_up  in  [L][E][2I][r]   (B_gu^T)
 *   a_down     in  [L][E][r][I]    (A_dn^T)
 *   b_down     in  [L][E][h][r]    (B_dn^T)
 *              (with MOELORA_FLAG_IN_OUT the untransposed matrices:
 *              [E][h][2I], [E][I][h], [L][E][h][r], [L][E][r][2I],
 *              [L][E][I][r], [L][E][r][h]; columns [0,I) of W_gu and B_gu gate)
 *   topk_ids   in  int32 [T][k] as produced by moelora_align (or the caller's own
 *              ids given to moelora_align_topk), or NULL: the ids the
 *              permutation was built from.  No kernel reads them: every
 *              sorted row takes the expert (and adapter) of its bucket in
 *              bucket_offsets.  Passing align's outputs unchanged is the
 *              intended use.
 *   topk_weights, sorted_slots, bucket_offsets: as produced by moelora_align
 *              (any stable bucketed permutation of the same keys is valid)
 *   out        out [T][h], fully overwritten
 *   workspace  device scratch of at least moelora_forward_workspace_size bytes;
 *              its contents after the call are the intermediates described by
 *              moelora_forward_workspace_layout.
 */
int moelora_forward(const moelora_dims* dims, const void* x, const void* w_gate_up,
                    const void* w_down, const void* a_gate_up, const void* b_gate_up,
                    const void* a_down, const void* b_down, const int32_t* topk_ids,
                    const float* topk_weights, const int32_t* sorted_slots,
                    const int32_t* bucket_offsets, void* out, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * moelora_forward_noalloc -- moelora_forward for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The arguments and the result are those of
 * moelora_forward without the workspace: the call runs in a static device
 * array of MOELORA_NOALLOC_SCRATCH_BYTES that the library holds, one per GPU
 * it runs on, from the first call on that GPU until the process ends.  It
 * calls no hipMalloc, hipFree or other allocating routine.
 *   - Dims whose moelora_forward_workspace_size exceeds the scratch are refused
 *     with MOELORA_ERR_TOO_LARGE before anything is enqueued (64 MiB holds every
 *     decode-sized batch, e.g. 64 tokens at h 4096, I 11008, or 256 tokens at
 *     h 2880, I 2880 over 32 experts top-4; a 4096-token prefill at h 4096,
 *     I 11008 needs ~0.35 GiB and goes through moelora_forward).
 *   - Every call on one GPU shares that GPU's scratch and finds in it what the
 *     previous call left (the kernels clear what must start at zero), so calls
 *     that overlap on one GPU (other streams, other threads) race: the caller
 *     serialises them.
 *   - The first call on a GPU looks up the scratch's device address with
 *     hipGetSymbolAddress (MOELORA_ERR_HIP if that fails) and keeps it.
 */
#define MOELORA_NOALLOC_SCRATCH_BYTES (64u << 20)
int moelora_forward_noalloc(const moelora_dims* dims, const void* x, const void* w_gate_up,
                            const void* w_down, const void* a_gate_up, const void* b_gate_up,
                            const void* a_down, const void* b_down, const int32_t* topk_ids,
                            const float* topk_weights, const int32_t* sorted_slots,
                            const int32_t* bucket_offsets, void* out, void* stream);

/*
 * Stages of moelora_forward, in launch order (one kernel each).
 */
enum moelora_stage {
  MOELORA_STAGE_PREP = 0,        /* inverse permutation, tile lists, clear the shrink
                                    accumulators                                     */
  MOELORA_STAGE_ZERO = 1,        /* clear the gate_up output when its GEMM is split
                                    over K (empty otherwise)                          */
  MOELORA_STAGE_SHRINK_GATE_UP = 2,
  MOELORA_STAGE_GEMM_GATE_UP = 3,    /* bf16 with unsplit K: also the LoRA expand and
                                        the SiLU-mul (moelora_forward_fusion)         */
  MOELORA_STAGE_EXPAND_GATE_UP = 4,  /* + base add + SiLU-mul; empty when fused       */
  MOELORA_STAGE_SHRINK_DOWN = 5,
  MOELORA_STAGE_GEMM_DOWN = 6,       /* fused LoRA expand under the same condition   */
  MOELORA_STAGE_EXPAND_DOWN = 7,     /* empty when fused                              */
  MOELORA_STAGE_COMBINE = 8,
  MOELORA_NUM_STAGES = 9
};

/*
 * moelora_forward with per-stage timing for profilers and benchmarks.
 * stage_events: NULL, or MOELORA_NUM_STAGES + 1 hipEvent_t handles created by
 * the caller (any of them may be NULL: that boundary is not recorded); event i
 * is recorded on `stream` before stage i is launched and event
 * MOELORA_NUM_STAGES after the last stage, so the elapsed time between events
 * i and i+1 is the duration of stage i.  Each recorded event adds a small gap
 * on the stream.  Everything else is identical to moelora_forward (which is
 * this call with stage_events == NULL).
 */
int moelora_forward_profiled(const moelora_dims* dims, const void* x, const void* w_gate_up,
                             const void* w_down, const void* a_gate_up, const void* b_gate_up,
                             const void* a_down, const void* b_down, const int32_t* topk_ids,
                             const float* topk_weights, const int32_t* sorted_slots,
                             const int32_t* bucket_offsets, void* out, void* workspace,
                             size_t workspace_bytes, void* stream, void* const* stage_events);

/*
 * Debug aid for layer-by-layer reconciliation: byte offsets, inside the forward
 * workspace, of the intermediates left there by moelora_forward, all indexed by
 * sorted position p (row p belongs to slot sorted_slots[p]):
 *   offsets[0]  G   float [T*k][2I]  gate_up base output xW (before the LoRA add);
 *                                    when the gate_up GEMM fuses the expand
 *                                    (moelora_forward_fusion; never with
 *                                    MOELORA_FLAG_UNFUSED) G is neither written
 *                                    nor given any workspace bytes
 *   offsets[1]  Z1  float [T*k][r]   gate_up shrink xA (the rows of base-only
 *                                    slots, MOELORA_FLAG_BASE_ONLY, are
 *                                    unspecified, as are those of Z2: no LoRA
 *                                    term reads them)
 *   offsets[2]  ACT dtype [T*k][I]   SiLU(gate) * up, including both LoRA terms
 *   offsets[3]  Z2  float [T*k][r]   down shrink a A
 *   offsets[4]  D   float [T*k][h]   down output including its LoRA term
 */
int moelora_forward_workspace_layout(const moelora_dims* dims, size_t offsets[5]);

/*
 * Which LoRA expands moelora_forward runs inside the base GEMM's epilogue for
 * these dimensions (the follow-on fusion named in the vLLM blog page
 * "Multi-LoRA", section "Implementing Multi-LoRA inference for MoE models in
 * vLLM"): *flags gets bit MOELORA_FUSED_GATE_UP (gate_up expand and SiLU-mul;
 * G is then not written) and bit MOELORA_FUSED_DOWN (down expand).  The
 * matching MOELORA_STAGE_EXPAND_* stages are then empty.  A projection can
 * fuse when the dtype is bf16 and its base GEMM is not split over K (split K
 * is chosen only when the output has too few tiles to fill the GPU); it does
 * unless MOELORA_FLAG_UNFUSED is set or dims->plan.fuse is 2.  Host only;
 * returns the validation status of dims (MOELORA_ERR_NULL for a NULL flags).
 */
#define MOELORA_FUSED_GATE_UP 1
#define MOELORA_FUSED_DOWN 2
/* MOELORA_FUSED_DOWN_SHRINK: the fused gate_up epilogue also computes the down
 * projection's LoRA shrink (z2 = a A_dn, summed over its columns with relaxed
 * fp32 atomics, or per-N-tile partials summed in order with
 * MOELORA_FLAG_DETERMINISTIC); the MOELORA_STAGE_SHRINK_DOWN stage is then
 * empty (deterministic: only the ordered sum).  Set when the gate_up
 * expand is fused and dims->plan.fuse is 3. */
#define MOELORA_FUSED_DOWN_SHRINK 4
int moelora_forward_fusion(const moelora_dims* dims, int* flags);

/*
 * The plan moelora_forward runs for these dims: dims->plan with every
 * automatic (0) field resolved and the split counts rounded as described at
 * moelora_plan; fuse is 1 when at least one projection fuses, else 2.
 * Host only; returns the validation status of dims (MOELORA_ERR_NULL for a
 * NULL plan).
 */
int moelora_forward_plan(const moelora_dims* dims, moelora_plan* plan);

/*
 * Dense multi-LoRA projection: the vLLM blog page "Multi-LoRA", section
 * "Implementing Multi-LoRA inference for MoE models in vLLM", notes that the
 * same multi-LoRA kernels serve dense layers (e.g. attention projections).  For
 * every token t with adapter l = adapter_ids[t]:
 *   out[t] = x_t W + (x_t A[l]) B[l]
 * with no experts, routing or activation.  Runs the layer's own kernels with
 * one expert and k = 1: tokens bucketed by adapter, the shrink, the grouped
 * GEMM (with the LoRA expand in its epilogue for bf16 with unsplit K), the
 * expand otherwise, and the write-back to token order in the output dtype.
 * flags as in moelora_dims (deterministic split-K, base-only adapter -1,
 * unfused expand).
 */
typedef struct moelora_dense_dims {
  int64_t tokens;        /* T                                                       */
  int64_t in_features;   /* K, a multiple of 64                                     */
  int64_t out_features;  /* N, a multiple of 64                                     */
  int32_t adapters;      /* L                                                       */
  int32_t rank;          /* r: 16, 32 or 64                                         */
  int32_t dtype;         /* moelora_dtype of x, weights and out                     */
  int32_t flags;         /* 0, or any of MOELORA_FLAG_*                              */
  moelora_plan plan;     /* as for the layer, with the projection planned as the
                            down GEMM: ksplit_down applies, ksplit_gate_up must
                            be 0                                                   */
} moelora_dense_dims;

int moelora_dense_workspace_size(const moelora_dense_dims* dims, size_t* bytes);

/* The resolved plan of moelora_dense_forward (as moelora_forward_plan). */
int moelora_dense_forward_plan(const moelora_dense_dims* dims, moelora_plan* plan);

/*
 *   x              in  dtype [T][K]
 *   w              in  dtype [N][K]      (W^T rows; [K][N] with MOELORA_FLAG_IN_OUT)
 *   a              in  dtype [L][r][K]   (A^T rows per adapter; [L][K][r] with the flag)
 *   b              in  dtype [L][N][r]   (B^T rows per adapter; [L][r][N] with the flag)
 *   adapter_ids    in  int32 [T], in [0, L) (or -1 with MOELORA_FLAG_BASE_ONLY)
 *   out            out dtype [T][N], fully overwritten
 *   device_status  out int32 [1] or NULL: 0 ok, 1 an adapter id out of range
 *   workspace      device scratch of at least moelora_dense_workspace_size bytes
 */
int moelora_dense_forward(const moelora_dense_dims* dims, const void* x, const void* w,
                          const void* a, const void* b, const int32_t* adapter_ids, void* out,
                          int32_t* device_status, void* workspace, size_t workspace_bytes,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOELORA_H */
