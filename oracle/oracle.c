/*
 * CPU oracle for the fused MoE multi-LoRA layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; it is used by tests/, by the
 * smoke check of __graft_entry__ and by the CPU-baseline leg of bench.py.  It
 * shares no source with the HIP library.
 *
 * What it computes follows the vLLM blog page "Multi-LoRA" (vllm.com.cn/blog/
 * multi-lora), section "Implementing Multi-LoRA inference for MoE models in
 * vLLM" and its Fig. 1:
 *   - a router sends every token to its most relevant experts and the experts'
 *     outputs are aggregated;
 *   - an expert is a gate_up projection (hidden h -> 2I, gate and up halves)
 *     followed by a down projection (I -> h);
 *   - every projection with frozen weight W (h_in x h_out) carries a LoRA
 *     adapter A (h_in x r), B (r x h_out) and computes y = xW + (xA)B, the
 *     "shrink" z = xA followed by the "expand" zB;
 *   - the adapter is chosen per request, the LoRA weights are per (adapter,
 *     expert), so each expert runs four LoRA ops.
 * Where the page leaves a step open the plainest reading is taken:
 *   - routing is softmax over the E router logits, keep the k largest
 *     (ties to the lower expert id, slots in descending logit order), and
 *     renormalise the kept probabilities to sum to one;
 *   - the gate_up output holds the gate in columns [0, I) and up in [I, 2I),
 *     and the activation is SiLU(gate) * up with SiLU(v) = v / (1 + e^-v);
 *   - the expert outputs are combined as sum_j w_tj * d_tj in slot order;
 *   - the (expert, adapter)-bucketed permutation is the stable sort of the
 *     slots s = t*k + j by key e*L + l.
 *
 * Storage: every weight is K-contiguous, i.e. the array holds the matrix
 * transposed: W^T [E][h_out][h_in], A^T [L][E][r][h_in], B^T [L][E][h_out][r].
 * The arithmetic is unaffected: entry (k, n) of W is element [n][k].
 *
 * Arithmetic: every element is expanded exactly to double (bf16 by bit shift),
 * every sum runs in ascending index order in double, no fused multiply-add
 * (built with -ffp-contract=off), no fast-math.
 *
 * Parity pins (tests/test_oracle.py): routing ids against a stable argsort,
 * weights against a library softmax, the permutation against a stable
 * argsort, the forward against a dense every-expert formulation, against
 * exact integer arithmetic, against the merged-weight identity
 * x(W + AB) = xW + (xA)B, B = 0 reducing to the base MoE, the E = 1 case
 * against a library SwiGLU MLP, and token-permutation invariance.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2

#define ORC_OK 0
#define ORC_EARG (-1)
#define ORC_EADAPTER 1
#define ORC_ENOMEM (-2)

static double elem(const void* base, int64_t i, int dtype) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  if (dtype == ORC_BF16) {
    uint32_t u = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return ((const double*)base)[i];
}

/* sum_{k < n} v[k] * M[off + k], ascending k */
static double dot(const double* v, const void* M, int64_t off, int64_t n, int dtype) {
  double acc = 0.0;
  int64_t k;
  if (dtype == ORC_F32) {
    const float* m = (const float*)M + off;
    for (k = 0; k < n; ++k) acc += v[k] * (double)m[k];
  } else if (dtype == ORC_BF16) {
    const uint16_t* m = (const uint16_t*)M + off;
    for (k = 0; k < n; ++k) {
      uint32_t u = ((uint32_t)m[k]) << 16;
      float f;
      memcpy(&f, &u, sizeof f);
      acc += v[k] * (double)f;
    }
  } else {
    const double* m = (const double*)M + off;
    for (k = 0; k < n; ++k) acc += v[k] * m[k];
  }
  return acc;
}

/*
 * Routing for every token: the k experts with the largest logits, in
 * descending logit order (exact float comparisons, ties to the lower id), and
 * their softmax probabilities renormalised over the k kept experts.  With
 * m = the largest logit, w_j = exp(l_j - m) / sum_i exp(l_i - m); this is the
 * full softmax restricted to the kept experts and rescaled to sum to one.
 * A NaN logit (the page never meets one) ranks as -infinity, below every
 * number, so every token still gets k distinct experts.
 */
static float rank_value(float v) { return isnan(v) ? -INFINITY : v; }

int oracle_route(int64_t T, int32_t E, int32_t k, const float* logits,
                 int32_t* topk_ids, double* topk_w) {
  if (T < 0 || E < 1 || k < 1 || k > E) return ORC_EARG;
  char* taken = (char*)malloc((size_t)E);
  double* ex = (double*)malloc(sizeof(double) * (size_t)k);
  if (!taken || !ex) { free(taken); free(ex); return ORC_ENOMEM; }
  for (int64_t t = 0; t < T; ++t) {
    const float* lg = logits + t * E;
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || rank_value(lg[e]) > rank_value(lg[best])) best = e;
      }
      taken[best] = 1;
      topk_ids[t * k + j] = best;
    }
    double m = (double)rank_value(lg[topk_ids[t * k]]);
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      ex[j] = exp((double)rank_value(lg[topk_ids[t * k + j]]) - m);
      sum += ex[j];
    }
    for (int32_t j = 0; j < k; ++j) topk_w[t * k + j] = ex[j] / sum;
  }
  free(taken);
  free(ex);
  return ORC_OK;
}

/*
 * The (expert, adapter)-bucketed permutation: slot s = t*k + j gets key
 * topk_ids[s] * Lb + l(t), with Lb = L buckets per expert and l(t) =
 * adapter_ids[t]; bucket_offsets[b] is the number of slots with key < b
 * (b in [0, E*Lb]); sorted_slots lists the slots bucket by bucket, ascending
 * slot index inside a bucket (a stable counting sort).
 * base_only != 0: a token may also carry adapter id -1 (the base model with no
 * adapter; the pages do not cover it, and this reading gives it no LoRA term).
 * Each expert then has Lb = L + 1 buckets, its base-only slots in the last one
 * (l(t) = L for adapter -1).
 * Returns ORC_EADAPTER if an adapter id is outside [0, L) (and not an allowed -1).
 */
/* Bucket key of slot s: expert-major, then the token's adapter (a base-only
 * token, adapter id -1, goes to its expert's bucket L). */
static int64_t slot_key(const int32_t* topk_ids, const int32_t* adapter_ids, int64_t s, int32_t k,
                        int32_t E, int64_t Lb, int32_t L) {
  int32_t l = adapter_ids[s / k];
  (void)E;  /* the key is expert-major: E does not enter it */
  return (int64_t)topk_ids[s] * Lb + (l < 0 ? L : l);
}

int oracle_align(int64_t T, int32_t k, int32_t E, int32_t L, int32_t base_only,
                 const int32_t* topk_ids, const int32_t* adapter_ids, int32_t* sorted_slots,
                 int32_t* bucket_offsets) {
  if (T < 0 || k < 1 || E < 1 || L < 1) return ORC_EARG;
  int64_t Lb = L + (base_only ? 1 : 0);
  int64_t S = T * k, nb = (int64_t)E * Lb;
  for (int64_t t = 0; t < T; ++t) {
    int32_t l = adapter_ids[t];
    if (!(l >= 0 && l < L) && !(base_only && l == -1)) return ORC_EADAPTER;
  }
  for (int64_t s = 0; s < S; ++s)
    if (topk_ids[s] < 0 || topk_ids[s] >= E) return ORC_EARG;
  int64_t* next = (int64_t*)calloc((size_t)nb + 1, sizeof(int64_t));
  if (!next) return ORC_ENOMEM;
  for (int64_t s = 0; s < S; ++s) {
    int64_t key = slot_key(topk_ids, adapter_ids, s, k, E, Lb, L);
    if (key < 0 || key >= nb) { /* a key outside the buckets: refuse, write nothing */
      free(next);
      return ORC_EARG;
    }
    next[key + 1] += 1;
  }
  for (int64_t b = 0; b < nb; ++b) next[b + 1] += next[b];
  for (int64_t b = 0; b <= nb; ++b) bucket_offsets[b] = (int32_t)next[b];
  for (int64_t s = 0; s < S; ++s)
    sorted_slots[next[slot_key(topk_ids, adapter_ids, s, k, E, Lb, L)]++] = (int32_t)s;
  free(next);
  return ORC_OK;
}

/*
 * One LoRA projection of an input row v (length K) with base weight W^T rows
 * Wt (N rows of K), shrink factor At (r rows of K) and expand factor Bt
 * (N rows of r):  y = vW + (vA)B.  z receives the shrink result vA.
 * adapter == 0 (a base-only token): y = vW and z = 0.
 */
static void lora_projection(const double* v, int64_t K, int64_t N, int32_t r,
                            const void* Wt, int64_t w_off, const void* At, int64_t a_off,
                            const void* Bt, int64_t b_off, int dtype, int adapter, double* z,
                            double* y) {
  for (int32_t q = 0; q < r; ++q) z[q] = adapter ? dot(v, At, a_off + (int64_t)q * K, K, dtype) : 0.0;
  for (int64_t n = 0; n < N; ++n) {
    double base = dot(v, Wt, w_off + n * K, K, dtype);
    y[n] = adapter ? base + dot(z, Bt, b_off + n * r, r, dtype) : base;
  }
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/*
 * Everything one slot computes: token t through expert e with adapter l.
 *   g  [2I] = x_t W_gu[e] + (x_t A_gu[l][e]) B_gu[l][e]     (z1 [r] = x_t A_gu)
 *   a  [I]  = SiLU(g[0:I]) * g[I:2I]
 *   d  [h]  = a W_dn[e] + (a A_dn[l][e]) B_dn[l][e]           (z2 [r] = a A_dn)
 * l = -1 (a base-only token): both LoRA terms are absent (z1 = z2 = 0).
 */
int oracle_slot(int64_t T, int64_t h, int64_t I, int32_t E, int32_t L, int32_t r, int32_t dtype,
                const void* x, const void* w_gu, const void* w_dn, const void* a_gu,
                const void* b_gu, const void* a_dn, const void* b_dn, int64_t t, int32_t e,
                int32_t l, double* g, double* z1, double* a, double* z2, double* d) {
  if (t < 0 || t >= T || e < 0 || e >= E || l < -1 || l >= L || r < 1 || h < 1 || I < 1)
    return ORC_EARG;
  double* xin = (double*)malloc(sizeof(double) * (size_t)h);
  if (!xin) return ORC_ENOMEM;
  for (int64_t i = 0; i < h; ++i) xin[i] = elem(x, t * h + i, dtype);
  int64_t le = (int64_t)(l < 0 ? 0 : l) * E + e;
  lora_projection(xin, h, 2 * I, r, w_gu, (int64_t)e * 2 * I * h, a_gu, le * r * h, b_gu,
                  le * 2 * I * r, dtype, l >= 0, z1, g);
  for (int64_t i = 0; i < I; ++i) a[i] = silu(g[i]) * g[I + i];
  lora_projection(a, I, h, r, w_dn, (int64_t)e * h * I, a_dn, le * r * I, b_dn, le * h * r, dtype,
                  l >= 0, z2, d);
  free(xin);
  return ORC_OK;
}

/*
 * Layer output for the selected tokens sel[0..n_sel): out[i][:] (double,
 * [n_sel][h]) = sum_{j<k} topk_w[t][j] * d(t, topk_ids[t][j], adapter_ids[t])
 * (adapter id -1: base-only, see oracle_slot),
 * accumulated in ascending j starting from zero.  Tokens are independent, so
 * they are spread over nthreads OpenMP threads (0 = library default).
 */
int oracle_forward(int64_t T, int64_t h, int64_t I, int32_t E, int32_t k, int32_t L, int32_t r,
                   int32_t dtype, const void* x, const void* w_gu, const void* w_dn,
                   const void* a_gu, const void* b_gu, const void* a_dn, const void* b_dn,
                   const int32_t* topk_ids, const double* topk_w, const int32_t* adapter_ids,
                   int64_t n_sel, const int64_t* sel, double* out, int32_t nthreads) {
  if (T < 0 || h < 1 || I < 1 || E < 1 || k < 1 || k > E || L < 1 || r < 1 || n_sel < 0)
    return ORC_EARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F64) return ORC_EARG;
  for (int64_t i = 0; i < n_sel; ++i) {
    if (sel[i] < 0 || sel[i] >= T) return ORC_EARG;
    int32_t l = adapter_ids[sel[i]];
    if (l < -1 || l >= L) return ORC_EADAPTER;
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = topk_ids[sel[i] * k + j];
      if (e < 0 || e >= E) return ORC_EARG;  /* an expert id outside [0, E) */
    }
  }
  int status = ORC_OK;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
  for (int64_t i = 0; i < n_sel; ++i) {
    int64_t t = sel[i];
    double* g = (double*)malloc(sizeof(double) * (size_t)(2 * I));
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    double* d = (double*)malloc(sizeof(double) * (size_t)h);
    double* z = (double*)malloc(sizeof(double) * (size_t)(2 * r));
    if (!g || !a || !d || !z) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = ORC_ENOMEM;
    } else {
      double* o = out + i * h;
      for (int64_t n = 0; n < h; ++n) o[n] = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        int32_t e = topk_ids[t * k + j];
        int rc = oracle_slot(T, h, I, E, L, r, dtype, x, w_gu, w_dn, a_gu, b_gu, a_dn, b_dn, t,
                             e, adapter_ids[t], g, z, a, z + r, d);
        if (rc != ORC_OK) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
          status = rc;
          break;
        }
        double w = topk_w[t * k + j];
        for (int64_t n = 0; n < h; ++n) o[n] += w * d[n];
      }
    }
    free(g);
    free(a);
    free(d);
    free(z);
  }
  return status;
}

/*
 * Dense multi-LoRA projection (no experts, no routing, no activation): the
 * same page notes that the multi-LoRA kernels serve dense layers too, e.g.
 * attention projections.  For each selected token t with adapter l = ids[t]:
 *   out[i][:] = x_t W + (x_t A[l]) B[l]      (out [n_sel][N], double)
 * with W^T rows Wt [N][K], A^T rows At [L][r][K], B^T rows Bt [L][N][r];
 * adapter -1 (base model only) drops the LoRA term.
 */
int oracle_dense(int64_t T, int64_t K, int64_t N, int32_t L, int32_t r, int32_t dtype,
                 const void* x, const void* Wt, const void* At, const void* Bt,
                 const int32_t* adapter_ids, int64_t n_sel, const int64_t* sel, double* out,
                 int32_t nthreads) {
  if (T < 0 || K < 1 || N < 1 || L < 1 || r < 1 || n_sel < 0) return ORC_EARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F64) return ORC_EARG;
  for (int64_t i = 0; i < n_sel; ++i) {
    if (sel[i] < 0 || sel[i] >= T) return ORC_EARG;
    if (adapter_ids[sel[i]] < -1 || adapter_ids[sel[i]] >= L) return ORC_EADAPTER;
  }
  int status = ORC_OK;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
  for (int64_t i = 0; i < n_sel; ++i) {
    int64_t t = sel[i];
    int32_t l = adapter_ids[t];
    double* xin = (double*)malloc(sizeof(double) * (size_t)K);
    double* z = (double*)malloc(sizeof(double) * (size_t)r);
    if (!xin || !z) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = ORC_ENOMEM;
    } else {
      for (int64_t k = 0; k < K; ++k) xin[k] = elem(x, t * K + k, dtype);
      int64_t lc = l < 0 ? 0 : l;
      lora_projection(xin, K, N, r, Wt, 0, At, lc * r * K, Bt, lc * N * r, dtype, l >= 0, z,
                      out + i * N);
    }
    free(xin);
    free(z);
  }
  return status;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
