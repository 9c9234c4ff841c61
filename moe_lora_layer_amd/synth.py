"""Seeded synthetic workloads for the fused MoE multi-LoRA layer.

This module only draws random numbers and packs them; it contains none of the
layer's arithmetic (no routing, no sorting, no products).  Both the HIP path
and the CPU oracle are fed from the arrays it returns.

Workload shapes follow the problem statement of "Multi-LoRA for MoE models in
vLLM" (vllm.com.cn/blog/multi-lora, section "Implementing Multi-LoRA inference
for MoE models in vLLM" and Fig. 1): hidden 4096 -> intermediate 11008, LoRA
rank 16-64, per-request adapters, top-k experts per token.

Layout of every weight is K-contiguous ("[out][in]"): for a projection with
weight W of shape h_in x h_out the array holds W transposed, so row n of the
array is column n of W.  The LoRA factors A (h_in x r) and B (r x h_out) are
stored the same way, as A^T [r][h_in] and B^T [h_out][r].

Random streams: tensor ``tid`` of a workload with seed ``seed`` is cut into
chunks of ``CHUNK`` elements; chunk ``c`` is drawn from
``PCG64(SeedSequence([seed, tid, c]))`` as float32 standard normals, then
scaled by the tensor's standard deviation in float32.  bf16 workloads round the
scaled float32 values to bfloat16 with round-to-nearest-even.  The result does
not depend on how many threads draw the chunks.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22

# tensor ids (fixed: changing them changes every workload)
TID_X, TID_LOGITS, TID_BIAS, TID_ADAPTERS = 0, 1, 2, 3
TID_W_GU, TID_W_DN, TID_A_GU, TID_B_GU, TID_A_DN, TID_B_DN = 4, 5, 6, 7, 8, 9

DTYPE_F32 = "f32"
DTYPE_BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    tokens: int          # T
    hidden: int          # h
    intermediate: int    # I (gate_up produces 2I columns: [gate | up])
    experts: int         # E
    top_k: int           # k
    adapters: int        # L
    rank: int            # r
    dtype: str           # "f32" or "bf16"
    requests: int        # tokens are split into this many equal contiguous requests
    adapter_dist: str = "uniform"   # "uniform" or "zipf"
    zipf_s: float = 1.1
    logit_bias_var: float = 0.0     # variance of a per-expert bias added to the logits
    seed: int = 0

    @property
    def slots(self) -> int:
        return self.tokens * self.top_k

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  Variances follow the notation N(mean, variance):
# W, A ~ N(0, 1/h_in), B ~ N(0, 1/r), x and router logits ~ N(0, 1).
WORKLOADS: dict[str, LayerConfig] = {
    # 64 tokens, h 256, I 512, 8 experts top-2, 4 adapters rank 16, fp32
    "tiny_f32": LayerConfig("tiny_f32", 64, 256, 512, 8, 2, 4, 16, DTYPE_F32,
                            requests=64, seed=1000),
    # decode: 64 requests of one token, h 4096, I 11008, 16 experts top-2, 8 adapters rank 32
    "decode_h4096": LayerConfig("decode_h4096", 64, 4096, 11008, 16, 2, 8, 32, DTYPE_BF16,
                                requests=64, seed=1001),
    # prefill: 8 requests x 512 tokens, same shapes, per-expert logit bias N(0, 0.5)
    "prefill_h4096": LayerConfig("prefill_h4096", 4096, 4096, 11008, 16, 2, 8, 32, DTYPE_BF16,
                                 requests=8, logit_bias_var=0.5, seed=1002),
    # GPT-OSS-20B-shaped decode: h 2880, I 2880, 32 experts top-4, 64 adapters rank 64, Zipf(1.1)
    "gptoss_h2880": LayerConfig("gptoss_h2880", 256, 2880, 2880, 32, 4, 64, 64, DTYPE_BF16,
                                requests=256, adapter_dist="zipf", seed=1003),
    # dense degenerate case: 1 expert top-1, Llama-3.3-70B MLP h 8192, I 28672, 16 adapters rank 16
    "dense_h8192": LayerConfig("dense_h8192", 128, 8192, 28672, 1, 1, 16, 16, DTYPE_BF16,
                               requests=128, seed=1004),
}
WORKLOAD_ORDER = ["tiny_f32", "decode_h4096", "prefill_h4096", "gptoss_h2880", "dense_h8192"]


@dataclasses.dataclass(frozen=True)
class DenseConfig:
    """A dense multi-LoRA projection: y_t = x_t W + (x_t A[l]) B[l] (no experts)."""
    name: str
    tokens: int          # T
    in_features: int     # K
    out_features: int    # N
    adapters: int        # L
    rank: int            # r
    dtype: str
    requests: int        # tokens split into this many equal contiguous requests (one adapter each)
    seed: int = 0


DENSE_WORKLOADS: dict[str, DenseConfig] = {
    # Llama-3.3-70B fused q/k/v projection (8192 -> 8192 + 2 x 1024 with 8 KV heads),
    # 128 decode tokens, 16 adapters rank 16, uniform per token
    "qkv_dense_h8192": DenseConfig("qkv_dense_h8192", 128, 8192, 10240, 16, 16, DTYPE_BF16,
                                   requests=128, seed=1005),
}


def make_dense_inputs(cfg: DenseConfig) -> dict:
    """x [T][K], w = W^T [N][K], a = A^T [L][r][K], b = B^T [L][N][r] (W, A ~ N(0, 1/K),
    B ~ N(0, 1/r)), adapter ids uniform per request."""
    T, K, N, L, r = cfg.tokens, cfg.in_features, cfg.out_features, cfg.adapters, cfg.rank
    g = _rng(cfg.seed, TID_ADAPTERS)
    req = g.integers(0, L, size=cfg.requests)
    return {"x": _normal_tensor(cfg.seed, TID_X, (T, K), 1.0, cfg.dtype),
            "w": _normal_tensor(cfg.seed, TID_W_GU, (N, K), K ** -0.5, cfg.dtype),
            "a": _normal_tensor(cfg.seed, TID_A_GU, (L, r, K), K ** -0.5, cfg.dtype),
            "b": _normal_tensor(cfg.seed, TID_B_GU, (L, N, r), r ** -0.5, cfg.dtype),
            "adapter_ids": np.repeat(req.astype(np.int32), T // cfg.requests)}


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs here are finite, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact expansion of bfloat16 bit patterns (uint16) to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_tensor(seed: int, tid: int, shape, std: float, dtype: str) -> np.ndarray:
    """std * N(0,1) samples of the given shape, in float32 or bf16 bits (uint16)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32 if dtype == DTYPE_F32 else np.uint16)
    nchunks = (n + CHUNK - 1) // CHUNK
    s = np.float32(std)

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, c])))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        v *= s
        if dtype == DTYPE_F32:
            out[lo:hi] = v
        else:
            out[lo:hi] = f32_to_bf16_bits(v)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, 0])))


def make_routing_inputs(cfg: LayerConfig) -> dict:
    """Router logits (fp32 [T][E]) and per-token adapter ids (int32 [T])."""
    T, E, L = cfg.tokens, cfg.experts, cfg.adapters
    logits = _normal_tensor(cfg.seed, TID_LOGITS, (T, E), 1.0, DTYPE_F32)
    if cfg.logit_bias_var > 0.0:
        bias = _normal_tensor(cfg.seed, TID_BIAS, (E,), float(np.sqrt(cfg.logit_bias_var)), DTYPE_F32)
        logits = (logits + bias[None, :]).astype(np.float32)
    R = cfg.requests
    if T > 0:
        if R <= 0 or T % R != 0:
            raise ValueError(f"{cfg.name}: tokens {T} not divisible into {R} requests")
        g = _rng(cfg.seed, TID_ADAPTERS)
        if cfg.adapter_dist == "uniform":
            req = g.integers(0, L, size=R)
        elif cfg.adapter_dist == "zipf":
            p = (np.arange(L, dtype=np.float64) + 1.0) ** (-cfg.zipf_s)
            req = g.choice(L, size=R, p=p / p.sum())
        else:
            raise ValueError(cfg.adapter_dist)
        adapter_ids = np.repeat(req.astype(np.int32), T // R)
    else:
        adapter_ids = np.zeros(0, dtype=np.int32)
    return {"logits": np.ascontiguousarray(logits, dtype=np.float32),
            "adapter_ids": np.ascontiguousarray(adapter_ids, dtype=np.int32)}


def make_inputs(cfg: LayerConfig, with_weights: bool = True) -> dict:
    """All inputs of one workload.  Weight arrays are K-contiguous:
    w_gate_up [E][2I][h], w_down [E][h][I], a_gate_up [L][E][r][h],
    b_gate_up [L][E][2I][r], a_down [L][E][r][I], b_down [L][E][h][r].
    bf16 tensors are uint16 bit patterns."""
    T, h, I, E, L, r = cfg.tokens, cfg.hidden, cfg.intermediate, cfg.experts, cfg.adapters, cfg.rank
    d = dict(make_routing_inputs(cfg))
    d["x"] = _normal_tensor(cfg.seed, TID_X, (T, h), 1.0, cfg.dtype)
    if with_weights:
        d["w_gate_up"] = _normal_tensor(cfg.seed, TID_W_GU, (E, 2 * I, h), h ** -0.5, cfg.dtype)
        d["w_down"] = _normal_tensor(cfg.seed, TID_W_DN, (E, h, I), I ** -0.5, cfg.dtype)
        d["a_gate_up"] = _normal_tensor(cfg.seed, TID_A_GU, (L, E, r, h), h ** -0.5, cfg.dtype)
        d["b_gate_up"] = _normal_tensor(cfg.seed, TID_B_GU, (L, E, 2 * I, r), r ** -0.5, cfg.dtype)
        d["a_down"] = _normal_tensor(cfg.seed, TID_A_DN, (L, E, r, I), I ** -0.5, cfg.dtype)
        d["b_down"] = _normal_tensor(cfg.seed, TID_B_DN, (L, E, h, r), r ** -0.5, cfg.dtype)
    return d


def to_float(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 view of a workload tensor (exact for bf16)."""
    return a if dtype == DTYPE_F32 else bf16_bits_to_f32(a)


def from_float(a: np.ndarray, dtype: str) -> np.ndarray:
    """Pack float values into a workload tensor of the given dtype (bf16: RNE)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a if dtype == DTYPE_F32 else f32_to_bf16_bits(a)
