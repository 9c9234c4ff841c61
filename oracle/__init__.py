"""CPU oracle for the fused MoE multi-LoRA layer (ctypes wrapper over liboracle.so).

TEST INFRASTRUCTURE ONLY: used by tests/, by ``__graft_entry__.smoke()`` and by
the CPU-baseline leg of ``bench.py``.  The HIP library never imports it and
shares no code with it.  Arithmetic lives in ``oracle.c`` (plain loops, double
precision); this file only marshals numpy arrays.

Functions follow the vLLM blog page "Multi-LoRA" (vllm.com.cn/blog/multi-lora),
section "Implementing Multi-LoRA inference for MoE models in vLLM": routing to
the top-k experts, the per-(expert, adapter) LoRA projections y = xW + (xA)B for
gate_up and down, SiLU(gate) * up between them, and the weighted combination.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT_F32, DT_BF16, DT_F64 = 0, 1, 2
_DT = {"f32": DT_F32, "bf16": DT_BF16, "f64": DT_F64}

_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc: plain C11, OpenMP, no FMA contraction, no fast-math."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile liboracle.so next to its source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def load_library(path: str):
    """Load an oracle library file and declare its C signatures."""
    L = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    L.oracle_route.argtypes = [i64, i32, i32, vp, vp, vp]
    L.oracle_align.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp]
    L.oracle_slot.argtypes = [i64, i64, i64, i32, i32, i32, i32] + [vp] * 7 + [i64, i32, i32] + [vp] * 5
    L.oracle_forward.argtypes = ([i64, i64, i64, i32, i32, i32, i32, i32] + [vp] * 7 +
                                 [vp, vp, vp, i64, vp, vp, i32])
    L.oracle_dense.argtypes = [i64, i64, i64, i32, i32, i32] + [vp] * 5 + [i64, vp, vp, i32]
    for f in (L.oracle_route, L.oracle_align, L.oracle_slot, L.oracle_forward, L.oracle_dense):
        f.restype = ctypes.c_int
    L.oracle_max_threads.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = load_library(_LIB)
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    return np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def route(logits: np.ndarray, k: int):
    """Top-k expert ids (int32 [T][k]) and renormalised weights (float64 [T][k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = lib().oracle_route(T, E, k, _p(logits), _p(ids), _p(w))
    if rc != 0:
        raise ValueError(f"oracle_route failed: {rc}")
    return ids, w


def align(topk_ids: np.ndarray, adapter_ids: np.ndarray, experts: int, adapters: int,
          base_only: bool = False):
    """Stable (expert, adapter)-bucketed permutation: (sorted_slots [S], bucket_offsets
    [E*Lb+1]) with Lb = adapters, or adapters + 1 when base_only (adapter id -1
    allowed, its slots in each expert's last bucket)."""
    topk_ids = _c(topk_ids, np.int32)
    adapter_ids = _c(adapter_ids, np.int32)
    T, k = topk_ids.shape
    sorted_slots = np.empty(T * k, np.int32)
    offsets = np.empty(experts * (adapters + (1 if base_only else 0)) + 1, np.int32)
    rc = lib().oracle_align(T, k, experts, adapters, int(bool(base_only)), _p(topk_ids),
                            _p(adapter_ids), _p(sorted_slots), _p(offsets))
    if rc != 0:
        raise ValueError(f"oracle_align failed: {rc}")
    return sorted_slots, offsets


def _weights(inp: dict, dtype: str):
    names = ["x", "w_gate_up", "w_down", "a_gate_up", "b_gate_up", "a_down", "b_down"]
    np_dt = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[dtype]
    return [_c(inp[n], np_dt) for n in names]


def slot(inp: dict, dims: dict, t: int, e: int, l: int):
    """Intermediates of one slot: dict(g [2I], z1 [r], a [I], z2 [r], d [h]) in float64."""
    h, I, E, L, r = dims["hidden"], dims["intermediate"], dims["experts"], dims["adapters"], dims["rank"]
    dtype = dims["dtype"]
    arrs = _weights(inp, dtype)
    T = arrs[0].shape[0]
    g = np.empty(2 * I); z1 = np.empty(r); a = np.empty(I); z2 = np.empty(r); d = np.empty(h)
    rc = lib().oracle_slot(T, h, I, E, L, r, _DT[dtype], *[_p(x) for x in arrs], t, e, l,
                           _p(g), _p(z1), _p(a), _p(z2), _p(d))
    if rc != 0:
        raise ValueError(f"oracle_slot failed: {rc}")
    return {"g": g, "z1": z1, "a": a, "z2": z2, "d": d}


def forward(inp: dict, dims: dict, topk_ids: np.ndarray, topk_w: np.ndarray,
            tokens=None, threads: int = 0) -> np.ndarray:
    """Layer output (float64) for the given tokens (default: all), [len(tokens)][h]."""
    h, I, E, L, r = dims["hidden"], dims["intermediate"], dims["experts"], dims["adapters"], dims["rank"]
    dtype = dims["dtype"]
    arrs = _weights(inp, dtype)
    T = arrs[0].shape[0]
    k = topk_ids.shape[1]
    sel = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    out = np.empty((len(sel), h), np.float64)
    ids = _c(topk_ids, np.int32)
    w = _c(topk_w, np.float64)
    ad = _c(inp["adapter_ids"], np.int32)
    rc = lib().oracle_forward(T, h, I, E, k, L, r, _DT[dtype], *[_p(x) for x in arrs],
                              _p(ids), _p(w), _p(ad), len(sel), _p(sel), _p(out), threads)
    if rc != 0:
        raise ValueError(f"oracle_forward failed: {rc}")
    return out


def dense(x: np.ndarray, w: np.ndarray, a: np.ndarray, b: np.ndarray, adapter_ids: np.ndarray,
          dtype: str, tokens=None, threads: int = 0) -> np.ndarray:
    """Dense multi-LoRA projection y_t = x_t W + (x_t A[l]) B[l] (float64 [len(tokens)][N]);
    x [T][K], w = W^T [N][K], a = A^T [L][r][K], b = B^T [L][N][r], adapter -1 = base only."""
    np_dt = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[dtype]
    x, w, a, b = (_c(v, np_dt) for v in (x, w, a, b))
    T, K = x.shape
    N = w.shape[0]
    L, r = a.shape[0], a.shape[1]
    sel = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    out = np.empty((len(sel), N), np.float64)
    ad = _c(adapter_ids, np.int32)
    rc = lib().oracle_dense(T, K, N, L, r, _DT[dtype], _p(x), _p(w), _p(a), _p(b), _p(ad),
                            len(sel), _p(sel), _p(out), threads)
    if rc != 0:
        raise ValueError(f"oracle_dense failed: {rc}")
    return out


def dims_of(cfg) -> dict:
    """Dimension dict from a workload config (any object with the usual fields)."""
    return {"hidden": cfg.hidden, "intermediate": cfg.intermediate, "experts": cfg.experts,
            "adapters": cfg.adapters, "rank": cfg.rank, "top_k": cfg.top_k, "dtype": cfg.dtype}


def layer(inp: dict, cfg, tokens=None, threads: int = 0):
    """Route + permutation + forward, as one call; returns (topk_ids, topk_w, sorted_slots,
    bucket_offsets, out)."""
    ids, w = route(inp["logits"], cfg.top_k)
    base_only = bool(np.any(np.asarray(inp["adapter_ids"]) < 0))
    ss, off = align(ids, inp["adapter_ids"], cfg.experts, cfg.adapters, base_only=base_only)
    out = forward(inp, dims_of(cfg), ids, w, tokens=tokens, threads=threads)
    return ids, w, ss, off, out
