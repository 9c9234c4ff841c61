"""moelora_dense_forward on the GPU against the oracle's dense projection
(y_t = x_t W + (x_t A[l]) B[l]), through the C ABI.  Tolerance as for the
layer: 1e-2 * max|oracle| (bf16), 1e-4 * max|oracle| (fp32)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, device, say, to_f64
from moe_lora_layer_amd import ops, synth, tune

pytestmark = pytest.mark.gpu


def _inputs(T, K, N, L, r, dtype, seed, base_frac=0.0):
    rng = np.random.default_rng(seed)
    f = lambda shape, std: synth.from_float((rng.standard_normal(shape) * std).astype(np.float32), dtype)
    inp = {"x": f((T, K), 1.0), "w": f((N, K), K ** -0.5), "a": f((L, r, K), K ** -0.5),
           "b": f((L, N, r), r ** -0.5)}
    ad = rng.integers(0, L, T).astype(np.int32)
    if base_frac > 0:
        ad = np.where(rng.random(T) < base_frac, -1, ad).astype(np.int32)
    inp["adapter_ids"] = ad
    return inp


def _run(inp, T, K, N, L, r, dtype, tuned=False, **flags):
    dev = device()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16
                   else torch.from_numpy(a)).to(dev)
    d = ops.make_dense_dims(T, K, N, L, r, dtype, **flags)
    if tuned:  # the plan the benchmark runs: the packaged table's, if it has one
        d, _ = tune.with_packaged_plan(d)
    ws = ops.workspace(ops.dense_workspace_size(d), dev)
    ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    out, st = ops.dense_forward(d, t(inp["x"]), t(inp["w"]), t(inp["a"]), t(inp["b"]),
                                torch.from_numpy(inp["adapter_ids"]).to(dev), workspace_buf=ws)
    torch.cuda.synchronize()
    assert out.dtype == tdt
    return out, int(st[0].item())


DENSE_SHAPES = [
    # (T, K, N, L, r, dtype): 32-, 64-, 128- and 256-row tiles (the last with the
    # expand in the GEMM epilogue in bf16), N tails, split-K (narrow N, long K)
    (24, 256, 320, 4, 16, "bf16"),
    (48, 192, 256, 3, 32, "f32"),
    (200, 320, 192, 5, 64, "bf16"),
    (700, 256, 384, 3, 32, "bf16"),
    (600, 128, 192, 2, 16, "f32"),
    (96, 2048, 128, 4, 16, "bf16"),
    # more adapters than the align kernel keeps bucket counters for in LDS
    # (40000 > 36864): the counters go to the workspace
    (300, 64, 64, 40000, 16, "bf16"),
]


@pytest.mark.parametrize("shape", DENSE_SHAPES, ids=lambda s: "T%d_K%d_N%d_L%d_r%d_%s" % s)
@pytest.mark.parametrize("mode", ["plain", "deterministic", "base_only"])
def test_dense_forward(shape, mode):
    T, K, N, L, r, dtype = shape
    say(f"dense {shape} {mode}")
    inp = _inputs(T, K, N, L, r, dtype, seed=T + K + N, base_frac=0.3 if mode == "base_only" else 0.0)
    out, st = _run(inp, T, K, N, L, r, dtype, deterministic=(mode == "deterministic"),
                   base_only=(mode == "base_only"))
    assert st == 0
    ref = oracle.dense(inp["x"], inp["w"], inp["a"], inp["b"], inp["adapter_ids"], dtype)
    assert_close(to_f64(out), ref, dtype, "dense out")
    if mode == "deterministic":
        again, _ = _run(inp, T, K, N, L, r, dtype, deterministic=True)
        assert torch.equal(again.view(torch.int16) if again.dtype == torch.bfloat16 else again.view(torch.int32),
                           out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32))


def test_dense_qkv_projection():
    """Llama-3.3-70B-shaped fused q/k/v projection (8192 -> 10240), 128 decode
    tokens over 16 rank-16 adapters (the benchmark's dense workload, in its
    plan); sampled tokens against the oracle."""
    cfg = synth.DENSE_WORKLOADS["qkv_dense_h8192"]
    T, K, N, L, r, dtype = cfg.tokens, cfg.in_features, cfg.out_features, cfg.adapters, cfg.rank, cfg.dtype
    inp = synth.make_dense_inputs(cfg)
    out, st = _run(inp, T, K, N, L, r, dtype, tuned=True)
    assert st == 0
    toks = np.arange(0, T, 9)
    ref = oracle.dense(inp["x"], inp["w"], inp["a"], inp["b"], inp["adapter_ids"], dtype, tokens=toks)
    assert_close(to_f64(out)[toks], ref, dtype, "qkv out")


def test_dense_reports_bad_adapter():
    T, K, N, L, r = 40, 128, 128, 3, 16
    inp = _inputs(T, K, N, L, r, "bf16", seed=2)
    inp["adapter_ids"][5] = L
    _, st = _run(inp, T, K, N, L, r, "bf16")
    assert st == 1
