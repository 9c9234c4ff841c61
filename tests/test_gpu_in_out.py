"""MOELORA_FLAG_IN_OUT: the weights passed as the Multi-LoRA page writes them
(W h_in x h_out, A h_in x r, B r x h_out, row-major), through the C ABI.
The test transposes the K-contiguous arrays on the host; the oracle is the
unchanged one on the original arrays.  Every tile family of both dtypes
(SMALL), the unfused, deterministic and base-only modes, the dense
projection, and the decode and prefill workloads at full size (every M-tile
covered) against the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (WEIGHTS, assert_close, device, device_inputs, in_out, run_align, run_forward,
                      say, sample_tokens, to_f64)
from moe_lora_layer_amd import ops, synth, tune
from test_gpu_dense import _inputs as dense_inputs
from test_gpu_forward import DET_SHAPES, SMALL, UNFUSED, _small, mtile_cover

pytestmark = pytest.mark.gpu
IDS = lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s" % s[:8]


def _run(cfg, inp, dims, base_frac=0.0):
    dev = device()
    dinp = device_inputs(in_out(inp), cfg, dev)
    ids, w, ss, off, st = run_align(cfg, dinp, dims)
    assert int(st[0].item()) == 0
    ws = ops.workspace(ops.forward_workspace_size(dims), dev)
    ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    out, _ = run_forward(cfg, dinp, w, ss, off, dims=dims, workspace_buf=ws)
    return ids, ss, off, out


@pytest.mark.parametrize("shape", SMALL, ids=IDS)
def test_in_out_small(shape):
    cfg = _small(*shape, seed=sum(shape[:7]))
    say(f"in_out small {shape}")
    inp = synth.make_inputs(cfg)
    ids, _, _, out = _run(cfg, inp, ops.dims_for(cfg, in_out=True))
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert_close(to_f64(out), oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w), cfg.dtype, "out")


@pytest.mark.parametrize("mode", ["unfused", "deterministic", "base_only"])
@pytest.mark.parametrize("shape", sorted(set(UNFUSED + DET_SHAPES)), ids=IDS)
def test_in_out_modes(shape, mode):
    cfg = _small(*shape, seed=sum(shape[:7]) + 5)
    say(f"in_out {mode} {shape}")
    inp = synth.make_inputs(cfg)
    if mode == "base_only":
        rng = np.random.default_rng(cfg.tokens)
        inp["adapter_ids"] = np.where(rng.random(cfg.tokens) < 0.3, -1, inp["adapter_ids"]).astype(np.int32)
    d = ops.dims_for(cfg, in_out=True, unfused=mode == "unfused", deterministic=mode == "deterministic",
                     base_only=mode == "base_only")
    _, _, _, out = _run(cfg, inp, d)
    if mode == "deterministic":
        _, _, _, again = _run(cfg, inp, d)
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                           again.view(torch.int16) if out.dtype == torch.bfloat16 else again.view(torch.int32))
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert_close(to_f64(out), oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w), cfg.dtype, "out")


@pytest.mark.parametrize("shape", [(24, 256, 320, 4, 16, "bf16"), (48, 192, 256, 3, 32, "f32"),
                                   (200, 320, 192, 5, 64, "bf16"), (700, 256, 384, 3, 32, "bf16"),
                                   (600, 128, 192, 2, 16, "f32"), (96, 2048, 128, 4, 16, "bf16")],
                         ids=lambda s: "T%d_K%d_N%d_L%d_r%d_%s" % s)
def test_in_out_dense(shape):
    T, K, N, L, r, dtype = shape
    say(f"in_out dense {shape}")
    inp = dense_inputs(T, K, N, L, r, dtype, seed=T + K + N + 1)
    dev = device()
    t = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
                   if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    d = ops.make_dense_dims(T, K, N, L, r, dtype, in_out=True)
    out, st = ops.dense_forward(d, t(inp["x"]), t(inp["w"].T), t(np.swapaxes(inp["a"], 1, 2)),
                                t(np.swapaxes(inp["b"], 1, 2)), torch.from_numpy(inp["adapter_ids"]).to(dev))
    torch.cuda.synchronize()
    assert int(st[0].item()) == 0
    ref = oracle.dense(inp["x"], inp["w"], inp["a"], inp["b"], inp["adapter_ids"], dtype)
    assert_close(to_f64(out), ref, dtype, "dense out")


@pytest.mark.parametrize("name", ["decode_h4096", "prefill_h4096"])
def test_in_out_workload(name):
    """Full size, the benchmark's plan, every M-tile holding a compared row."""
    cfg = synth.WORKLOADS[name]
    say(f"in_out workload {name}: generating inputs")
    inp = synth.make_inputs(cfg)
    d, _ = tune.with_packaged_plan(ops.dims_for(cfg, in_out=True))
    plan = ops.forward_plan(d)
    ids, ss, off, out = _run(cfg, inp, d)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ss_h, off_h = ss.cpu().numpy(), off.cpu().numpy()
    toks = sample_tokens(cfg.tokens, 24 if cfg.tokens > 64 else cfg.tokens)
    _, _, extra = mtile_cover(off_h, cfg.experts, cfg.adapters, plan["gemm_rows"], ss_h, cfg.top_k, toks)
    toks = np.unique(np.concatenate([toks, np.array(extra, np.int64)]))
    covered, tiles, _ = mtile_cover(off_h, cfg.experts, cfg.adapters, plan["gemm_rows"], ss_h, cfg.top_k, toks)
    say(f"in_out workload {name}: plan {plan}, {len(toks)} tokens, M-tiles {covered}/{tiles}")
    assert covered == tiles
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w, tokens=toks)
    assert_close(to_f64(out)[toks], ref, cfg.dtype, f"{name} in_out out")
