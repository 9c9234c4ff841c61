"""The plan tuner on a small layer and a small dense projection: it returns a
valid resolved plan whose run matches the oracle, and its table round-trips
through plan_for."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, device, device_inputs, run_align, run_forward, say, to_f64
from moe_lora_layer_amd import ops, synth, tune

pytestmark = pytest.mark.gpu


def test_tune_layer_and_table(tmp_path):
    cfg = synth.LayerConfig("tune_small", 96, 192, 320, 5, 2, 3, 32, "bf16", requests=96, seed=31)
    logs = []
    entry = tune.tune_layer(cfg, steps=2, rounds=1, log=logs.append)
    say(f"tuned {entry['plan']} {entry['us']} us (automatic {entry['auto_us']} us)")
    assert entry["us"] <= entry["auto_us"]
    d = ops.dims_for(cfg, plan=entry["plan"])
    assert ops.forward_plan(d) == entry["plan"]
    path = str(tmp_path / "plans.json")
    tune.save_table(path, [entry])
    assert tune.plan_for(ops.dims_for(cfg), tune.load_table(path)) == entry["plan"]
    inp = synth.make_inputs(cfg)
    dinp = device_inputs(inp, cfg, device())
    ids, w, ss, off, _ = run_align(cfg, dinp)
    out, _ = run_forward(cfg, dinp, w, ss, off, dims=d)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert_close(to_f64(out), oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w), "bf16",
                 "tuned plan out")


def test_tune_dense():
    cfg = synth.DenseConfig("tune_dense", 64, 256, 384, 4, 16, "bf16", requests=64, seed=32)
    entry = tune.tune_dense(cfg, steps=2, rounds=1, log=lambda s: None)
    assert entry["kind"] == "dense" and entry["plan"]["ksplit_gate_up"] == 0
    d = ops.make_dense_dims(cfg.tokens, cfg.in_features, cfg.out_features, cfg.adapters, cfg.rank,
                            cfg.dtype, plan=entry["plan"])
    assert ops.dense_forward_plan(d) == entry["plan"]
