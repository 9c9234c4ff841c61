"""moelora_forward and moelora_dense_forward under forced tile plans
(moelora_plan): every tile family, LoRA tile height, split count and fusion
choice must give the oracle's result within the layer's tolerance, on shapes
with ragged tails (the tuner may pick any of them)."""
import itertools

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, device, device_inputs, run_align, run_forward, say, to_f64
from moe_lora_layer_amd import ops, synth

pytestmark = pytest.mark.gpu

GEMM_SHAPES = [(32, 1), (64, 1), (128, 1), (128, 2), (128, 3), (256, 2)]


def _supported(plan, dtype):
    # the 128 x 256 DMA tiles (form 3) are bf16 only
    return plan.get("gemm_form") != 3 or dtype == "bf16"
PLANS = [dict(gemm_rows=r, gemm_form=f, lora_rows=lr, ksplit_gate_up=kg, ksplit_down=kd, fuse=fu)
         for (r, f), lr, (kg, kd), fu in itertools.product(GEMM_SHAPES, (16, 64), ((0, 0), (3, 2)),
                                                           (1, 2))]

# (T, h, I, E, k, L, r, dtype): rows per expert 38 (many buckets of a few rows),
# 150, and a fp32 layer; h and 2I tails against every tile width; 300 rows per
# expert over 16 adapters at rank 32 (a 256-row tile meets more buckets than
# one LDS group of the staged expand holds)
SHAPES = [(96, 192, 320, 5, 2, 3, 32, "bf16"), (300, 320, 192, 4, 2, 6, 64, "bf16"),
          (96, 192, 320, 5, 2, 3, 16, "f32"), (300, 256, 192, 2, 2, 16, 32, "bf16")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s" % s)
@pytest.mark.parametrize("det", [False, True])
def test_forward_every_plan(shape, det):
    cfg = synth.LayerConfig("plans", *shape, requests=shape[0], seed=sum(shape[:7]) + 7)
    inp = synth.make_inputs(cfg)
    dinp = device_inputs(inp, cfg, device())
    ids, w, ss, off, st = run_align(cfg, dinp)
    assert int(st[0].item()) == 0
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w)
    seen = set()
    for plan in PLANS:
        if not _supported(plan, cfg.dtype):
            continue
        d = ops.dims_for(cfg, deterministic=det, plan=plan)
        eff = ops.forward_plan(d)
        key = tuple(sorted(eff.items()))
        if key in seen:
            continue
        seen.add(key)
        say(f"forward {shape} det={det} plan {eff}")
        out, _ = run_forward(cfg, dinp, w, ss, off, dims=d)
        assert_close(to_f64(out), ref, cfg.dtype, f"plan {eff}")
    assert len(seen) >= 20


DENSE_PLANS = [dict(gemm_rows=r, gemm_form=f, lora_rows=lr, ksplit_down=kd, fuse=fu)
               for (r, f), lr, kd, fu in itertools.product(GEMM_SHAPES, (16, 64), (0, 3), (1, 2))]


def test_dense_every_plan():
    cfg = synth.DenseConfig("plans", 160, 384, 704, 5, 32, "bf16", requests=160, seed=77)
    inp = synth.make_dense_inputs(cfg)
    dev = device()
    t = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16
                   else torch.from_numpy(a)).to(dev)
    x, w, a, b, aid = (t(inp[n]) for n in ["x", "w", "a", "b", "adapter_ids"])
    ref = oracle.dense(inp["x"], inp["w"], inp["a"], inp["b"], inp["adapter_ids"], cfg.dtype)
    seen = set()
    for plan in DENSE_PLANS:
        d = ops.make_dense_dims(cfg.tokens, cfg.in_features, cfg.out_features, cfg.adapters,
                                cfg.rank, cfg.dtype, plan=plan)
        eff = ops.dense_forward_plan(d)
        key = tuple(sorted(eff.items()))
        if key in seen:
            continue
        seen.add(key)
        say(f"dense plan {eff}")
        out, st = ops.dense_forward(d, x, w, a, b, aid)
        torch.cuda.synchronize()
        assert int(st[0].item()) == 0
        assert_close(to_f64(out), ref, cfg.dtype, f"dense plan {eff}")
    assert len(seen) >= 15


@pytest.mark.parametrize("shape", SHAPES[:2] + SHAPES[2:3], ids=lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s" % s)
def test_forward_every_workgroup_order(shape):
    """plan.order 1-5 (launch order, XCD-grouped, rotated K walk, both, XCD-grouped
    with staggered K walks) on every
    GEMM tile family, split-K included, for both weight layouts: the oracle's
    result within tolerance."""
    from gpu_util import in_out
    cfg = synth.LayerConfig("orders", *shape, requests=shape[0], seed=sum(shape[:7]) + 9)
    inp = synth.make_inputs(cfg)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w)
    for io in (False, True):
        dinp = device_inputs(in_out(inp) if io else inp, cfg, device())
        ids, w, ss, off, st = run_align(cfg, dinp)
        assert int(st[0].item()) == 0
        seen = set()
        for (r, f), (kg, kd), order in itertools.product(GEMM_SHAPES, ((0, 0), (3, 2)), (1, 2, 3, 4, 5)):
            if not _supported(dict(gemm_form=f), cfg.dtype):
                continue
            d = ops.dims_for(cfg, in_out=io, plan=dict(gemm_rows=r, gemm_form=f, ksplit_gate_up=kg,
                                                       ksplit_down=kd, order=order))
            eff = ops.forward_plan(d)
            assert eff["order"] == order
            key = tuple(sorted(eff.items()))
            if key in seen:
                continue
            seen.add(key)
            say(f"forward {shape} in_out={io} plan {eff}")
            out, _ = run_forward(cfg, dinp, w, ss, off, dims=d)
            assert_close(to_f64(out), ref, cfg.dtype, f"plan {eff}")
