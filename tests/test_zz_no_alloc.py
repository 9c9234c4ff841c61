"""moelora_forward_noalloc (the forward in the library's static device
scratch, for callers that cannot allocate) against moelora_forward, through
the C ABI: two calls in a row, the second on a smaller batch, each within the
layer's tolerance of moelora_forward's output (and bit-identical to it in
deterministic mode), plus the refusal of a batch too large for the scratch."""
import ctypes

import pytest
import torch

import oracle
from gpu_util import WEIGHTS, assert_close, device, device_inputs, run_align, say, to_f64
from moe_lora_layer_amd import ops, synth

pytestmark = pytest.mark.gpu


def _cfg(T, seed):
    return synth.LayerConfig("noalloc", T, 512, 1024, 8, 2, 4, 32, "bf16", requests=T, seed=seed)


@pytest.mark.parametrize("det", [False, True], ids=["atomics", "deterministic"])
def test_noalloc_matches_forward_twice(det):
    dev = device()
    for T, seed in [(96, 3), (17, 4)]:          # the second call on a smaller batch
        cfg = _cfg(T, seed)
        say(f"noalloc T={T} deterministic={det}")
        inp = synth.make_inputs(cfg)
        dinp = device_inputs(inp, cfg, dev)
        d = ops.dims_for(cfg, deterministic=det)
        assert ops.forward_workspace_size(d) <= ops.NOALLOC_SCRATCH_BYTES
        ids, w, ss, off, st = run_align(cfg, dinp, dims=d)
        assert int(st[0].item()) == 0
        args = [d, dinp["x"], *[dinp[n] for n in WEIGHTS], w, ss, off]
        ref = ops.forward(*args, topk_ids=ids)
        out = torch.full((T, cfg.hidden), float("nan"), dtype=torch.bfloat16, device=dev)
        ops.forward_noalloc(*args, topk_ids=ids, out=out)
        torch.cuda.synchronize()
        if det:
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        else:
            assert_close(to_f64(out), to_f64(ref), "bf16", f"noalloc vs forward T={T}")
        ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
        assert_close(to_f64(out), oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w), "bf16",
                     f"noalloc vs oracle T={T}")


def test_noalloc_refuses_batches_beyond_the_scratch():
    cfg = synth.WORKLOADS["prefill_h4096"]
    d = ops.dims_for(cfg)
    assert ops.forward_workspace_size(d) > ops.NOALLOC_SCRATCH_BYTES
    lib = ops.library()
    fake = torch.empty(16, dtype=torch.uint8, device=device())
    p = [ops._ptr(fake)] * 12
    assert lib.moelora_forward_noalloc(ctypes.byref(d), *p, None) == 7
