"""A layer step (moelora_align then moelora_forward, through the C ABI)
captured into a HIP graph and replayed: every replay, on new inputs copied
into the captured buffers and with its outputs clobbered beforehand, with
eager work and synchronisations in between, against the eager step on the
same inputs (routing and permutation bit for bit; the output bit-identical in
deterministic mode, within the layer's tolerance with atomics) and, for one
replay, against the oracle."""
import pytest
import torch

import oracle
from gpu_util import WEIGHTS, assert_close, device, device_inputs, in_out, say, to_f64
from moe_lora_layer_amd import ops, synth

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16_decode", lambda seed: synth.LayerConfig("graph", 64, 512, 1024, 8, 2, 4, 32, "bf16",
                                                   requests=64, seed=seed)),
    ("bf16_decode_in_out", lambda seed: synth.LayerConfig("graph_io", 64, 512, 1024, 8, 2, 4, 32, "bf16",
                                                          requests=64, seed=seed)),
    ("bf16_ragged", lambda seed: synth.LayerConfig("graph", 37, 256, 768, 6, 3, 5, 16, "bf16",
                                                   requests=37, seed=seed)),
    ("f32_tiny", lambda seed: synth.LayerConfig("graph", 64, 256, 512, 8, 2, 4, 16, "f32",
                                                requests=64, seed=seed)),
]


@pytest.mark.parametrize("det", [False, True], ids=["atomics", "deterministic"])
@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, make, det):
    dev = device()
    cfgs = [make(seed) for seed in (11, 12, 13, 14)]
    inps = [synth.make_inputs(c) for c in cfgs]
    kn = name.endswith("in_out")  # weights h_in x h_out (MOELORA_FLAG_IN_OUT); the oracle keeps inps
    dinps = [device_inputs(in_out(i) if kn else i, c, dev) for i, c in zip(inps, cfgs)]
    d = ops.dims_for(cfgs[0], deterministic=det, in_out=kn)
    W = {n: dinps[0][n] for n in WEIGHTS}  # one layer's weights (seed 11) for every input set
    eager = ops.MoELoRALayer(d, W, dev)
    refs, routings = [], []
    for di in dinps:
        refs.append(eager(di["x"], di["logits"], di["adapter_ids"]).clone())
        routings.append([t.clone() for t in eager.routing])
    torch.cuda.synchronize()
    assert int(eager.status[0].item()) == 0

    graphed = ops.MoELoRALayer(d, W, dev)
    x = dinps[0]["x"].clone()
    logits = dinps[0]["logits"].clone()
    aid = dinps[0]["adapter_ids"].clone()
    step = ops.CapturedStep(graphed, x, logits, aid)
    for rep in range(2):
        for i, di in enumerate(dinps):
            say(f"graph {name} det={det} pass {rep} input {i}")
            x.copy_(di["x"])
            logits.copy_(di["logits"])
            aid.copy_(di["adapter_ids"])
            graphed.out.fill_(-1.0)           # every output is rewritten by the replay
            for t in graphed.routing:
                t.fill_(-7)
            torch.cuda.synchronize()
            out = step.replay()
            torch.cuda.synchronize()
            assert int(graphed.status[0].item()) == 0
            for a, b in zip(graphed.routing, routings[i]):  # routing and permutation bit for bit
                assert torch.equal(a, b), (rep, i)
            if det:
                assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                                   refs[i].view(torch.int16) if out.dtype == torch.bfloat16 else refs[i])
            else:
                assert_close(to_f64(out), to_f64(refs[i]), cfgs[0].dtype, f"graph vs eager {i}")
            # eager work between replays
            eager(di["x"], di["logits"], di["adapter_ids"])
    # the last replay's input set against the oracle (weights of seed 11, inputs of seed 14)
    inp = dict(inps[0])
    for n in ("x", "logits", "adapter_ids"):
        inp[n] = inps[-1][n]
    ids, wts = oracle.route(inp["logits"], cfgs[0].top_k)
    out = step.replay()
    torch.cuda.synchronize()
    assert_close(to_f64(out), oracle.forward(inp, oracle.dims_of(cfgs[0]), ids, wts), cfgs[0].dtype,
                 f"graph {name} vs oracle")
