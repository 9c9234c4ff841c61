"""moelora_forward on the GPU against the oracle, through the C ABI.

Tolerance: max|gpu - oracle| <= 1e-2 * max|oracle| for bf16 layers and
1e-4 * max|oracle| for fp32 layers, over every compared output.  Small shapes
(several tiles and ragged tails in M, N and K) are compared in full; the five
workloads at full size are compared on sampled tokens, in the same launch
configuration the benchmark times."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (WEIGHTS, assert_close, device, device_inputs, run_align, run_forward, say,
                      sample_tokens, to_f64, workspace_view)
from moe_lora_layer_amd import ops, synth, tune

pytestmark = pytest.mark.gpu


def _layer(cfg, inp, dims=None):
    dev = device()
    dinp = device_inputs(inp, cfg, dev)
    ids, w, ss, off, st = run_align(cfg, dinp, dims)
    assert int(st[0].item()) == 0
    out, ws = run_forward(cfg, dinp, w, ss, off, dims)
    return dinp, (ids, w, ss, off), out, ws


def _small(T, h, I, E, k, L, r, dtype, seed, requests=None, **kw):
    return synth.LayerConfig("small", T, h, I, E, k, L, r, dtype,
                             requests=requests if requests is not None else T, seed=seed, **kw)


# 1024 (expert, adapter) buckets over 2048 slots: enough 16-row LoRA tiles
# times K chunks for the persistent streaming shrink (gate_up only; the down
# shrink, K = 256, stays on the per-tile kernel)
STREAM_SHAPE = (512, 1088, 256, 16, 4, 64, 64, "bf16")
# the streaming shrink's other item shapes: rank 32 with 8-step chunks
# (h = 2048), rank 16 with 2-step chunks (h = 1088: 34 steps of 32), rank 64
# with 4-step chunks (h = 1024)
STREAM_SHAPES_R32_R16 = [(512, 2048, 128, 16, 4, 64, 32, "bf16"), (512, 1088, 128, 16, 4, 64, 16, "bf16"),
                         (512, 1024, 128, 16, 4, 64, 64, "bf16")]

SMALL = [
    # (T, h, I, E, k, L, r, dtype): rows/expert 16 (BM 32), 38 (BM 64), 67 (BM 128);
    # N tails (2I, h not multiples of 128), K of 64..640, ranks 16/32/64
    (64, 256, 512, 8, 2, 4, 16, "f32"),
    (96, 192, 320, 5, 2, 3, 32, "f32"),
    (200, 320, 192, 6, 2, 3, 64, "f32"),
    (64, 256, 512, 8, 2, 4, 16, "bf16"),
    (96, 192, 320, 5, 2, 3, 32, "bf16"),
    (200, 320, 192, 6, 2, 3, 64, "bf16"),
    (300, 640, 448, 4, 1, 7, 32, "bf16"),
    (33, 128, 64, 3, 3, 2, 16, "bf16"),
    (1, 64, 64, 4, 2, 2, 64, "bf16"),
    (7, 64, 128, 1, 1, 3, 16, "f32"),
    # > 200 rows per expert: 256-row tiles (N tails: 2I = 384, h = 128); in bf16
    # the LoRA expand (and SiLU-mul) runs in the GEMM epilogue: I and h tails,
    # ranks 16/32/64, many adapter buckets per tile, one expert with 16 adapters
    (600, 128, 192, 4, 2, 3, 16, "bf16"),
    (600, 192, 128, 4, 2, 2, 32, "f32"),
    (700, 256, 320, 3, 2, 5, 32, "bf16"),
    (520, 192, 256, 2, 1, 9, 64, "bf16"),
    (300, 128, 256, 1, 1, 16, 16, "bf16"),
    # one expert, narrow output: the down GEMM split over K into partial
    # planes that the combine sums
    (96, 128, 2048, 1, 1, 4, 16, "bf16"),
    # 175 rows per expert: one 256-row tile per expert (bf16 above 160 rows
    # per expert; the 128-row reuse tiles run under forced plans)
    (350, 192, 320, 4, 2, 3, 32, "bf16"),
    # top-8 routing over 64 experts; and the largest bucket count (E x L =
    # 8192) with most experts and buckets empty
    (64, 128, 192, 64, 8, 4, 16, "bf16"),
    (40, 128, 128, 128, 2, 64, 32, "bf16"),
    # many one- and two-row adapter buckets per tile, the expand in the GEMM
    # epilogue with the buckets' B staged in LDS: 32-, 64- and 128-row tiles,
    # ranks 16, 64, 32
    (48, 256, 192, 4, 2, 32, 16, "bf16"),
    (96, 192, 320, 4, 2, 64, 64, "bf16"),
    (350, 192, 320, 4, 2, 64, 32, "bf16"),
    # many short adapter buckets (~2 rows each): the gate_up shrink streams
    # (tile, K chunk) items, h = 1088 ends in a half chunk
    STREAM_SHAPE,
    *STREAM_SHAPES_R32_R16,
    # E * L = 65536 (expert, adapter) buckets, the largest the layer takes
    (300, 64, 64, 16, 2, 4096, 16, "bf16"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s" % s)
def test_forward_small(shape):
    cfg = _small(*shape, seed=sum(shape[:7]))
    say(f"forward small {shape}")
    inp = synth.make_inputs(cfg)
    _, (ids, w, ss, off), out, _ = _layer(cfg, inp)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w)
    assert_close(to_f64(out), ref, cfg.dtype, "out")


def _times_pow2(a, dtype, factor):
    """a * factor for a power of two (exact: bf16 patterns are widened to fp32,
    scaled and narrowed back without rounding)."""
    if dtype == "f32":
        return (a * np.float32(factor)).astype(np.float32)
    f = (a.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# Gate values far outside SiLU's curved part: gate_up weights times 2^6 (exact)
# put G = xW at a standard deviation near 64, so the epilogues meet SiLU's
# linear side and its saturated side, where e^-v overflows fp32 (v < -88):
# the 256-row direct-to-LDS tiles (first shape) and the register-staged ones
LARGE_GATE = [(600, 128, 192, 4, 2, 3, 16, "bf16"), (96, 192, 320, 5, 2, 3, 32, "bf16"),
              (96, 192, 320, 5, 2, 3, 32, "f32")]


@pytest.mark.parametrize("shape", LARGE_GATE, ids=lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s" % s)
def test_forward_large_gate_values(shape):
    cfg = _small(*shape, seed=7 + sum(shape[:7]))
    say(f"forward large gate values {shape}")
    inp = dict(synth.make_inputs(cfg))
    inp["w_gate_up"] = _times_pow2(inp["w_gate_up"], cfg.dtype, 64)
    # the premise: the gate values reach both SiLU regions
    f64 = lambda a: (a if cfg.dtype == "f32" else (a.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    g = np.einsum("th,enh->ten", f64(inp["x"]), f64(inp["w_gate_up"])[:, :cfg.intermediate, :])
    assert g.max() > 88.0 and g.min() < -88.0
    _, (ids, w, ss, off), out, _ = _layer(cfg, inp)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w)
    assert_close(to_f64(out), ref, cfg.dtype, "out")


# bf16 shapes run again with MOELORA_FLAG_UNFUSED: the LoRA expands as
# kernels of their own after each GEMM (one shape per GEMM tile shape)
UNFUSED = [(64, 256, 512, 8, 2, 4, 16, "bf16"), (96, 192, 320, 5, 2, 3, 32, "bf16"),
           (200, 320, 192, 6, 2, 3, 64, "bf16"), (350, 192, 320, 4, 2, 3, 32, "bf16"),
           (700, 256, 320, 3, 2, 5, 32, "bf16")]


@pytest.mark.parametrize("shape", UNFUSED, ids=lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s" % s)
def test_forward_small_unfused(shape):
    cfg = _small(*shape, seed=sum(shape[:7]))
    say(f"forward small unfused {shape}")
    inp = synth.make_inputs(cfg)
    d = ops.dims_for(cfg, unfused=True)
    assert ops.forward_fusion(d) == {"gate_up": False, "down": False, "down_shrink": False}
    assert ops.forward_fusion(ops.dims_for(cfg)) == {"gate_up": True, "down": True, "down_shrink": False}
    _, (ids, w, ss, off), out, _ = _layer(cfg, inp, d)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w)
    assert_close(to_f64(out), ref, cfg.dtype, "out")


def mtile_cover(off, experts, buckets, rows, ss, top_k, toks):
    """The M-tiles of the base GEMMs (each expert's sorted rows cut into tiles of
    `rows`, the last one partial) and the fraction of them holding a slot of a
    token in `toks`; plus one token per tile (the tile's last row), so that a
    sample can be completed to cover every tile."""
    have = set(int(t) for t in toks)
    covered, tiles, extra = 0, 0, []
    for e in range(experts):
        r0, r1 = int(off[e * buckets]), int(off[(e + 1) * buckets])
        for a in range(r0, r1, rows):
            b = min(r1, a + rows)
            tiles += 1
            tile_toks = {int(ss[p]) // top_k for p in range(a, b)}
            if tile_toks & have:
                covered += 1
            extra.append(int(ss[b - 1]) // top_k)
    return covered, tiles, extra


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_forward_workload(name):
    """Every workload at full size in the benchmark's launch configuration.
    The compared tokens are a random sample completed so that every M-tile of
    the base GEMMs (every expert's first and last, partial, tile included;
    with the 256-row plan also the down GEMM's stream-K tiles, which are M x N
    tiles of the same M-tiles) holds a compared row: the test asserts 100 %
    M-tile coverage.  The dense 70B-MLP workload (128 tokens) is compared in
    full."""
    cfg = synth.WORKLOADS[name]
    say(f"forward workload {name}: generating inputs")
    inp = synth.make_inputs(cfg)
    # the benchmark's launch configuration: the packaged tuned plan, if any
    d, source = tune.with_packaged_plan(ops.dims_for(cfg))
    plan = ops.forward_plan(d)
    say(f"forward workload {name}: running on GPU, plan {plan} ({source})")
    _, (ids, w, ss, off), out, _ = _layer(cfg, inp, d)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ss_h, off_h = ss.cpu().numpy(), off.cpu().numpy()
    if name == "dense_h8192":
        toks = np.arange(cfg.tokens)
    else:
        toks = sample_tokens(cfg.tokens, 24 if cfg.tokens > 64 else cfg.tokens)
        _, _, extra = mtile_cover(off_h, cfg.experts, cfg.adapters, plan["gemm_rows"], ss_h,
                                  cfg.top_k, toks)
        toks = np.unique(np.concatenate([toks, np.array(extra, np.int64)]))
    covered, tiles, _ = mtile_cover(off_h, cfg.experts, cfg.adapters, plan["gemm_rows"], ss_h,
                                    cfg.top_k, toks)
    say(f"forward workload {name}: oracle on {len(toks)} tokens, M-tile coverage "
        f"{covered}/{tiles} ({plan['gemm_rows']}-row tiles)")
    assert covered == tiles
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w, tokens=toks)
    assert_close(to_f64(out)[toks], ref, cfg.dtype, f"{name} out")


def test_persistent_gate_up_queues():
    """More gate_up tiles than CUs (bf16, 256-row tiles, XCD-grouped order:
    6 M-tiles x 64 N-tiles): the gate_up GEMM runs one workgroup per CU over
    per-XCD tile queues, stealing from the other XCDs' queues at the end.
    Against the oracle, and bit for bit against the same plan in launch order
    (one workgroup per tile) in deterministic mode."""
    cfg = _small(512, 64, 8192, 3, 2, 4, 16, "bf16", seed=71)
    inp = synth.make_inputs(cfg)
    d = ops.dims_for(cfg, deterministic=True)
    plan = ops.forward_plan(d)
    assert (plan["gemm_rows"], plan["order"], plan["ksplit_gate_up"]) == (256, 2, 1)
    _, _, out, _ = _layer(cfg, inp, d)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w)
    assert_close(to_f64(out), ref, "bf16", "persistent gate_up")
    for _ in range(2):  # the queues start empty on every call
        _, _, again, _ = _layer(cfg, inp, d)
        assert torch.equal(again, out)
    d1 = ops.dims_for(cfg, deterministic=True, plan=dict(plan, order=1))
    _, _, out1, _ = _layer(cfg, inp, d1)
    assert torch.equal(out1, out)


def test_forward_tile_boundaries():
    """Routing crafted so that, with 256-row tiles, one expert's last tile has
    exactly 128 rows (the largest tile whose second wave row has no rows),
    another has 129 (the smallest with rows in both), a third exactly 256 and a
    fourth 256 + 44."""
    sizes = [384, 129, 256, 300]
    cfg = _small(sum(sizes), 128, 192, len(sizes), 1, 3, 32, "bf16", seed=21)
    inp = synth.make_inputs(cfg)
    owner = np.repeat(np.arange(len(sizes)), sizes)
    np.random.default_rng(4).shuffle(owner)
    logits = np.zeros((cfg.tokens, len(sizes)), np.float32)
    logits[np.arange(cfg.tokens), owner] = 4.0
    inp["logits"] = logits
    assert ops.forward_fusion(ops.dims_for(cfg)) == {"gate_up": True, "down": True, "down_shrink": False}
    _, (ids, w, ss, off), out, _ = _layer(cfg, inp)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.array_equal(np.bincount(ref_ids.ravel(), minlength=len(sizes)), sizes)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w)
    assert_close(to_f64(out), ref, cfg.dtype, "out")


def test_stream_k_down_projection():
    """The down projection's stream-K launch.  With 256-row tiles, h = 4096 (16
    N-tiles) and 20 M-tiles, the 320 tiles exceed one round of 256 workgroups:
    the last 64 tiles' 16 K-steps each are cut into 256 equal ranges (four
    workgroups per tile adding their parts with atomics, the one holding K-step
    0 adding the LoRA expand).  Full output against the oracle, with the
    workspace filled with NaN first (the data-parallel launch must clear every
    stream-K tile), also with base-only tokens; the deterministic mode, which
    has no stream-K, agrees within the same bound."""
    cfg = _small(2048, 4096, 1024, 5, 2, 4, 16, "bf16", seed=31, requests=32)
    inp = synth.make_inputs(cfg)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    rows = np.bincount(ref_ids.ravel(), minlength=cfg.experts)
    tiles = int(sum((rows + 255) // 256)) * (cfg.hidden // 256)
    assert tiles > 256 and 0 < tiles % 256 <= 204, (rows, tiles)
    plan = dict(gemm_rows=256, gemm_form=2)
    dev = device()
    for det, base_only in [(False, False), (True, False), (False, True)]:
        case = dict(inp)
        if base_only:
            rng = np.random.default_rng(5)
            case["adapter_ids"] = np.where(rng.random(cfg.tokens) < 0.3, -1,
                                           inp["adapter_ids"]).astype(np.int32)
        d = ops.dims_for(cfg, deterministic=det, base_only=base_only, plan=plan)
        assert ops.forward_plan(d)["ksplit_down"] == 1 and ops.forward_fusion(d)["down"]
        say(f"stream-K shape, deterministic={det}, base_only={base_only}")
        dinp = device_inputs(case, cfg, dev)
        ids, w, ss, off, st = run_align(cfg, dinp, dims=d)
        assert int(st[0].item()) == 0
        ws = ops.workspace(ops.forward_workspace_size(d), dev)
        ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
        out, _ = run_forward(cfg, dinp, w, ss, off, dims=d, workspace_buf=ws)
        ref = oracle.forward(case, oracle.dims_of(cfg), ref_ids, ref_w)
        assert_close(to_f64(out), ref, cfg.dtype, f"out det={det} base_only={base_only}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_intermediates(dtype):
    """Layer-by-layer reconciliation: G, Z1, ACT, Z2, D read from the workspace
    against the oracle's per-slot intermediates (bf16: unfused, so that G is
    written; ACT is then bf16)."""
    cfg = _small(96, 192, 320, 5, 2, 3, 32, dtype, seed=5)
    inp = synth.make_inputs(cfg)
    d = ops.dims_for(cfg, unfused=True)
    _, (ids, w, ss, off), out, ws = _layer(cfg, inp, d)
    lay = ops.forward_workspace_layout(d)
    S, I, h, r = cfg.slots, cfg.intermediate, cfg.hidden, cfg.rank
    G = to_f64(workspace_view(ws, lay["G"], (S, 2 * I), torch.float32))
    Z1 = to_f64(workspace_view(ws, lay["Z1"], (S, r), torch.float32))
    ACT = to_f64(workspace_view(ws, lay["ACT"], (S, I), torch.float32 if dtype == "f32" else torch.bfloat16))
    Z2 = to_f64(workspace_view(ws, lay["Z2"], (S, r), torch.float32))
    D = to_f64(workspace_view(ws, lay["D"], (S, h), torch.float32))
    ss = ss.cpu().numpy()
    ids = ids.cpu().numpy()
    dims = oracle.dims_of(cfg)
    base_inp = dict(inp, b_gate_up=np.zeros_like(inp["b_gate_up"]))
    for p in sample_tokens(S, 20, seed=3):
        s = int(ss[p])
        t, j = divmod(s, cfg.top_k)
        e, l = int(ids[t, j]), int(inp["adapter_ids"][t])
        ref = oracle.slot(inp, dims, t, e, l)
        base = oracle.slot(base_inp, dims, t, e, l)["g"]   # xW alone
        assert_close(G[p], base, "f32", f"G p={p}")
        assert_close(Z1[p], ref["z1"], "f32", f"Z1 p={p}")
        assert_close(ACT[p], ref["a"], dtype, f"ACT p={p}")
        assert_close(Z2[p], ref["z2"], dtype, f"Z2 p={p}")
        assert_close(D[p], ref["d"], dtype, f"D p={p}")


@pytest.mark.parametrize("T", [128, 24])   # LDS-tiled GEMM / weight-streaming GEMM
def test_integer_exact_gate_up(T):
    """x, W, A, B in {-2..2} (exact in bf16); every partial sum of xW and xA stays
    below 2^24, so the GPU's G = xW and Z1 = xA are exact in fp32 whatever the
    summation order (split-K atomics included) and must equal the oracle's bit
    for bit."""
    cfg = _small(T, 4096, 256, 4, 2, 3, 32, "bf16", seed=9)
    rng = np.random.default_rng(11)
    inp = synth.make_inputs(cfg)
    for n in ["x"] + WEIGHTS:
        inp[n] = synth.from_float(rng.integers(-2, 3, inp[n].shape).astype(np.float32), "bf16")
    d = ops.dims_for(cfg, unfused=True)
    _, (ids, w, ss, off), out, ws = _layer(cfg, inp, d)
    lay = ops.forward_workspace_layout(d)
    S, I, r = cfg.slots, cfg.intermediate, cfg.rank
    G = to_f64(workspace_view(ws, lay["G"], (S, 2 * I), torch.float32))
    Z1 = to_f64(workspace_view(ws, lay["Z1"], (S, r), torch.float32))
    ss, ids = ss.cpu().numpy(), ids.cpu().numpy()
    dims = oracle.dims_of(cfg)
    base_inp = dict(inp, b_gate_up=np.zeros_like(inp["b_gate_up"]))
    for p in range(0, S, 7):
        t, j = divmod(int(ss[p]), cfg.top_k)
        e, l = int(ids[t, j]), int(inp["adapter_ids"][t])
        ref = oracle.slot(base_inp, dims, t, e, l)
        assert np.array_equal(G[p], ref["g"]), p
        assert np.array_equal(Z1[p], ref["z1"]), p


def test_zero_lora_matches_between_a_and_b():
    """A = 0 and B = 0 both make the LoRA term exactly zero: the two GPU runs
    must agree bit for bit, and match the oracle's base MoE."""
    cfg = _small(200, 320, 192, 6, 2, 3, 64, "bf16", seed=13)
    inp = synth.make_inputs(cfg)
    zb = dict(inp, b_gate_up=np.zeros_like(inp["b_gate_up"]), b_down=np.zeros_like(inp["b_down"]))
    za = dict(inp, a_gate_up=np.zeros_like(inp["a_gate_up"]), a_down=np.zeros_like(inp["a_down"]))
    _, _, out_b, _ = _layer(cfg, zb)
    _, _, out_a, _ = _layer(cfg, za)
    assert torch.equal(out_a, out_b)
    ids, w = oracle.route(inp["logits"], cfg.top_k)
    assert_close(to_f64(out_b), oracle.forward(zb, oracle.dims_of(cfg), ids, w), "bf16", "base")


def test_forward_with_oracle_permutation():
    """Forward fed with the oracle's routing and permutation (isolates align)."""
    cfg = _small(150, 256, 320, 7, 3, 5, 32, "bf16", seed=17)
    inp = synth.make_inputs(cfg)
    dev = device()
    dinp = device_inputs(inp, cfg, dev)
    ids, w = oracle.route(inp["logits"], cfg.top_k)
    ss, off = oracle.align(ids, inp["adapter_ids"], cfg.experts, cfg.adapters)
    out, _ = run_forward(cfg, dinp, torch.from_numpy(w.astype(np.float32)).to(dev),
                         torch.from_numpy(ss).to(dev), torch.from_numpy(off).to(dev))
    assert_close(to_f64(out), oracle.forward(inp, oracle.dims_of(cfg), ids, w), "bf16", "out")


def test_forward_after_align_topk():
    """A caller that routes itself: its own expert ids (one token repeats an
    expert) and weights (not a softmax) through moelora_align_topk and forward."""
    cfg = _small(300, 256, 320, 6, 2, 4, 32, "bf16", seed=23)
    inp = synth.make_inputs(cfg)
    dev = device()
    dinp = device_inputs(inp, cfg, dev)
    rng = np.random.default_rng(29)
    ids = np.stack([rng.permutation(cfg.experts)[:cfg.top_k] for _ in range(cfg.tokens)]).astype(np.int32)
    ids[5] = ids[5, 0]
    w = rng.uniform(0.1, 1.0, ids.shape).astype(np.float32)
    ss, off, st = ops.align_topk(ops.dims_for(cfg), torch.from_numpy(ids).to(dev), dinp["adapter_ids"])
    torch.cuda.synchronize()
    assert int(st[0].item()) == 0
    out, _ = run_forward(cfg, dinp, torch.from_numpy(w).to(dev), ss, off)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ids.astype(np.int64), w.astype(np.float64))
    assert_close(to_f64(out), ref, "bf16", "out")


def test_canaries_and_second_stream():
    """Guard bytes around the output and the workspace stay untouched, and a run
    on a second stream with its own workspace gives the same result."""
    cfg = _small(96, 192, 320, 5, 2, 3, 32, "bf16", seed=19)
    inp = synth.make_inputs(cfg)
    dev = device()
    dinp = device_inputs(inp, cfg, dev)
    d = ops.dims_for(cfg)
    ids, w, ss, off, _ = run_align(cfg, dinp)
    G = 4096
    wsz = ops.forward_workspace_size(d)
    ws_full = torch.full((wsz + 2 * G,), 0xA5, dtype=torch.uint8, device=dev)
    out_full = torch.full((cfg.tokens * cfg.hidden + 2 * G,), 7.0, dtype=torch.bfloat16, device=dev)
    ws = ws_full[G:G + wsz]
    out = out_full[G:G + cfg.tokens * cfg.hidden].view(cfg.tokens, cfg.hidden)
    ops.forward(d, dinp["x"], *[dinp[n] for n in WEIGHTS], w, ss, off, out=out, workspace_buf=ws)
    torch.cuda.synchronize()
    assert torch.all(ws_full[:G] == 0xA5) and torch.all(ws_full[G + wsz:] == 0xA5)
    assert torch.all(out_full[:G] == 7.0) and torch.all(out_full[G + cfg.tokens * cfg.hidden:] == 7.0)
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        out2 = ops.forward(d, dinp["x"], *[dinp[n] for n in WEIGHTS], w, ss, off)
    s2.synchronize()
    ids_ref, w_ref = oracle.route(inp["logits"], cfg.top_k)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ids_ref, w_ref)
    assert_close(to_f64(out), ref, "bf16", "stream 1")
    assert_close(to_f64(out2), ref, "bf16", "stream 2")


DET_SHAPES = [
    (96, 128, 2048, 1, 1, 4, 16, "bf16"),    # down GEMM split over K
    (64, 256, 512, 8, 2, 4, 16, "f32"),      # short buckets: k_shrink
    (600, 128, 192, 4, 2, 3, 16, "bf16"),    # tall buckets: DMA shrink, fused epilogues
    (520, 192, 256, 2, 1, 9, 64, "bf16"),
    (600, 192, 128, 4, 2, 2, 32, "f32"),     # tall fp32 shrink
    STREAM_SHAPE,                            # streaming shrink: one partial per K chunk
    STREAM_SHAPES_R32_R16[0],
]


@pytest.mark.parametrize("shape", DET_SHAPES, ids=lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s" % s)
def test_deterministic_mode_is_bit_reproducible(shape):
    """MOELORA_FLAG_DETERMINISTIC: three runs, each on a fresh workspace filled
    with NaN (nothing may rely on cleared memory), give the same output bit for
    bit, within tolerance of the oracle."""
    cfg = _small(*shape, seed=sum(shape[:7]) + 1)
    inp = synth.make_inputs(cfg)
    dev = device()
    dinp = device_inputs(inp, cfg, dev)
    _, w, ss, off, st = run_align(cfg, dinp)
    d = ops.dims_for(cfg, deterministic=True)
    outs = []
    for _ in range(3):
        ws = ops.workspace(ops.forward_workspace_size(d), dev)
        ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
        out, _ = run_forward(cfg, dinp, w, ss, off, dims=d, workspace_buf=ws)
        outs.append(out.clone())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                           outs[0].view(torch.int16) if o.dtype == torch.bfloat16 else outs[0].view(torch.int32))
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w)
    assert_close(to_f64(outs[0]), ref, cfg.dtype, "out")


def test_deterministic_mode_dense_workload():
    """The dense workload splits its down GEMM 16 ways: deterministic mode gives
    identical outputs on two runs and stays within tolerance on sampled tokens."""
    cfg = synth.WORKLOADS["dense_h8192"]
    inp = synth.make_inputs(cfg)
    dev = device()
    dinp = device_inputs(inp, cfg, dev)
    _, w, ss, off, st = run_align(cfg, dinp)
    d = ops.dims_for(cfg, deterministic=True)
    ws = ops.workspace(ops.forward_workspace_size(d), dev)
    a, _ = run_forward(cfg, dinp, w, ss, off, dims=d, workspace_buf=ws)
    a = a.clone()
    b, _ = run_forward(cfg, dinp, w, ss, off, dims=d, workspace_buf=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    toks = sample_tokens(cfg.tokens, 16)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w, tokens=toks)
    assert_close(to_f64(a)[toks], ref, cfg.dtype, "dense det out")


BASE_ONLY_SHAPES = [
    (64, 256, 512, 8, 2, 4, 16, "bf16", 0.3),    # 32-row tiles
    (96, 192, 320, 5, 2, 3, 32, "f32", 0.3),     # 64-row tiles, fp32
    (200, 320, 192, 6, 2, 3, 64, "bf16", 0.3),   # 128-row tiles
    (600, 128, 192, 4, 2, 3, 16, "bf16", 0.3),   # 256-row tiles: fused epilogues, DMA shrink
    (600, 192, 128, 4, 2, 2, 32, "f32", 0.5),    # 256-row fp32 tiles, tall shrink
    (96, 128, 2048, 1, 1, 4, 16, "bf16", 0.3),   # split-K down GEMM
    (300, 128, 256, 3, 2, 2, 32, "bf16", 1.0),   # every token base-only
    STREAM_SHAPE + (0.3,),                       # streaming shrink over base-only tiles
]


@pytest.mark.parametrize("shape", BASE_ONLY_SHAPES, ids=lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s_p%.1f" % s)
@pytest.mark.parametrize("det", [False, True], ids=["atomics", "deterministic"])
def test_forward_base_only_tokens(shape, det):
    """MOELORA_FLAG_BASE_ONLY: tokens with adapter id -1 get the base MoE output
    (no LoRA term), the others their adapter's, against the oracle."""
    *dims, frac = shape
    cfg = _small(*dims, seed=sum(dims[:7]) + 3)
    inp = synth.make_inputs(cfg)
    rng = np.random.default_rng(cfg.tokens)
    inp["adapter_ids"] = np.where(rng.random(cfg.tokens) < frac, -1, inp["adapter_ids"]).astype(np.int32)
    dev = device()
    dinp = device_inputs(inp, cfg, dev)
    d = ops.dims_for(cfg, deterministic=det, base_only=True)
    ids, w, ss, off, st = run_align(cfg, dinp, dims=d)
    assert int(st[0].item()) == 0
    ws = ops.workspace(ops.forward_workspace_size(d), dev)
    ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    out, _ = run_forward(cfg, dinp, w, ss, off, dims=d, workspace_buf=ws)
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    ref = oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w)
    assert_close(to_f64(out), ref, cfg.dtype, "out")


FOLD_SHAPES = [(64, 256, 512, 8, 2, 4, 16, "bf16"), (96, 192, 320, 5, 2, 3, 32, "bf16"),
               (200, 320, 192, 6, 2, 3, 64, "bf16"), (350, 192, 320, 4, 2, 3, 32, "bf16"),
               (600, 128, 192, 4, 2, 3, 16, "bf16"), (700, 256, 320, 3, 2, 5, 32, "bf16")]


@pytest.mark.parametrize("in_out", [False, True], ids=["k_contig", "in_out"])
@pytest.mark.parametrize("det", [False, True], ids=["atomics", "deterministic"])
@pytest.mark.parametrize("shape", FOLD_SHAPES, ids=lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s" % s)
def test_folded_down_shrink_z2(shape, det, in_out):
    """Plan fuse = 3: the down projection's shrink folded into the fused
    gate_up epilogue (every fused tile family the automatic plan picks: 32-,
    64-row, 128-row streaming and reuse, 256-row; both weight layouts): Z2
    read back from the workspace against the oracle's z2 = a A_dn per slot,
    and the layer output against the oracle."""
    _check_folded(shape, det, in_out, dict(fuse=3))


@pytest.mark.parametrize("in_out", [False, True], ids=["k_contig", "in_out"])
@pytest.mark.parametrize("det", [False, True], ids=["atomics", "deterministic"])
@pytest.mark.parametrize("shape", FOLD_SHAPES[1:4], ids=lambda s: "T%d_h%d_I%d_E%d_k%d_L%d_r%d_%s" % s)
def test_folded_down_shrink_z2_dma128(shape, det, in_out):
    """The same on the 128 x 256 DMA tiles (plan form 3)."""
    _check_folded(shape, det, in_out, dict(fuse=3, gemm_rows=128, gemm_form=3))


def _check_folded(shape, det, in_out, plan):
    from gpu_util import in_out as to_in_out
    cfg = _small(*shape, seed=sum(shape[:7]) + 11)
    inp = synth.make_inputs(cfg)
    d = ops.dims_for(cfg, deterministic=det, in_out=in_out, plan=plan)
    assert ops.forward_fusion(d)["down_shrink"] and ops.forward_plan(d)["fuse"] == 3
    assert not ops.forward_fusion(ops.dims_for(cfg))["down_shrink"]   # never automatic
    if "gemm_form" in plan:
        assert ops.forward_plan(d)["gemm_form"] == plan["gemm_form"]
    _, (ids, w, ss, off), out, ws = _layer(cfg, to_in_out(inp) if in_out else inp, d)
    lay = ops.forward_workspace_layout(d)
    S, r = cfg.slots, cfg.rank
    Z2 = to_f64(workspace_view(ws, lay["Z2"], (S, r), torch.float32))
    ss, ids_h = ss.cpu().numpy(), ids.cpu().numpy()
    dims = oracle.dims_of(cfg)
    ref_z2 = np.stack([oracle.slot(inp, dims, int(ss[p]) // cfg.top_k,
                                   int(ids_h[int(ss[p]) // cfg.top_k, int(ss[p]) % cfg.top_k]),
                                   int(inp["adapter_ids"][int(ss[p]) // cfg.top_k]))["z2"]
                       for p in range(S)])
    assert_close(Z2, ref_z2, "bf16", "Z2")
    ref_ids, ref_w = oracle.route(inp["logits"], cfg.top_k)
    assert_close(to_f64(out), oracle.forward(inp, oracle.dims_of(cfg), ref_ids, ref_w), "bf16", "out")
