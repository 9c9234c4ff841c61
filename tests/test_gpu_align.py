"""moelora_align on the GPU against the oracle: routing ids, the bucketed
permutation and the bucket offsets must be bit-exact; routing weights within
1e-6.  Runs through the C ABI (ops.align is ctypes marshalling only)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import device, run_align, say
from moe_lora_layer_amd import ops, synth

pytestmark = pytest.mark.gpu


def _check(cfg, rinp, repeats=1):
    dev = device()
    logits = torch.from_numpy(rinp["logits"]).to(dev)
    ad = torch.from_numpy(rinp["adapter_ids"]).to(dev)
    ref_ids, ref_w = oracle.route(rinp["logits"], cfg.top_k)
    ref_ss, ref_off = oracle.align(ref_ids, rinp["adapter_ids"], cfg.experts, cfg.adapters)
    first = None
    for rep in range(repeats):
        ids, w, ss, off, st = run_align(cfg, {"logits": logits, "adapter_ids": ad})
        got = (ids.cpu().numpy(), w.cpu().numpy(), ss.cpu().numpy(), off.cpu().numpy())
        assert int(st[0].item()) == 0
        assert np.array_equal(got[0], ref_ids), "topk ids"
        assert np.array_equal(got[2], ref_ss), "sorted slots"
        assert np.array_equal(got[3], ref_off), "bucket offsets"
        assert np.max(np.abs(got[1].astype(np.float64) - ref_w)) <= 1e-6 if got[1].size else True
        if first is None:
            first = got
        else:
            for a, b in zip(first, got):
                assert np.array_equal(a, b), "align is not deterministic"


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_align_workloads(name):
    cfg = synth.WORKLOADS[name]
    say(f"align {name}: T={cfg.tokens} E={cfg.experts} k={cfg.top_k} L={cfg.adapters}")
    _check(cfg, synth.make_routing_inputs(cfg), repeats=3)


def _cfg(T, E, k, L, seed=1, **kw):
    return synth.LayerConfig("edge", T, 64, 64, E, k, L, 16, "bf16", requests=T if T else 1,
                             seed=seed, **kw)


@pytest.mark.parametrize("T,E,k,L", [(1, 8, 2, 4), (1, 1, 1, 1), (3, 4, 4, 2), (1000, 32, 8, 16),
                                     (5000, 16, 2, 8), (257, 256, 8, 32), (70, 8192, 1, 1),
                                     (4096, 64, 6, 128), (20000, 2, 2, 3),
                                     # E * L = 65536 buckets, more than LDS holds
                                     # counters for: counters in the workspace
                                     (2048, 64, 4, 1024), (300, 256, 2, 256), (9000, 1, 1, 65536)])
def test_align_shapes(T, E, k, L):
    cfg = _cfg(T, E, k, L)
    say(f"align shape T={T} E={E} k={k} L={L}")
    _check(cfg, synth.make_routing_inputs(cfg), repeats=2)


def test_align_degenerate_routing():
    # every token on the same experts and adapter; ties everywhere; empty experts
    T, E, k, L = 700, 16, 3, 4
    cfg = _cfg(T, E, k, L)
    r = {"logits": np.zeros((T, E), np.float32), "adapter_ids": np.full(T, 2, np.int32)}
    _check(cfg, r, repeats=3)
    r = {"logits": np.tile(np.arange(E, dtype=np.float32)[::-1] // 4, (T, 1)).astype(np.float32),
         "adapter_ids": (np.arange(T) % L).astype(np.int32)}
    _check(cfg, r, repeats=2)


def test_align_empty_tokens():
    dev = device()
    d = ops.make_dims(0, 64, 64, 4, 2, 3, 16, "bf16")
    ids, w, ss, off, st = ops.align(d, torch.empty((0, 4), dtype=torch.float32, device=dev),
                                    torch.empty((0,), dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert off.cpu().numpy().tolist() == [0] * 13
    assert int(st[0].item()) == 0


def test_align_reports_bad_adapter():
    cfg = _cfg(50, 8, 2, 4)
    r = synth.make_routing_inputs(cfg)
    r["adapter_ids"][7] = 4        # out of range
    dev = device()
    _, _, ss, off, st = ops.align(ops.dims_for(cfg), torch.from_numpy(r["logits"]).to(dev),
                                  torch.from_numpy(r["adapter_ids"]).to(dev))
    torch.cuda.synchronize()
    assert int(st[0].item()) == 1
    # still a permutation of the slots, in bounds
    assert sorted(ss.cpu().numpy().tolist()) == list(range(100))


def _topk(cfg, ids, adapter_ids):
    dev = device()
    ss, off, st = ops.align_topk(ops.dims_for(cfg), torch.from_numpy(ids).to(dev),
                                 torch.from_numpy(adapter_ids).to(dev))
    torch.cuda.synchronize()
    return ss.cpu().numpy(), off.cpu().numpy(), int(st[0].item())


@pytest.mark.parametrize("T,E,k,L", [(1, 8, 2, 4), (3, 4, 4, 2), (1000, 32, 8, 16), (5000, 16, 2, 8),
                                     (70, 8192, 1, 1), (20000, 2, 2, 3)])
def test_align_topk_caller_ids(T, E, k, L):
    """moelora_align_topk with the caller's expert ids (repeats within a token
    allowed): the permutation and offsets equal the oracle's, bit for bit."""
    cfg = _cfg(T, E, k, L, seed=3)
    rng = np.random.default_rng(T + E)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ad = rng.integers(0, L, T).astype(np.int32)
    say(f"align_topk T={T} E={E} k={k} L={L}")
    ss, off, st = _topk(cfg, ids, ad)
    ref_ss, ref_off = oracle.align(ids, ad, E, L)
    assert st == 0
    assert np.array_equal(ss, ref_ss) and np.array_equal(off, ref_off)


def test_align_topk_equals_align_on_routed_ids():
    cfg = synth.WORKLOADS["prefill_h4096"]
    r = synth.make_routing_inputs(cfg)
    ref_ids, _ = oracle.route(r["logits"], cfg.top_k)
    dev = device()
    _, _, ss_a, off_a, _ = run_align(cfg, {"logits": torch.from_numpy(r["logits"]).to(dev),
                                           "adapter_ids": torch.from_numpy(r["adapter_ids"]).to(dev)})
    ss, off, st = _topk(cfg, ref_ids.astype(np.int32), r["adapter_ids"])
    assert st == 0
    assert np.array_equal(ss, ss_a.cpu().numpy()) and np.array_equal(off, off_a.cpu().numpy())


def test_align_topk_reports_bad_ids():
    cfg = _cfg(40, 8, 2, 4)
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 8, (40, 2)).astype(np.int32)
    ad = rng.integers(0, 4, 40).astype(np.int32)
    bad_e = ids.copy()
    bad_e[3, 1] = 8
    ss, _, st = _topk(cfg, bad_e, ad)
    assert st == 3 and sorted(ss.tolist()) == list(range(80))
    bad_l = ad.copy()
    bad_l[9] = -1
    assert _topk(cfg, ids, bad_l)[2] == 1
    assert _topk(cfg, bad_e, bad_l)[2] == 3      # the larger code is reported


@pytest.mark.parametrize("T,E,k,L", [(50, 8, 2, 4), (1000, 32, 8, 16), (5000, 16, 2, 8), (300, 64, 4, 1),
                                     (2000, 256, 2, 256)])
def test_align_base_only_tokens(T, E, k, L):
    """MOELORA_FLAG_BASE_ONLY: adapter id -1 goes to each expert's extra last
    bucket; routing and permutation equal the oracle's bit for bit, for
    moelora_align and moelora_align_topk."""
    cfg = _cfg(T, E, k, L, seed=6)
    r = synth.make_routing_inputs(cfg)
    rng = np.random.default_rng(T)
    ad = np.where(rng.random(T) < 0.3, -1, r["adapter_ids"]).astype(np.int32)
    dev = device()
    d = ops.dims_for(cfg, base_only=True)
    ids, w, ss, off, st = ops.align(d, torch.from_numpy(r["logits"]).to(dev), torch.from_numpy(ad).to(dev))
    torch.cuda.synchronize()
    ref_ids, _ = oracle.route(r["logits"], k)
    ref_ss, ref_off = oracle.align(ref_ids, ad, E, L, base_only=True)
    assert int(st[0].item()) == 0
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.array_equal(ss.cpu().numpy(), ref_ss) and np.array_equal(off.cpu().numpy(), ref_off)
    ss2, off2, st2 = ops.align_topk(d, ids, torch.from_numpy(ad).to(dev))
    torch.cuda.synchronize()
    assert int(st2[0].item()) == 0
    assert np.array_equal(ss2.cpu().numpy(), ref_ss) and np.array_equal(off2.cpu().numpy(), ref_off)


def test_align_minus_one_needs_the_flag():
    cfg = _cfg(20, 4, 2, 3)
    r = synth.make_routing_inputs(cfg)
    r["adapter_ids"][2] = -1
    dev = device()
    _, _, ss, _, st = ops.align(ops.dims_for(cfg), torch.from_numpy(r["logits"]).to(dev),
                                torch.from_numpy(r["adapter_ids"]).to(dev))
    torch.cuda.synchronize()
    assert int(st[0].item()) == 1 and sorted(ss.cpu().numpy().tolist()) == list(range(40))


@pytest.mark.parametrize("E,k", [(8, 2), (16, 4), (300, 8)])
def test_align_nan_logits(E, k):
    """NaN router logits rank below every number, as in the oracle: an all-NaN
    row takes experts 0..k-1, a row with some NaN keeps its numeric experts
    first; every id stays in range, so the other tokens' slots and the whole
    permutation are bit-exact; weights match on the rows without NaN."""
    T, L = 96, 4
    cfg = _cfg(T, E, k, L, seed=E)
    rinp = synth.make_routing_inputs(cfg)
    logits = rinp["logits"].copy()
    logits[0, :] = np.nan
    logits[17, 1] = np.nan
    logits[40, : E // 2] = np.nan
    logits[95, :] = np.nan
    say(f"align NaN logits E={E} k={k}")
    dev = device()
    ids, w, ss, off, st = run_align(cfg, {"logits": torch.from_numpy(logits).to(dev),
                                          "adapter_ids": torch.from_numpy(rinp["adapter_ids"]).to(dev)})
    ref_ids, ref_w = oracle.route(logits, k)
    ref_ss, ref_off = oracle.align(ref_ids, rinp["adapter_ids"], E, L)
    assert int(st[0].item()) == 0
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert ref_ids[0].tolist() == list(range(k))
    assert np.array_equal(ss.cpu().numpy(), ref_ss)
    assert np.array_equal(off.cpu().numpy(), ref_off)
    clean = ~np.isnan(logits).any(axis=1)
    assert np.max(np.abs(w.cpu().numpy()[clean].astype(np.float64) - ref_w[clean])) <= 1e-6
