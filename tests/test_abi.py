"""The C-ABI library on the CPU: it loads, exports every function that
include/moelora.h declares, and rejects bad arguments before any HIP call.
No kernel is launched here."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (binds the library to torch's HIP runtime)

from moe_lora_layer_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moelora.h")

OK, ERR_NULL, ERR_DIMS, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_WORKSPACE, ERR_HIP = range(7)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moelora_\w+)\s*\(", text)))


def good_dims(**kw):
    base = dict(tokens=64, hidden=256, intermediate=512, experts=8, top_k=2, adapters=4, rank=16,
                dtype="bf16")
    base.update(kw)
    return ops.make_dims(**base)


def test_library_exports_every_declared_function():
    lib = ops.library()
    names = declared_functions()
    assert {"moelora_align", "moelora_forward"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.moelora_abi_version() == 8


def test_status_strings():
    for rc in range(8):
        s = ops.status_string(rc)
        assert s.startswith("moelora:")
    assert "unknown" in ops.status_string(99)


@pytest.mark.parametrize("kw,rc", [
    (dict(dtype=7), ERR_UNSUPPORTED), (dict(rank=8), ERR_UNSUPPORTED), (dict(rank=128), ERR_UNSUPPORTED),
    (dict(hidden=100), ERR_DIMS), (dict(intermediate=96), ERR_DIMS), (dict(tokens=-1), ERR_DIMS),
    (dict(top_k=9, experts=16), ERR_DIMS), (dict(top_k=3, experts=2), ERR_DIMS), (dict(experts=0), ERR_DIMS),
    (dict(adapters=0), ERR_DIMS), (dict(experts=256, adapters=257), ERR_DIMS),
    (dict(experts=1, top_k=1, adapters=65537), ERR_DIMS), (dict(experts=1, top_k=1, adapters=65536), OK),
    (dict(experts=256, adapters=256), OK), (dict(experts=256, adapters=256, flags=2), OK),
    (dict(tokens=1 << 30, top_k=2), ERR_DIMS), (dict(flags=8), OK), (dict(flags=16), ERR_UNSUPPORTED),
    (dict(flags=15), OK),
    (dict(flags=-1), ERR_UNSUPPORTED), (dict(flags=3), OK), (dict(flags=7), OK),
    (dict(experts=128, adapters=64), OK), (dict(experts=128, adapters=64, flags=2), OK),
])
def test_dims_validation(kw, rc):
    d = good_dims(**kw)
    n = ctypes.c_size_t()
    lib = ops.library()
    assert lib.moelora_forward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == rc
    assert lib.moelora_align_workspace_size(ctypes.byref(d), ctypes.byref(n)) == rc


def test_null_dims_and_outputs():
    lib = ops.library()
    n = ctypes.c_size_t()
    assert lib.moelora_forward_workspace_size(None, ctypes.byref(n)) == ERR_NULL
    assert lib.moelora_forward_workspace_size(ctypes.byref(good_dims()), None) == ERR_NULL
    assert lib.moelora_forward_workspace_layout(ctypes.byref(good_dims()), None) == ERR_NULL


def test_workspace_sizes_and_layout():
    d = good_dims(tokens=100, hidden=320, intermediate=192, experts=5, top_k=2, adapters=3, rank=32,
                  unfused=True)
    fused = good_dims(tokens=100, hidden=320, intermediate=192, experts=5, top_k=2, adapters=3, rank=32)
    # the fused gate_up GEMM never writes G: the workspace holds no bytes for it
    assert ops.forward_workspace_size(fused) <= ops.forward_workspace_size(d) - 200 * 2 * 192 * 4
    size = ops.forward_workspace_size(d)
    lay = ops.forward_workspace_layout(d)
    S, I, h, r = 200, 192, 320, 32
    extent = {"G": S * 2 * I * 4, "Z1": S * r * 4, "ACT": S * I * 2, "Z2": S * r * 4, "D": S * h * 4}
    assert all(o % 16 == 0 for o in lay.values())
    spans = sorted((lay[n], lay[n] + extent[n], n) for n in extent)
    for (a0, a1, na), (b0, b1, nb) in zip(spans, spans[1:]):
        assert a1 <= b0, (na, nb)          # no two intermediates overlap
    assert spans[-1][1] <= size
    assert lay["Z2"] == lay["Z1"] + S * r * 4 and lay["D"] == lay["Z2"] + S * r * 4
    assert ops.align_workspace_size(d) >= 2 * S * 4
    assert ops.forward_workspace_size(good_dims(tokens=0)) == 0


def _vp(v):
    return ctypes.c_void_p(v)


def test_align_argument_errors():
    lib = ops.library()
    d = good_dims()
    fake = 1 << 20
    ws = ops.align_workspace_size(d)
    args = [_vp(fake)] * 7
    # NULL output
    a = list(args); a[4] = None
    assert lib.moelora_align(ctypes.byref(d), *a[:6], None, _vp(fake), ws, None) == ERR_NULL
    # workspace too small / missing
    assert lib.moelora_align(ctypes.byref(d), *args[:6], None, _vp(fake), ws - 1, None) == ERR_WORKSPACE
    assert lib.moelora_align(ctypes.byref(d), *args[:6], None, None, ws, None) == ERR_WORKSPACE
    # misaligned pointer
    a = list(args); a[1] = _vp(fake + 4)
    assert lib.moelora_align(ctypes.byref(d), *a[:6], None, _vp(fake), ws, None) == ERR_ALIGNMENT
    # bad dims first
    bad = good_dims(rank=3)
    assert lib.moelora_align(ctypes.byref(bad), *args[:6], None, _vp(fake), ws, None) == ERR_UNSUPPORTED


def test_forward_argument_errors():
    lib = ops.library()
    d = good_dims()
    fake = 1 << 20
    ws = ops.forward_workspace_size(d)
    ptrs = [_vp(fake)] * 12
    p = list(ptrs); p[3] = None
    assert lib.moelora_forward(ctypes.byref(d), *p, _vp(fake), ws, None) == ERR_NULL
    assert lib.moelora_forward(ctypes.byref(d), *ptrs, _vp(fake), ws - 1, None) == ERR_WORKSPACE
    assert lib.moelora_forward(ctypes.byref(d), *ptrs, None, ws, None) == ERR_WORKSPACE
    p = list(ptrs); p[0] = _vp(fake + 2)
    assert lib.moelora_forward(ctypes.byref(d), *p, _vp(fake), ws, None) == ERR_ALIGNMENT
    assert lib.moelora_forward(ctypes.byref(d), *ptrs, _vp(fake + 8), ws, None) == ERR_ALIGNMENT
    # T == 0 is a no-op that touches nothing
    z = good_dims(tokens=0)
    assert lib.moelora_forward(ctypes.byref(z), *([None] * 12), None, 0, None) == OK
    # topk_ids (argument 8) may be NULL: not read by any kernel
    p = list(ptrs); p[7] = None
    assert lib.moelora_forward(ctypes.byref(d), *p, _vp(fake), ws - 1, None) == ERR_WORKSPACE


@pytest.mark.parametrize("kw,flags", [
    (dict(), {"gate_up": True, "down": True, "down_shrink": False}),                            # 16 rows per expert
    (dict(unfused=True), {"gate_up": False, "down": False, "down_shrink": False}),
    (dict(tokens=4096, hidden=4096, intermediate=11008, experts=16), {"gate_up": True, "down": True, "down_shrink": False}),
    (dict(tokens=4096, hidden=4096, intermediate=11008, experts=16, dtype="f32"),
     {"gate_up": False, "down": False, "down_shrink": False}),                                   # fused forms are bf16 only
    (dict(tokens=4096, hidden=4096, intermediate=11008, experts=16, unfused=True),
     {"gate_up": False, "down": False, "down_shrink": False}),
    (dict(tokens=600, hidden=128, intermediate=192, experts=4), {"gate_up": True, "down": True, "down_shrink": False}),
    # 32 rows per expert over 64 adapters: 64-row tiles stage the buckets' B in LDS
    (dict(tokens=256, hidden=2880, intermediate=2880, experts=32, top_k=4, adapters=64, rank=64),
     {"gate_up": True, "down": True, "down_shrink": False}),
    # 128 rows per expert over 16 adapters (eight-wave tiles): the gate_up GEMM
    # fuses; the down GEMM (N = 8192, one M-tile) splits K and does not
    (dict(tokens=128, hidden=8192, intermediate=28672, experts=1, top_k=1, adapters=16),
     {"gate_up": True, "down": False, "down_shrink": False}),
    # one token on one expert: both GEMMs split K to fill the GPU, no fusion
    (dict(tokens=4, hidden=4096, intermediate=1024, experts=1, top_k=1), {"gate_up": False, "down": False, "down_shrink": False}),
])
def test_forward_fusion_flags(kw, flags):
    assert ops.forward_fusion(good_dims(**kw)) == flags


def test_forward_fusion_rejects_null_and_bad_dims():
    lib = ops.library()
    assert lib.moelora_forward_fusion(ctypes.byref(good_dims()), None) == ERR_NULL
    f = ctypes.c_int()
    assert lib.moelora_forward_fusion(ctypes.byref(good_dims(rank=8)), ctypes.byref(f)) == ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(), dict(tokens=96, hidden=128, intermediate=2048, experts=1, top_k=1),
                                dict(tokens=4096, hidden=4096, intermediate=11008, experts=16)])
def test_deterministic_workspace_holds_the_partials(kw):
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    lib = ops.library()
    assert lib.moelora_forward_workspace_size(ctypes.byref(good_dims(**kw)), ctypes.byref(n0)) == OK
    assert lib.moelora_forward_workspace_size(ctypes.byref(good_dims(flags=1, **kw)), ctypes.byref(n1)) == OK
    # tall bf16 LoRA tiles (the third shape) sum shrink partials in both modes
    tall = ops.forward_plan(good_dims(**kw))["lora_rows"] == 64
    assert n1.value >= n0.value if tall else n1.value > n0.value


# ---------------------------------------------------------------- tile plans
PLAN_CASES = [
    dict(gemm_rows=48), dict(gemm_rows=-32), dict(gemm_form=3), dict(gemm_form=1),  # form needs rows
    dict(gemm_rows=256, gemm_form=1), dict(gemm_rows=64, gemm_form=2), dict(lora_rows=32),
    dict(ksplit_gate_up=-1), dict(ksplit_down=1025), dict(fuse=4), dict(fuse=-1), dict(order=6),
    dict(order=-1), dict(gemm_rows=64, gemm_form=3), dict(gemm_rows=256, gemm_form=3),
    dict(gemm_form=4),
]


@pytest.mark.parametrize("plan", PLAN_CASES)
def test_bad_plans_are_refused_everywhere(plan):
    d = good_dims(plan=plan)
    n = ctypes.c_size_t()
    lib = ops.library()
    assert lib.moelora_forward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == ERR_UNSUPPORTED
    assert lib.moelora_align_workspace_size(ctypes.byref(d), ctypes.byref(n)) == ERR_UNSUPPORTED
    out = ops.Plan()
    assert lib.moelora_forward_plan(ctypes.byref(d), ctypes.byref(out)) == ERR_UNSUPPORTED
    dd = ops.make_dense_dims(64, 256, 512, 4, 16, "bf16", plan=plan)
    assert lib.moelora_dense_workspace_size(ctypes.byref(dd), ctypes.byref(n)) == ERR_UNSUPPORTED


def test_dma128_tiles_are_bf16_only():
    # plan form 3 (128 x 256 DMA tiles) resolves for bf16 and is refused for fp32
    p = ops.forward_plan(good_dims(plan=dict(gemm_rows=128, gemm_form=3)))
    assert (p["gemm_rows"], p["gemm_form"]) == (128, 3)
    n = ctypes.c_size_t()
    lib = ops.library()
    d = good_dims(dtype="f32", plan=dict(gemm_rows=128, gemm_form=3))
    assert lib.moelora_forward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == ERR_UNSUPPORTED
    dd = ops.make_dense_dims(64, 256, 512, 4, 16, "f32", plan=dict(gemm_rows=128, gemm_form=3))
    assert lib.moelora_dense_workspace_size(ctypes.byref(dd), ctypes.byref(n)) == ERR_UNSUPPORTED


def test_plan_resolution():
    # automatic: every field resolved; a forced field is kept, the others stay automatic
    auto = ops.forward_plan(good_dims())
    assert all(auto[f] != 0 for f in ops.PLAN_FIELDS)
    assert auto == {"gemm_rows": 32, "gemm_form": 1, "lora_rows": 16, "ksplit_gate_up": 1,
                    "ksplit_down": 1, "fuse": 1, "order": 3}
    forced = ops.forward_plan(good_dims(plan=dict(gemm_rows=128, gemm_form=2, lora_rows=64)))
    # weight-reuse tiles default to the XCD-grouped order
    assert forced == dict(auto, gemm_rows=128, gemm_form=2, lora_rows=64, order=2)
    assert ops.forward_plan(good_dims(in_out=True))["order"] == 1
    assert ops.forward_plan(good_dims(plan=dict(order=4)))["order"] == 4
    # resolving a resolved plan changes nothing
    for kw in [dict(), dict(tokens=4096, hidden=4096, intermediate=11008, experts=16),
               dict(tokens=4, hidden=4096, intermediate=1024, experts=1, top_k=1)]:
        p = ops.forward_plan(good_dims(**kw))
        assert ops.forward_plan(good_dims(plan=p, **kw)) == p
    # split counts: capped at the K-steps and rounded so that no K range is empty
    # (h = 256: 4 steps of 64; I = 512: 8 steps)
    p = ops.forward_plan(good_dims(plan=dict(ksplit_gate_up=3, ksplit_down=1000)))
    assert (p["ksplit_gate_up"], p["ksplit_down"]) == (2, 8)
    # a split GEMM cannot fuse its expand; fuse=2 turns fusion off
    assert ops.forward_fusion(good_dims(plan=dict(ksplit_down=2))) == {"gate_up": True, "down": False, "down_shrink": False}
    assert ops.forward_fusion(good_dims(plan=dict(fuse=2))) == {"gate_up": False, "down": False, "down_shrink": False}
    many = dict(tokens=256, hidden=2880, intermediate=2880, experts=32, top_k=4, adapters=64, rank=64)
    assert ops.forward_fusion(good_dims(plan=dict(fuse=1), **many)) == {"gate_up": True, "down": True, "down_shrink": False}
    # the workspace follows the plan (split partials in deterministic mode)
    n1 = ops.forward_workspace_size(good_dims(flags=1))
    n2 = ops.forward_workspace_size(good_dims(flags=1, plan=dict(ksplit_down=4)))
    assert n2 > n1


def test_dense_plan():
    dd = ops.make_dense_dims(128, 8192, 10240, 16, 16, "bf16")
    p = ops.dense_forward_plan(dd)
    assert p["ksplit_gate_up"] == 0 and p["ksplit_down"] > 1
    n = ctypes.c_size_t()
    bad = ops.make_dense_dims(128, 8192, 10240, 16, 16, "bf16", plan=dict(ksplit_gate_up=2))
    assert ops.library().moelora_dense_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == ERR_UNSUPPORTED
    assert ops.dense_forward_plan(ops.make_dense_dims(128, 8192, 10240, 16, 16, "bf16",
                                                      plan=dict(ksplit_down=1)))["ksplit_down"] == 1


def test_dense_automatic_plan_fills_one_round():
    # 128 rows: the 128-row weight-streaming tiles would make 80 workgroups for
    # 10240 outputs; the automatic plan takes the 128 x 256 DMA tiles (bf16:
    # 40 of them) split over K into about one round of 256 instead (6 splits),
    # fp32 the weight-reuse tiles (80, 3 splits), and keeps unsplit streaming
    # tiles when they fill a round by themselves (65536 outputs: 512 tiles;
    # bf16 streams them on the DMA tiles)
    p = ops.dense_forward_plan(ops.make_dense_dims(128, 8192, 10240, 16, 16, "bf16"))
    assert (p["gemm_rows"], p["gemm_form"], p["ksplit_down"]) == (128, 3, 6)
    p = ops.dense_forward_plan(ops.make_dense_dims(128, 8192, 10240, 16, 16, "f32"))
    assert (p["gemm_rows"], p["gemm_form"], p["ksplit_down"]) == (128, 2, 3)
    p = ops.dense_forward_plan(ops.make_dense_dims(128, 8192, 65536, 16, 16, "bf16"))
    assert (p["gemm_rows"], p["gemm_form"], p["ksplit_down"]) == (128, 3, 1)
    # decode-sized rows keep their own tiles; an explicit field is respected
    assert ops.dense_forward_plan(ops.make_dense_dims(16, 8192, 10240, 16, 16, "bf16"))["gemm_rows"] == 32
    p = ops.dense_forward_plan(ops.make_dense_dims(128, 8192, 10240, 16, 16, "bf16",
                                                   plan=dict(gemm_rows=128, gemm_form=1)))
    assert p["gemm_form"] == 1 and p["ksplit_down"] > 3  # the streaming rule: ~512 workgroups
    # a narrow output over a short K: the forced split keeps >= 8 K-steps per
    # split (96 rows, K 2048 = 32 steps, N 128: 4 splits, not 256 / 1)
    p = ops.dense_forward_plan(ops.make_dense_dims(96, 2048, 128, 4, 16, "bf16"))
    assert (p["gemm_rows"], p["gemm_form"], p["ksplit_down"]) == (128, 3, 4)


def test_plan_table_round_trip(tmp_path):
    from moe_lora_layer_amd import tune
    d = good_dims()
    dd = ops.make_dense_dims(128, 8192, 10240, 16, 16, "bf16")
    e1 = {"kind": "layer", "dims": {k: int(getattr(d, k)) for k in tune.LAYER_KEYS},
          "plan": dict(ops.forward_plan(d), gemm_rows=64), "us": 1.0, "auto_us": 2.0}
    e2 = {"kind": "dense", "dims": {k: int(getattr(dd, k)) for k in tune.DENSE_KEYS},
          "plan": ops.dense_forward_plan(dd), "us": 1.0, "auto_us": 1.0}
    path = str(tmp_path / "t.json")
    tune.save_table(path, tune.merge([], [e1, e2]))
    t = tune.load_table(path)
    assert tune.plan_for(d, t) == e1["plan"]
    assert tune.plan_for(dd, t) == e2["plan"]
    assert tune.plan_for(good_dims(tokens=65), t) is None
    # the plan field of the dims does not enter the key; a new entry replaces the old one
    assert tune.plan_for(good_dims(plan=dict(gemm_rows=256)), t) == e1["plan"]
    e1b = dict(e1, plan=dict(e1["plan"], gemm_rows=32))
    assert tune.plan_for(d, tune.merge(t, [e1b])) == e1b["plan"]
    # the packaged table's plans are all valid for their dims
    if os.path.exists(tune.PACKAGED_TABLE):
        for e in tune.load_table(tune.PACKAGED_TABLE):
            if e["kind"] == "layer":
                dims = ops.make_dims(*[e["dims"][k] for k in tune.LAYER_KEYS[:-1]],
                                     flags=e["dims"]["flags"], plan=e["plan"])
                assert ops.forward_plan(dims) == e["plan"]
            else:
                k = e["dims"]
                dims = ops.make_dense_dims(k["tokens"], k["in_features"], k["out_features"],
                                           k["adapters"], k["rank"], k["dtype"], plan=e["plan"])
                dims.flags = k["flags"]
                assert ops.dense_forward_plan(dims) == e["plan"]


def test_noalloc_refuses_before_touching_the_gpu():
    """moelora_forward_noalloc checks the dims and the static scratch's size on
    the host: a batch beyond the scratch (4096-token prefill) is refused with
    status 7, bad dims with their own status, T == 0 is a no-op."""
    lib = ops.library()
    fake = [_vp(1 << 20)] * 12
    big = good_dims(tokens=4096, hidden=4096, intermediate=11008, experts=16)
    assert ops.forward_workspace_size(big) > ops.NOALLOC_SCRATCH_BYTES
    assert lib.moelora_forward_noalloc(ctypes.byref(big), *fake, None) == 7
    assert lib.moelora_forward_noalloc(ctypes.byref(good_dims(rank=8)), *fake, None) == ERR_UNSUPPORTED
    assert lib.moelora_forward_noalloc(ctypes.byref(good_dims(tokens=0)), *([None] * 12), None) == OK
    assert "static scratch" in ops.status_string(7)
