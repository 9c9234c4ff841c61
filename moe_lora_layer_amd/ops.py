"""Python binding of libmoelora.so: the C ABI of include/moelora.h via ctypes.

Argument marshalling only.  Every step of the layer runs in the library's HIP
kernels; torch supplies device memory and the current stream.  There is no
fallback: if the library is missing, every call raises.

torch must be imported before the library is loaded, so that the library
binds to the HIP runtime torch already uses (one runtime per process).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoelora.so")

MOELORA_F32, MOELORA_BF16 = 0, 1
MOELORA_FLAG_DETERMINISTIC = 1
MOELORA_FLAG_BASE_ONLY = 2
MOELORA_FLAG_UNFUSED = 4
MOELORA_FLAG_IN_OUT = 8
STAGES = ["prep", "zero", "shrink_gate_up", "gemm_gate_up", "expand_gate_up", "shrink_down",
          "gemm_down", "expand_down", "combine"]
_TORCH_DT = {MOELORA_F32: torch.float32, MOELORA_BF16: torch.bfloat16}
_DT_NAME = {"f32": MOELORA_F32, "bf16": MOELORA_BF16}


PLAN_FIELDS = ["gemm_rows", "gemm_form", "lora_rows", "ksplit_gate_up", "ksplit_down", "fuse",
               "order"]


class Plan(ctypes.Structure):
    """moelora_plan: tile-plan overrides, 0 = automatic (include/moelora.h)."""
    _fields_ = [(f, ctypes.c_int32) for f in PLAN_FIELDS]

    def as_dict(self) -> dict:
        return {f: int(getattr(self, f)) for f in PLAN_FIELDS}


def make_plan(plan=None) -> Plan:
    """A Plan from None (all automatic), a Plan, or a dict of some of its fields."""
    if plan is None:
        return Plan()
    if isinstance(plan, Plan):
        return plan
    unknown = set(plan) - set(PLAN_FIELDS)
    if unknown:
        raise ValueError(f"unknown plan fields {sorted(unknown)}")
    return Plan(*[int(plan.get(f, 0)) for f in PLAN_FIELDS])


class Dims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("intermediate", ctypes.c_int64), ("experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("adapters", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("plan", Plan)]

    def __repr__(self):
        return ("Dims(T=%d, h=%d, I=%d, E=%d, k=%d, L=%d, r=%d, dtype=%d, flags=%d, plan=%s)" %
                (self.tokens, self.hidden, self.intermediate, self.experts, self.top_k,
                 self.adapters, self.rank, self.dtype, self.flags, self.plan.as_dict()))


class DenseDims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("in_features", ctypes.c_int64),
                ("out_features", ctypes.c_int64), ("adapters", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("plan", Plan)]


_lib = None


def library():
    """The loaded libmoelora.so (raises RuntimeError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m moe_lora_layer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        pd = ctypes.POINTER(Dims)
        L.moelora_abi_version.restype = ctypes.c_int
        L.moelora_status_string.argtypes = [ctypes.c_int]
        L.moelora_status_string.restype = ctypes.c_char_p
        L.moelora_align_workspace_size.argtypes = [pd, ctypes.POINTER(sz)]
        L.moelora_forward_workspace_size.argtypes = [pd, ctypes.POINTER(sz)]
        L.moelora_forward_workspace_layout.argtypes = [pd, ctypes.POINTER(sz)]
        L.moelora_forward_fusion.argtypes = [pd, ctypes.POINTER(ctypes.c_int)]
        L.moelora_forward_plan.argtypes = [pd, ctypes.POINTER(Plan)]
        L.moelora_align.argtypes = [pd] + [vp] * 8 + [sz, vp]
        L.moelora_align_topk.argtypes = [pd] + [vp] * 6 + [sz, vp]
        L.moelora_forward.argtypes = [pd] + [vp] * 13 + [sz, vp]
        L.moelora_forward_profiled.argtypes = [pd] + [vp] * 13 + [sz, vp, vp]
        L.moelora_forward_noalloc.argtypes = [pd] + [vp] * 13
        pdd = ctypes.POINTER(DenseDims)
        L.moelora_dense_workspace_size.argtypes = [pdd, ctypes.POINTER(sz)]
        L.moelora_dense_forward.argtypes = [pdd] + [vp] * 8 + [sz, vp]
        L.moelora_dense_forward_plan.argtypes = [pdd, ctypes.POINTER(Plan)]
        for f in (L.moelora_align_workspace_size, L.moelora_forward_workspace_size,
                  L.moelora_forward_workspace_layout, L.moelora_forward_fusion,
                  L.moelora_forward_plan, L.moelora_align, L.moelora_align_topk,
                  L.moelora_forward, L.moelora_forward_profiled, L.moelora_forward_noalloc,
                  L.moelora_dense_workspace_size,
                  L.moelora_dense_forward, L.moelora_dense_forward_plan):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(rc: int) -> str:
    return library().moelora_status_string(rc).decode()


def _flags(deterministic, base_only, unfused, in_out=False) -> int:
    return ((MOELORA_FLAG_DETERMINISTIC if deterministic else 0) |
            (MOELORA_FLAG_BASE_ONLY if base_only else 0) |
            (MOELORA_FLAG_UNFUSED if unfused else 0) |
            (MOELORA_FLAG_IN_OUT if in_out else 0))


def weight_shapes(d) -> dict:
    """Shapes of the weight arrays the library expects for dims d: K-contiguous
    (transposed) by default, h_in x h_out with MOELORA_FLAG_IN_OUT."""
    io = bool(d.flags & MOELORA_FLAG_IN_OUT)
    if isinstance(d, DenseDims):
        K, N, L, r = d.in_features, d.out_features, d.adapters, d.rank
        return ({"w": (K, N), "a": (L, K, r), "b": (L, r, N)} if io else
                {"w": (N, K), "a": (L, r, K), "b": (L, N, r)})
    h, I, E, L, r = d.hidden, d.intermediate, d.experts, d.adapters, d.rank
    if io:
        return {"w_gate_up": (E, h, 2 * I), "w_down": (E, I, h), "a_gate_up": (L, E, h, r),
                "b_gate_up": (L, E, r, 2 * I), "a_down": (L, E, I, r), "b_down": (L, E, r, h)}
    return {"w_gate_up": (E, 2 * I, h), "w_down": (E, h, I), "a_gate_up": (L, E, r, h),
            "b_gate_up": (L, E, 2 * I, r), "a_down": (L, E, r, I), "b_down": (L, E, h, r)}


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what}: {status_string(rc)} (status {rc})")


def make_dims(tokens, hidden, intermediate, experts, top_k, adapters, rank, dtype,
              deterministic=False, base_only=False, unfused=False, in_out=False, flags=None,
              plan=None) -> Dims:
    if isinstance(dtype, str):
        dtype = _DT_NAME[dtype]
    elif isinstance(dtype, torch.dtype):
        dtype = MOELORA_BF16 if dtype == torch.bfloat16 else MOELORA_F32
    if flags is None:
        flags = _flags(deterministic, base_only, unfused, in_out)
    return Dims(int(tokens), int(hidden), int(intermediate), int(experts), int(top_k),
                int(adapters), int(rank), int(dtype), int(flags), make_plan(plan))


def dims_for(cfg, tokens=None, deterministic=False, base_only=False, unfused=False,
             in_out=False, plan=None) -> Dims:
    """Dims of a workload config (moe_lora_layer_amd.synth.LayerConfig)."""
    return make_dims(cfg.tokens if tokens is None else tokens, cfg.hidden, cfg.intermediate,
                     cfg.experts, cfg.top_k, cfg.adapters, cfg.rank, cfg.dtype,
                     deterministic=deterministic, base_only=base_only, unfused=unfused,
                     in_out=in_out, plan=plan)


def forward_plan(d: Dims) -> dict:
    """moelora_forward_plan: the plan moelora_forward runs for d, every field resolved."""
    out = Plan()
    _check(library().moelora_forward_plan(ctypes.byref(d), ctypes.byref(out)),
           "moelora_forward_plan")
    return out.as_dict()


def buckets(d: Dims) -> int:
    """(expert, adapter) buckets: E * L, or E * (L + 1) with base-only tokens."""
    return d.experts * (d.adapters + (1 if d.flags & MOELORA_FLAG_BASE_ONLY else 0))


def align_workspace_size(d: Dims) -> int:
    n = ctypes.c_size_t()
    _check(library().moelora_align_workspace_size(ctypes.byref(d), ctypes.byref(n)),
           "moelora_align_workspace_size")
    return n.value


def forward_workspace_size(d: Dims) -> int:
    n = ctypes.c_size_t()
    _check(library().moelora_forward_workspace_size(ctypes.byref(d), ctypes.byref(n)),
           "moelora_forward_workspace_size")
    return n.value


def forward_workspace_layout(d: Dims) -> dict:
    offs = (ctypes.c_size_t * 5)()
    _check(library().moelora_forward_workspace_layout(ctypes.byref(d), offs),
           "moelora_forward_workspace_layout")
    return dict(zip(["G", "Z1", "ACT", "Z2", "D"], list(offs)))


def forward_fusion(d: Dims) -> dict:
    """Which LoRA expands run inside the base GEMM epilogue for these dims."""
    flags = ctypes.c_int()
    _check(library().moelora_forward_fusion(ctypes.byref(d), ctypes.byref(flags)),
           "moelora_forward_fusion")
    return {"gate_up": bool(flags.value & 1), "down": bool(flags.value & 2),
            "down_shrink": bool(flags.value & 4)}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _expect(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace(nbytes: int, device) -> torch.Tensor:
    """A device byte buffer usable as a workspace (at least 256 bytes)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def align(d: Dims, logits: torch.Tensor, adapter_ids: torch.Tensor, *, out=None,
          workspace_buf=None, status=None, stream=None):
    """moelora_align.  Returns (topk_ids, topk_weights, sorted_slots, bucket_offsets, status)."""
    dev = logits.device
    T, E, k, L = d.tokens, d.experts, d.top_k, d.adapters
    _expect(logits, "logits", (T, E), torch.float32, dev)
    _expect(adapter_ids, "adapter_ids", (T,), torch.int32, dev)
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T * k,), dtype=torch.int32, device=dev),
               torch.empty((buckets(d) + 1,), dtype=torch.int32, device=dev))
    topk_ids, topk_w, sorted_slots, offsets = out
    if status is None:
        status = torch.zeros((4,), dtype=torch.int32, device=dev)
    if workspace_buf is None:
        workspace_buf = workspace(align_workspace_size(d), dev)
    _check(library().moelora_align(ctypes.byref(d), _ptr(logits), _ptr(adapter_ids), _ptr(topk_ids),
                                   _ptr(topk_w), _ptr(sorted_slots), _ptr(offsets), _ptr(status),
                                   _ptr(workspace_buf), workspace_buf.numel(), _stream(stream)),
           "moelora_align")
    return topk_ids, topk_w, sorted_slots, offsets, status


def align_topk(d: Dims, topk_ids: torch.Tensor, adapter_ids: torch.Tensor, *, out=None,
               workspace_buf=None, status=None, stream=None):
    """moelora_align_topk (the caller's own expert ids).  Returns
    (sorted_slots, bucket_offsets, status)."""
    dev = topk_ids.device
    T, E, k, L = d.tokens, d.experts, d.top_k, d.adapters
    _expect(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _expect(adapter_ids, "adapter_ids", (T,), torch.int32, dev)
    if out is None:
        out = (torch.empty((T * k,), dtype=torch.int32, device=dev),
               torch.empty((buckets(d) + 1,), dtype=torch.int32, device=dev))
    sorted_slots, offsets = out
    if status is None:
        status = torch.zeros((4,), dtype=torch.int32, device=dev)
    if workspace_buf is None:
        workspace_buf = workspace(align_workspace_size(d), dev)
    _check(library().moelora_align_topk(ctypes.byref(d), _ptr(topk_ids), _ptr(adapter_ids),
                                        _ptr(sorted_slots), _ptr(offsets), _ptr(status),
                                        _ptr(workspace_buf), workspace_buf.numel(), _stream(stream)),
           "moelora_align_topk")
    return sorted_slots, offsets, status


def forward(d: Dims, x, w_gate_up, w_down, a_gate_up, b_gate_up, a_down, b_down, topk_weights,
            sorted_slots, bucket_offsets, *, topk_ids=None, out=None, workspace_buf=None,
            stream=None, stage_events=None):
    """moelora_forward (moelora_forward_profiled when stage_events, a list of
    len(STAGES) + 1 recorded-once torch.cuda.Event(enable_timing=True) or None,
    is given).  topk_ids: align's expert ids, or None (the library does not
    read them).  Returns out [T][h]."""
    dev = x.device
    T, h, I, E, k, L, r = d.tokens, d.hidden, d.intermediate, d.experts, d.top_k, d.adapters, d.rank
    dt = _TORCH_DT[d.dtype]
    _expect(x, "x", (T, h), dt, dev)
    ws = weight_shapes(d)
    for name, t in (("w_gate_up", w_gate_up), ("w_down", w_down), ("a_gate_up", a_gate_up),
                    ("b_gate_up", b_gate_up), ("a_down", a_down), ("b_down", b_down)):
        _expect(t, name, ws[name], dt, dev)
    if topk_ids is not None:
        _expect(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _expect(topk_weights, "topk_weights", (T, k), torch.float32, dev)
    _expect(sorted_slots, "sorted_slots", (T * k,), torch.int32, dev)
    _expect(bucket_offsets, "bucket_offsets", (buckets(d) + 1,), torch.int32, dev)
    if out is None:
        out = torch.empty((T, h), dtype=dt, device=dev)
    _expect(out, "out", (T, h), dt, dev)
    if workspace_buf is None:
        workspace_buf = workspace(forward_workspace_size(d), dev)
    args = [ctypes.byref(d), _ptr(x), _ptr(w_gate_up), _ptr(w_down), _ptr(a_gate_up),
            _ptr(b_gate_up), _ptr(a_down), _ptr(b_down), _ptr(topk_ids), _ptr(topk_weights),
            _ptr(sorted_slots), _ptr(bucket_offsets), _ptr(out), _ptr(workspace_buf),
            workspace_buf.numel(), _stream(stream)]
    if stage_events is None:
        _check(library().moelora_forward(*args), "moelora_forward")
    else:
        if len(stage_events) != len(STAGES) + 1:
            raise ValueError(f"need {len(STAGES) + 1} events")
        hs = [None if ev is None else ev.cuda_event for ev in stage_events]
        if any(ev is not None and not h for ev, h in zip(stage_events, hs)):
            raise ValueError("record every event once before passing it (creates the handle)")
        handles = (ctypes.c_void_p * len(hs))(*hs)
        _check(library().moelora_forward_profiled(*args, handles), "moelora_forward_profiled")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_noalloc(d: Dims, x, w_gate_up, w_down, a_gate_up, b_gate_up, a_down, b_down,
                    topk_weights, sorted_slots, bucket_offsets, *, topk_ids=None, out=None,
                    stream=None):
    """moelora_forward_noalloc: moelora_forward in the library's static device
    scratch (no workspace argument).  out must be given when the caller cannot
    allocate; with out=None one is allocated here.  Returns out [T][h]."""
    dev = x.device
    T, h, I, E, k, L, r = d.tokens, d.hidden, d.intermediate, d.experts, d.top_k, d.adapters, d.rank
    dt = _TORCH_DT[d.dtype]
    _expect(x, "x", (T, h), dt, dev)
    ws = weight_shapes(d)
    for name, t in (("w_gate_up", w_gate_up), ("w_down", w_down), ("a_gate_up", a_gate_up),
                    ("b_gate_up", b_gate_up), ("a_down", a_down), ("b_down", b_down)):
        _expect(t, name, ws[name], dt, dev)
    if topk_ids is not None:
        _expect(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _expect(topk_weights, "topk_weights", (T, k), torch.float32, dev)
    _expect(sorted_slots, "sorted_slots", (T * k,), torch.int32, dev)
    _expect(bucket_offsets, "bucket_offsets", (buckets(d) + 1,), torch.int32, dev)
    if out is None:
        out = torch.empty((T, h), dtype=dt, device=dev)
    _expect(out, "out", (T, h), dt, dev)
    _check(library().moelora_forward_noalloc(
        ctypes.byref(d), _ptr(x), _ptr(w_gate_up), _ptr(w_down), _ptr(a_gate_up), _ptr(b_gate_up),
        _ptr(a_down), _ptr(b_down), _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_slots),
        _ptr(bucket_offsets), _ptr(out), _stream(stream)), "moelora_forward_noalloc")
    return out


class MoELoRALayer:
    """One layer's weights plus preallocated outputs and workspaces for a fixed
    token count; ``__call__`` runs moelora_align then moelora_forward with no
    allocation."""

    def __init__(self, d: Dims, weights: dict, device):
        self.d = d
        self.w = weights
        T, E, k, L, h = d.tokens, d.experts, d.top_k, d.adapters, d.hidden
        dt = _TORCH_DT[d.dtype]
        self.routing = (torch.empty((T, k), dtype=torch.int32, device=device),
                        torch.empty((T, k), dtype=torch.float32, device=device),
                        torch.empty((T * k,), dtype=torch.int32, device=device),
                        torch.empty((buckets(d) + 1,), dtype=torch.int32, device=device))
        self.status = torch.zeros((4,), dtype=torch.int32, device=device)
        self.ws_align = workspace(align_workspace_size(d), device)
        self.ws_fwd = workspace(forward_workspace_size(d), device)
        self.out = torch.empty((T, h), dtype=dt, device=device)

    def __call__(self, x, logits, adapter_ids, stream=None):
        ids, w, ss, off, _ = align(self.d, logits, adapter_ids, out=self.routing,
                                   workspace_buf=self.ws_align, status=self.status, stream=stream)
        W = self.w
        return forward(self.d, x, W["w_gate_up"], W["w_down"], W["a_gate_up"], W["b_gate_up"],
                       W["a_down"], W["b_down"], w, ss, off, topk_ids=ids, out=self.out,
                       workspace_buf=self.ws_fwd, stream=stream)


class CapturedStep:
    """A MoELoRALayer step (moelora_align then moelora_forward) captured once
    into a HIP graph over fixed input buffers x [T][h], logits [T][E] and
    adapter_ids [T]; replay() runs it again on whatever those buffers hold
    and returns the layer's output buffer.  Nothing is allocated or
    synchronised inside the step and the library clears its memory with fill
    kernels, so the graph holds kernel launches only.  One warm-up call runs
    outside the capture (the library's first-call lookups)."""

    def __init__(self, layer: MoELoRALayer, x, logits, adapter_ids):
        self.layer, self.x, self.logits, self.adapter_ids = layer, x, logits, adapter_ids
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer(x, logits, adapter_ids)
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.out = layer(x, logits, adapter_ids)

    def replay(self):
        self.graph.replay()
        return self.out


def make_dense_dims(tokens, in_features, out_features, adapters, rank, dtype, deterministic=False,
                    base_only=False, unfused=False, in_out=False, plan=None) -> DenseDims:
    if isinstance(dtype, str):
        dtype = _DT_NAME[dtype]
    flags = _flags(deterministic, base_only, unfused, in_out)
    return DenseDims(int(tokens), int(in_features), int(out_features), int(adapters), int(rank),
                     int(dtype), flags, make_plan(plan))


def dense_forward_plan(d: DenseDims) -> dict:
    """moelora_dense_forward_plan: the resolved plan of the dense projection."""
    out = Plan()
    _check(library().moelora_dense_forward_plan(ctypes.byref(d), ctypes.byref(out)),
           "moelora_dense_forward_plan")
    return out.as_dict()


def dense_workspace_size(d: DenseDims) -> int:
    n = ctypes.c_size_t()
    _check(library().moelora_dense_workspace_size(ctypes.byref(d), ctypes.byref(n)),
           "moelora_dense_workspace_size")
    return n.value


def dense_forward(d: DenseDims, x, w, a, b, adapter_ids, *, out=None, workspace_buf=None,
                  status=None, stream=None):
    """moelora_dense_forward: out[t] = x_t W + (x_t A[l]) B[l].  Returns (out, status)."""
    dev = x.device
    T, K, N, L, r = d.tokens, d.in_features, d.out_features, d.adapters, d.rank
    dt = _TORCH_DT[d.dtype]
    _expect(x, "x", (T, K), dt, dev)
    ws = weight_shapes(d)
    _expect(w, "w", ws["w"], dt, dev)
    _expect(a, "a", ws["a"], dt, dev)
    _expect(b, "b", ws["b"], dt, dev)
    _expect(adapter_ids, "adapter_ids", (T,), torch.int32, dev)
    if out is None:
        out = torch.empty((T, N), dtype=dt, device=dev)
    _expect(out, "out", (T, N), dt, dev)
    if status is None:
        status = torch.zeros((4,), dtype=torch.int32, device=dev)
    if workspace_buf is None:
        workspace_buf = workspace(dense_workspace_size(d), dev)
    _check(library().moelora_dense_forward(ctypes.byref(d), _ptr(x), _ptr(w), _ptr(a), _ptr(b),
                                           _ptr(adapter_ids), _ptr(out), _ptr(status),
                                           _ptr(workspace_buf), workspace_buf.numel(), _stream(stream)),
           "moelora_dense_forward")
    return out, status
