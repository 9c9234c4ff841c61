"""Helpers shared by the GPU tests: move seeded workloads to the device, run the
two C-ABI calls, compare against the oracle with the parity tolerance."""
from __future__ import annotations

import sys

import numpy as np
import torch

from moe_lora_layer_amd import ops, synth

WEIGHTS = ["w_gate_up", "w_down", "a_gate_up", "b_gate_up", "a_down", "b_down"]

# max|gpu - oracle| <= TOL * max|oracle|
TOL = {"bf16": 1e-2, "f32": 1e-4}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def device() -> torch.device:
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str, dev) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def in_out(inp: dict) -> dict:
    """The weights of a workload in the page's h_in x h_out orientation (the
    layout of MOELORA_FLAG_IN_OUT): every K-contiguous weight array transposed
    in its last two axes.  The oracle keeps taking the K-contiguous arrays."""
    out = dict(inp)
    for n in WEIGHTS:
        out[n] = np.ascontiguousarray(np.swapaxes(inp[n], -1, -2))
    return out


def device_inputs(inp: dict, cfg, dev) -> dict:
    d = {n: to_dev(inp[n], cfg.dtype, dev) for n in ["x"] + WEIGHTS if n in inp}
    d["logits"] = torch.from_numpy(inp["logits"]).to(dev)
    d["adapter_ids"] = torch.from_numpy(inp["adapter_ids"]).to(dev)
    return d


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_align(cfg, dinp, dims=None):
    d = dims or ops.dims_for(cfg)
    ids, w, ss, off, st = ops.align(d, dinp["logits"], dinp["adapter_ids"])
    torch.cuda.synchronize()
    return ids, w, ss, off, st


def run_forward(cfg, dinp, w, ss, off, dims=None, workspace_buf=None):
    d = dims or ops.dims_for(cfg)
    if workspace_buf is None:
        workspace_buf = ops.workspace(ops.forward_workspace_size(d), dinp["x"].device)
    out = ops.forward(d, dinp["x"], *[dinp[n] for n in WEIGHTS], w, ss, off,
                      workspace_buf=workspace_buf)
    torch.cuda.synchronize()
    return out, workspace_buf


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


def assert_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    err = rel_err(gpu, ref)
    say(f"  {what} max|gpu-oracle|/max|oracle| = {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype], f"{what}: {err} > {TOL[dtype]}"


def workspace_view(ws: torch.Tensor, offset: int, shape, dtype) -> torch.Tensor:
    n = int(np.prod(shape))
    esz = torch.empty((), dtype=dtype).element_size()
    return ws[offset: offset + n * esz].view(dtype).view(*shape)


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    pick = set([0, T - 1]) | set(rng.choice(T, n - 2, replace=False).tolist())
    return np.array(sorted(pick))
