"""Torch-side harness around libmuon: tensors own the device memory, libmuon computes.

`Plan` wraps one muon_plan*: it builds the descriptors from torch tensors, allocates the
workspace as a torch uint8 tensor, binds it, and forwards the step calls with the
current torch stream.  Every step of the optimizer runs in libmuon's HIP kernels; this
module only marshals arguments.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

from . import binding as L
from . import workloads as wl


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


@dataclass
class ParamTensors:
    weight: torch.Tensor
    momentum: torch.Tensor
    grad: torch.Tensor
    exp_avg_sq: Optional[torch.Tensor] = None   # AdamW second moment
    optimizer: int = 0                          # MUON_OPT_*


def _desc(p: ParamTensors) -> L.muon_param_desc:
    d = L.muon_param_desc()
    d.ndim = p.weight.dim()
    d.optimizer = int(p.optimizer)
    adam = p.optimizer == L.MUON_OPT_ADAMW or (p.optimizer == L.MUON_OPT_DEFAULT and d.ndim != 2
                                                and p.exp_avg_sq is not None)
    if not adam and (d.ndim != 2 or p.optimizer == L.MUON_OPT_NONE):
        return d
    tensors = [("weight", p.weight), ("momentum", p.momentum), ("grad", p.grad)]
    if adam:
        tensors.append(("exp_avg_sq", p.exp_avg_sq))
    for name, t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        if t.shape != p.weight.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} differs from weight {tuple(p.weight.shape)}")
    if p.weight.dtype != torch.float32 or p.momentum.dtype != torch.float32:
        raise ValueError("weight and momentum must be float32")
    if p.grad.dtype == torch.float32:
        d.grad_dtype = L.MUON_DTYPE_F32
    elif p.grad.dtype == torch.bfloat16:
        d.grad_dtype = L.MUON_DTYPE_BF16
    else:
        raise ValueError("grad must be float32 or bfloat16")
    if adam:
        if p.exp_avg_sq.dtype != torch.float32:
            raise ValueError("exp_avg_sq must be float32")
        d.rows, d.cols = p.weight.numel(), 1
        d.exp_avg_sq = p.exp_avg_sq.data_ptr()
    else:
        d.rows, d.cols = p.weight.shape
    d.weight = p.weight.data_ptr()
    d.momentum = p.momentum.data_ptr()
    d.grad = p.grad.data_ptr()
    return d


class Plan:
    """One bound libmuon plan over a list of parameters."""

    def __init__(self, params: Sequence[ParamTensors], max_workspace_bytes: int = 0,
                 scales: Optional[Sequence[float]] = None, device=None, bind: bool = True, flags: int = 0,
                 scale_mode: int = 0):
        self.params = list(params)
        n = len(self.params)
        self._descs = (L.muon_param_desc * max(n, 1))()
        for i, p in enumerate(self.params):
            self._descs[i] = _desc(p)
        opts = L.muon_plan_opts()
        opts.max_workspace_bytes = int(max_workspace_bytes)
        opts.flags = int(flags)
        opts.scale_mode = int(scale_mode)
        self._scales = None
        if scales is not None:
            self._scales = (C.c_float * max(n, 1))(*[float(s) for s in scales])
            opts.scale = self._scales
        self._plan = C.c_void_p()
        L.check(L.muon_plan_buckets(self._descs, n, C.byref(opts), C.byref(self._plan)), "muon_plan_buckets")
        nb = C.c_uint64()
        L.check(L.muon_plan_workspace_bytes(self._plan, C.byref(nb)), "muon_plan_workspace_bytes")
        self.workspace_bytes = int(nb.value)
        nc, nbk, ninc, nex = C.c_int32(), C.c_int32(), C.c_int64(), C.c_int64()
        L.check(L.muon_plan_counts(self._plan, C.byref(nc), C.byref(nbk), C.byref(ninc), C.byref(nex)),
                "muon_plan_counts")
        self.n_chunks, self.n_buckets = nc.value, nbk.value
        self.n_included, self.n_excluded = ninc.value, nex.value
        self.device = device if device is not None else (
            self.params[0].weight.device if self.params else torch.device("cuda"))
        self.workspace = None
        if bind:
            self.bind()

    # ---- lifetime ------------------------------------------------------------------------
    def bind(self, stream=None):
        # 512 extra bytes let the base be moved up to a 256-byte boundary if needed
        self.workspace = torch.empty(self.workspace_bytes + 512, dtype=torch.uint8, device=self.device)
        base = self.workspace.data_ptr()
        self._ws_off = (-base) % 256
        L.check(L.muon_plan_bind(self._plan, base + self._ws_off, self.workspace_bytes, _stream_ptr(stream)),
                "muon_plan_bind")

    def close(self):
        if self._plan:
            L.muon_plan_destroy(self._plan)
            self._plan = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- the step ----------------------------------------------------------------------
    def momentum_update(self, beta: float, chunk: int = -1, stream=None):
        L.check(L.muon_momentum_update(self._plan, chunk, beta, _stream_ptr(stream)), "muon_momentum_update")

    def ns_batched(self, a=wl.NS_A, b=wl.NS_B, c=wl.NS_C, steps=wl.NS_STEPS, eps=wl.NS_EPS,
                   chunk: int = -1, stream=None):
        L.check(L.muon_ns_batched(self._plan, chunk, a, b, c, steps, eps, _stream_ptr(stream)), "muon_ns_batched")

    def apply(self, lr: float, wd: float, chunk: int = -1, stream=None):
        L.check(L.muon_apply(self._plan, chunk, lr, wd, _stream_ptr(stream)), "muon_apply")

    def step(self, beta, lr, wd, a=wl.NS_A, b=wl.NS_B, c=wl.NS_C, steps=wl.NS_STEPS, eps=wl.NS_EPS,
             chunk: int = -1, stream=None):
        L.check(L.muon_step(self._plan, chunk, beta, a, b, c, steps, eps, lr, wd, _stream_ptr(stream)),
                "muon_step")

    def ns_schedule(self, coeffs, eps=wl.NS_EPS, chunk: int = -1, stream=None):
        """Newton–Schulz with per-iteration coefficients: coeffs is a (steps, 3) sequence."""
        flat = [float(v) for row in coeffs for v in row]
        arr = (C.c_float * len(flat))(*flat)
        L.check(L.muon_ns_batched_schedule(self._plan, chunk, arr, len(flat) // 3, eps, _stream_ptr(stream)),
                "muon_ns_batched_schedule")

    @staticmethod
    def config(beta, lr, wd, a=wl.NS_A, b=wl.NS_B, c=wl.NS_C, steps=wl.NS_STEPS, eps=wl.NS_EPS,
               coeffs=None, nesterov=False, dev_scalars: Optional[torch.Tensor] = None, adamw=None,
               pipeline=False):
        """A muon_step_config (and the host arrays it points to, which must stay alive)."""
        k = L.muon_step_config()
        k.beta, k.lr, k.wd, k.eps = beta, lr, wd, eps
        k.a, k.b, k.c = a, b, c
        keep = None
        if coeffs is not None:
            flat = [float(v) for row in coeffs for v in row]
            keep = (C.c_float * len(flat))(*flat)
            k.coeffs = keep
            steps = len(flat) // 3
        k.steps = steps
        k.nesterov = 1 if nesterov else 0
        k.pipeline = 1 if pipeline else 0
        if adamw is not None:
            keep = (keep, adamw)
            k.adamw = C.pointer(adamw)
        if dev_scalars is not None:
            assert dev_scalars.dtype == torch.float32 and dev_scalars.numel() >= 3 and dev_scalars.is_cuda
            k.dev_scalars = dev_scalars.data_ptr()
        return k, keep

    @staticmethod
    def adamw_config(lr, beta1, beta2, eps, wd, step, dev_scalars: Optional[torch.Tensor] = None):
        k = L.muon_adamw_config()
        k.lr, k.beta1, k.beta2, k.eps, k.wd, k.step = lr, beta1, beta2, eps, wd, step
        if dev_scalars is not None:
            assert dev_scalars.dtype == torch.float32 and dev_scalars.numel() >= 4 and dev_scalars.is_cuda
            k.dev_scalars = dev_scalars.data_ptr()
        return k

    def adamw_step(self, lr, beta1, beta2, eps, wd, step, stream=None, dev_scalars=None):
        k = self.adamw_config(lr, beta1, beta2, eps, wd, step, dev_scalars)
        L.check(L.muon_adamw_step(self._plan, C.byref(k), _stream_ptr(stream)), "muon_adamw_step")

    def adamw_counts(self):
        n, e = C.c_int64(), C.c_int64()
        L.check(L.muon_plan_adamw_counts(self._plan, C.byref(n), C.byref(e)), "muon_plan_adamw_counts")
        return int(n.value), int(e.value)

    def step_ex(self, beta, lr, wd, chunk: int = -1, stream=None, **kw):
        k, keep = self.config(beta, lr, wd, **kw)
        L.check(L.muon_step_ex(self._plan, chunk, C.byref(k), _stream_ptr(stream)), "muon_step_ex")
        del keep

    def step_noalloc(self, beta, lr, wd, stream=None, **kw):
        """The whole step on one stream with libmuon's static scratch as the workspace
        (muon_step_noalloc; the plan need not be bound)."""
        k, keep = self.config(beta, lr, wd, **kw)
        L.check(L.muon_step_noalloc(self._plan, C.byref(k), _stream_ptr(stream)), "muon_step_noalloc")
        del keep

    def capture_ex(self, beta, lr, wd, **kw) -> "Graph":
        k, keep = self.config(beta, lr, wd, **kw)
        g = C.c_void_p()
        L.check(L.muon_graph_capture_ex(self._plan, C.byref(k), C.byref(g)), "muon_graph_capture_ex")
        del keep
        return Graph(g, self)

    def capture(self, beta, lr, wd, a=wl.NS_A, b=wl.NS_B, c=wl.NS_C, steps=wl.NS_STEPS,
                eps=wl.NS_EPS) -> "Graph":
        """The whole step (every chunk) as one replayable graph, tied to this workspace."""
        g = C.c_void_p()
        L.check(L.muon_graph_capture(self._plan, beta, a, b, c, steps, eps, lr, wd, C.byref(g)),
                "muon_graph_capture")
        return Graph(g, self)

    # ---- queries -----------------------------------------------------------------------
    def chunk_info(self, chunk: int) -> L.muon_chunk_info:
        info = L.muon_chunk_info()
        L.check(L.muon_plan_info(self._plan, chunk, C.byref(info)), "muon_plan_info")
        return info

    def param_info(self, index: int) -> L.muon_param_info:
        info = L.muon_param_info()
        L.check(L.muon_plan_param_info(self._plan, index, C.byref(info)), "muon_plan_param_info")
        return info

    def validate(self) -> int:
        return L.muon_plan_validate(self._plan, self._descs, len(self.params))

    def output(self, index: int) -> torch.Tensor:
        """View of parameter `index`'s update O in the workspace: bf16, canonical m x n."""
        info = self.param_info(index)
        if not info.included:
            raise ValueError(f"parameter {index} is not a matrix")
        rows, cols = self.params[index].weight.shape
        m, n = min(rows, cols), max(rows, cols)
        ci = self.chunk_info(info.chunk)
        start = self._ws_off + int(info.output_offset)
        flat = self.workspace[start:start + ci.m_pad * ci.n_pad * 2].view(torch.bfloat16)
        return flat.view(ci.m_pad, ci.n_pad)[:m, :n]

    def output_oriented(self, index: int) -> torch.Tensor:
        """O in the parameter's own rows x cols orientation."""
        o = self.output(index)
        return o.t() if self.param_info(index).transposed else o

    # ---- timing ------------------------------------------------------------------------
    def timing_enable(self, capacity: int):
        L.check(L.muon_timing_enable(self._plan, capacity), "muon_timing_enable")

    def timing_reset(self):
        L.check(L.muon_timing_reset(self._plan), "muon_timing_reset")

    def timing_read(self, kernel: int):
        ms, n, work = C.c_double(), C.c_int64(), C.c_double()
        L.check(L.muon_timing_read(self._plan, kernel, C.byref(ms), C.byref(n), C.byref(work)),
                "muon_timing_read")
        return float(ms.value), int(n.value), float(work.value)


class Graph:
    """An instantiated graph of one step; keeps its plan (and so the workspace) alive."""

    def __init__(self, handle: C.c_void_p, plan: Plan):
        self._g = handle
        self.plan = plan
        n = C.c_int64()
        L.check(L.muon_graph_node_count(self._g, C.byref(n)), "muon_graph_node_count")
        self.nodes = int(n.value)

    def launch(self, stream=None):
        L.check(L.muon_graph_launch(self._g, _stream_ptr(stream)), "muon_graph_launch")

    def close(self):
        if self._g:
            L.muon_graph_destroy(self._g)
            self._g = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_params(w: wl.Workload, device="cuda", indices: Optional[Sequence[int]] = None) -> List[ParamTensors]:
    """Seeded W, M, G tensors of a workload on `device` (G in the workload's dtype)."""
    out = []
    for i in (range(len(w.params)) if indices is None else indices):
        t = wl.generate(w, i, device=device)
        g = t["G"]
        if w.params[i].grad_dtype == "bf16":
            g = g.to(torch.bfloat16)
        out.append(ParamTensors(t["W"], t["M"], g))
    return out
