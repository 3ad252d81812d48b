"""Device-side plumbing around the C ABI: torch allocates the weights, inputs,
outputs and workspace on the GPU and supplies the stream; the layer itself runs
only in libmoe.so (``binding``).  There is no CPU fallback: without the built
library or a GPU every call raises.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np
import torch

from . import binding as B
from .workloads import MoEConfig, Workload


def _bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)


def host_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Stored numpy array -> CPU torch tensor of the storage type."""
    if dtype == "bf16":
        return _bf16(a)
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a))
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


class DeviceLayer:
    """One layer's weights resident in HBM plus its C handle."""

    def __init__(self, cfg: MoEConfig, tensors: dict, max_tokens: int):
        self.cfg = cfg
        self.t = tensors
        self.max_tokens = int(max_tokens)
        c = B.MoEConfig(d=cfg.d, latent=cfg.latent, n_experts=cfg.n_experts, top_k=cfg.top_k,
                        ffn=cfg.ffn, n_shared=cfg.n_shared, shared_ffn=cfg.shared_ffn,
                        max_tokens=self.max_tokens, has_latent_proj=int(cfg.has_latent_proj),
                        act_dtype=B.DTYPES[cfg.act], expert_dtype=B.DTYPES[cfg.expert],
                        router_on_x=int(cfg.router_on_x), shared_fp8=int(cfg.shared_fp8))
        w = B.MoEWeights()
        for name in ("w_down", "w_router", "b_router", "w1", "w2", "w1_scale", "w2_scale",
                     "w1_gscale", "w2_gscale", "w_up", "ws1", "ws2", "act_scale", "ws1_scale",
                     "ws2_scale", "shared_act_scale"):
            setattr(w, name, _ptr(tensors.get(name)))
        self._c, self._w = c, w
        _, self.handle = B.moe_init(c, w)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                B.moe_destroy(h)
            except Exception:
                pass
            self.handle = None

    # ------------------------------------------------------------ construction
    @classmethod
    def from_workload(cls, wl: Workload, device="cuda", max_tokens: Optional[int] = None,
                      threads: int = 8) -> "DeviceLayer":
        cfg = wl.cfg
        dev = torch.device(device)
        t = {}

        def put(name, arr, dtype):
            if arr is not None:
                t[name] = host_tensor(arr, dtype).to(dev)

        put("w_down", wl.w_down(), cfg.act)
        put("w_up", wl.w_up(), cfg.act)
        put("w_router", wl.w_router(), "f32")
        put("b_router", wl.b_router(), "f32")
        if cfg.shared_fp8 and cfg.n_shared:
            for name, (codes, sc) in (("ws1", wl.ws1()), ("ws2", wl.ws2())):
                put(name, codes, "u8")
                put(name + "_scale", np.array([sc], dtype=np.float32), "f32")
            put("shared_act_scale", wl.shared_act_scales(), "f32")
        else:
            put("ws1", wl.ws1(), cfg.act)
            put("ws2", wl.ws2(), cfg.act)
        put("act_scale", wl.act_scales(), "f32")
        N, m, l = cfg.n_experts, cfg.ffn, cfg.latent
        for which, (rows, cols) in (("w1", (m, l)), ("w2", (l, m))):
            fn = wl.w1 if which == "w1" else wl.w2
            if cfg.expert == "nvfp4":
                codes = torch.empty((N, rows, cols // 2), dtype=torch.uint8, device=dev)
                scales = torch.empty((N, rows, cols // 16), dtype=torch.uint8, device=dev)
                gs = np.zeros(N, dtype=np.float32)
            elif cfg.expert == "fp8":
                codes = torch.empty((N, rows, cols), dtype=torch.uint8, device=dev)
                gs = np.zeros(N, dtype=np.float32)
            else:
                tdt = torch.bfloat16 if cfg.expert == "bf16" else torch.float32
                full = torch.empty((N, rows, cols), dtype=tdt, device=dev)
            with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
                for e, part in enumerate(ex.map(fn, range(N))):
                    if cfg.expert == "nvfp4":
                        codes[e].copy_(torch.from_numpy(part[0]))
                        scales[e].copy_(torch.from_numpy(part[1]))
                        gs[e] = part[2]
                    elif cfg.expert == "fp8":
                        codes[e].copy_(torch.from_numpy(part[0]))
                        gs[e] = part[1]
                    else:
                        full[e].copy_(host_tensor(part, cfg.expert))
            if cfg.expert == "nvfp4":
                # the library reads NVFP4 weights k-tiled: permute on the device
                tiled = torch.empty_like(codes), torch.empty_like(scales)
                B.moe_nvfp4_tile(_ptr(codes), _ptr(scales), _ptr(tiled[0]), _ptr(tiled[1]), N, rows,
                                 cols, torch.cuda.current_stream(dev).cuda_stream)
                torch.cuda.synchronize(dev)
                del codes, scales
                t[which], t[which + "_scale"] = tiled
                t[which + "_gscale"] = torch.from_numpy(gs).to(dev)
            elif cfg.expert == "fp8":
                t[which] = codes
                t[which + "_gscale"] = torch.from_numpy(gs).to(dev)
            else:
                t[which] = full
        return cls(cfg, t, cfg.T if max_tokens is None else max_tokens)

    # ------------------------------------------------------------ calls
    def workspace_bytes(self, T: int) -> int:
        return B.moe_workspace_size(self.handle, T)[1]

    def new_workspace(self, T: int) -> torch.Tensor:
        n = max(1, self.workspace_bytes(T))
        return torch.empty(n, dtype=torch.uint8, device=self.t["w_router"].device)

    def act_torch_dtype(self):
        return torch.bfloat16 if self.cfg.act == "bf16" else torch.float32

    def route(self, x: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None):
        T = x.shape[0]
        dev = x.device
        K, N = self.cfg.top_k, self.cfg.n_experts
        idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        gate = torch.empty((T, K), dtype=torch.float32, device=dev)
        counts = torch.empty((N,), dtype=torch.int32, device=dev)
        if ws is None:
            ws = self.new_workspace(T)
        s = (stream or torch.cuda.current_stream(dev)).cuda_stream
        B.moe_route(self.handle, x.data_ptr(), T, idx.data_ptr(), gate.data_ptr(),
                    counts.data_ptr(), ws.data_ptr(), ws.numel(), s)
        return idx, gate, counts

    def forward(self, x: torch.Tensor, ws: Optional[torch.Tensor] = None, y=None,
                routing: bool = False, stream=None):
        T = x.shape[0]
        dev = x.device
        if y is None:
            y = torch.empty((T, self.cfg.d), dtype=self.act_torch_dtype(), device=dev)
        if ws is None:
            ws = self.new_workspace(T)
        idx = gate = counts = None
        if routing:
            K, N = self.cfg.top_k, self.cfg.n_experts
            idx = torch.empty((T, K), dtype=torch.int32, device=dev)
            gate = torch.empty((T, K), dtype=torch.float32, device=dev)
            counts = torch.empty((N,), dtype=torch.int32, device=dev)
        s = (stream or torch.cuda.current_stream(dev)).cuda_stream
        B.moe_forward(self.handle, x.data_ptr(), T, y.data_ptr(), _ptr(idx), _ptr(gate),
                      _ptr(counts), ws.data_ptr(), ws.numel(), s)
        if routing:
            return y, idx, gate, counts
        return y

    def forward_noalloc(self, x: torch.Tensor, y=None, routing: bool = False, stream=None):
        """moe_forward_noalloc: the library's own scratch array as the workspace."""
        T = x.shape[0]
        dev = x.device
        if y is None:
            y = torch.empty((T, self.cfg.d), dtype=self.act_torch_dtype(), device=dev)
        idx = gate = counts = None
        if routing:
            K, N = self.cfg.top_k, self.cfg.n_experts
            idx = torch.empty((T, K), dtype=torch.int32, device=dev)
            gate = torch.empty((T, K), dtype=torch.float32, device=dev)
            counts = torch.empty((N,), dtype=torch.int32, device=dev)
        s = (stream or torch.cuda.current_stream(dev)).cuda_stream
        B.moe_forward_noalloc(self.handle, x.data_ptr(), T, y.data_ptr(), _ptr(idx), _ptr(gate),
                              _ptr(counts), s)
        if routing:
            return y, idx, gate, counts
        return y


def x_to_device(wl: Workload, device="cuda") -> torch.Tensor:
    return host_tensor(wl.x(), wl.cfg.act).to(device)
