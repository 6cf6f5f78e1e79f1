"""Device buffers for one layer of the path (torch is used for memory only).

`LayerBuffers` uploads one layer's synthetic inputs and allocates every output
and intermediate in the layouts of include/gdn.h.  It does no arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import binding

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16}


def scratch(nbytes: int, device) -> torch.Tensor:
    """Device scratch of at least nbytes, 256-byte aligned (torch's caching
    allocator hands out blocks aligned to at least 512 bytes)."""
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def upload(arr: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


@dataclass
class LayerBuffers:
    shape: binding.gdn_shape
    cu: torch.Tensor
    qkv: torch.Tensor
    conv_w: torch.Tensor
    a: torch.Tensor
    b: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    z: torch.Tensor
    gamma: torch.Tensor
    hist: torch.Tensor
    state: torch.Tensor
    qn: torch.Tensor
    kn: torch.Tensor
    vc: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    o: torch.Tensor
    y: torch.Tensor

    @classmethod
    def create(cls, w, inp: dict, device="cuda", out: str | None = None, cu=None):
        """w: synth.Workload (sizes and dtypes); inp: synth.layer_inputs(w, l)."""
        out = out or w.out
        cu_np = w.cu_seqlens() if cu is None else np.asarray(cu, np.int32)
        T = int(cu_np[-1])
        n_seq = len(cu_np) - 1
        max_T = int(np.diff(cu_np).max()) if n_seq else 0
        shape = binding.make_shape(w.hk, w.hv, n_seq, T, max_T, io=w.io, out=out)
        f32 = dict(dtype=torch.float32, device=device)
        hk, hv = w.hk, w.hv
        return cls(
            shape=shape,
            cu=upload(cu_np.astype(np.int32), device),
            qkv=upload(inp["qkv"], device), conv_w=upload(inp["conv_w"], device),
            a=upload(inp["a"], device), b=upload(inp["b"], device),
            A_log=upload(inp["A_log"], device), dt_bias=upload(inp["dt_bias"], device),
            z=upload(inp["z"], device), gamma=upload(inp["gamma"], device),
            hist=upload(inp["hist"], device), state=upload(inp["S0"], device),
            qn=torch.empty((T, hk, 128), **f32), kn=torch.empty((T, hk, 128), **f32),
            vc=torch.empty((T, hv, 128), **f32), g=torch.empty((T, hv), **f32),
            beta=torch.empty((T, hv), **f32), o=torch.empty((T, hv, 128), **f32),
            y=torch.empty((T, hv * 128), dtype=TORCH_DTYPE[out], device=device),
        )

    def run_pre(self, stream=None):
        binding.gdn_pre(self.shape, self.cu, self.qkv, self.conv_w, self.a, self.b, self.A_log,
                        self.dt_bias, self.hist, self.qn, self.kn, self.vc, self.g, self.beta,
                        stream=stream)

    def scan_workspace(self) -> torch.Tensor:
        return scratch(binding.gdn_scan_workspace_bytes(self.shape), self.qkv.device)

    def run_scan(self, workspace=None, stream=None):
        ws = self.scan_workspace() if workspace is None else workspace
        binding.gdn_scan(self.shape, self.cu, self.qn, self.kn, self.vc, self.g, self.beta,
                         self.state, self.o, ws, stream=stream)

    def run_post(self, stream=None):
        binding.gdn_post(self.shape, self.o, self.z, self.gamma, self.y, stream=stream)

    def workspace(self) -> torch.Tensor:
        return scratch(binding.gdn_prefill_workspace_bytes(self.shape), self.qkv.device)

    def run_layer(self, workspace: torch.Tensor, stream=None):
        binding.gdn_prefill_layer(self.shape, self.cu, self.qkv, self.conv_w, self.a, self.b,
                                  self.A_log, self.dt_bias, self.z, self.gamma, self.hist,
                                  self.state, self.y, workspace, stream=stream)
