"""torch-facing wrapper around the C ABI: device tensors in, device tensors out.

Marshalling only.  torch allocates device memory and provides the stream;
every step of the decision runs in libphx_expert.so.
"""
from __future__ import annotations

import numpy as np

from . import binding as B


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU: the action expert runs only on the HIP device (there is no CPU path)")
    return torch


def device_blob(values: np.ndarray, bits, device):
    """Upload a float32 array, or raw bfloat16 bits (uint16), as one device tensor."""
    torch = _torch()
    if bits is not None:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).to(device)


class Expert:
    """One handle of the library for one deployment shape."""

    def __init__(self, cfg: dict, weights: np.ndarray, weights_bits=None, device: str = "cuda:0", flags: int = 0):
        torch = _torch()
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.c = B.make_config(cfg, flags)
        blob = device_blob(weights, weights_bits, self.device)
        nbytes = blob.numel() * blob.element_size()
        self.stream = torch.cuda.current_stream(self.device).cuda_stream
        self.h = B.phx_expert_create(self.c, blob.data_ptr(), nbytes, self.stream)
        del blob

    def load_prefix_kv(self, request: int, k, v, prefix_len: int):
        """k, v: device tensors [layers][prefix_len][KVH*Dh] of the kv dtype
        (int16 raw bfloat16 bits or float32)."""
        kp = k.data_ptr() if prefix_len > 0 else 0
        vp = v.data_ptr() if prefix_len > 0 else 0
        B.phx_expert_load_prefix_kv(self.h, request, kp, vp, prefix_len, self.stream)

    def load_all(self, inp: dict):
        """Load every request's prefix from a phx_inputs dictionary."""
        torch = self.torch
        cfg = self.cfg
        keep = []
        for b in range(cfg["batch"]):
            L = int(inp["lens"][b])
            if cfg["dtype"] == "bf16":
                kb = np.ascontiguousarray(inp["kv_k_bits"][b, :, :L]).view(np.int16)
                vb = np.ascontiguousarray(inp["kv_v_bits"][b, :, :L]).view(np.int16)
            else:
                kb = np.ascontiguousarray(inp["kv_k"][b, :, :L])
                vb = np.ascontiguousarray(inp["kv_v"][b, :, :L])
            kt = torch.from_numpy(kb).to(self.device)
            vt = torch.from_numpy(vb).to(self.device)
            self.load_prefix_kv(b, kt, vt, L)
            keep.append((kt, vt))
        torch.cuda.synchronize(self.device)
        return keep

    def decide(self, noise, out=None):
        """noise: device float32 tensor [batch][rows][state_dim]."""
        torch = self.torch
        if out is None:
            out = torch.empty_like(noise)
        B.phx_expert_decide(self.h, noise.data_ptr(), out.data_ptr(), self.stream)
        return out

    def kernels_per_decision(self) -> int:
        return B.phx_expert_kernels_per_decision(self.h)

    def close(self):
        if getattr(self, "h", 0):
            self.torch.cuda.synchronize(self.device)
            B.phx_expert_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
