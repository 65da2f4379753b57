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

    def decide_noalloc(self, noise, out):
        """As decide, through the allocation-free entry point (the device's
        static exchange memory); out must be preallocated."""
        B.phx_expert_decide_noalloc(self.h, noise.data_ptr(), out.data_ptr(), self.stream)
        return out

    def status(self) -> int:
        """0 if the last decision completed; nonzero if the persistent kernel gave up waiting."""
        return B.phx_expert_status(self.h)

    def timeline(self):
        return B.phx_expert_timeline(self.h)

    def commit_chunk(self, chunk):
        """Commit a chunk (device float32 [rows][state_dim]) into the history."""
        B.phx_expert_commit_chunk(self.h, chunk.data_ptr(), self.stream)

    def prefill(self, x, prefix_len: int, k=None, v=None):
        """Prefix prefill: x device float32 [>= prefix_len][width]; returns
        (k, v) device int16 tensors (raw bfloat16) [layers][prefix_len][KVH*Dh],
        the layout load_prefix_kv takes."""
        torch = self.torch
        cfg = self.cfg
        shape = (cfg["layers"], prefix_len, cfg["n_kv_heads"] * cfg["head_dim"])
        if k is None:
            k = torch.empty(shape, dtype=torch.int16, device=self.device)
        if v is None:
            v = torch.empty(shape, dtype=torch.int16, device=self.device)
        B.phx_expert_prefill(self.h, x.data_ptr(), prefix_len, k.data_ptr(), v.data_ptr(), self.stream)
        return k, v

    def weight_codes(self, layer: int, matrix: int):
        """The 8-bit tier's int8 codes [K][N] and scales [N] of one matrix
        (0 W_qkv, 1 W_o, 2 W_gu, 3 W_down) as device tensors."""
        torch = self.torch
        cfg = self.cfg
        D, F, H, KVH, Dh = cfg["width"], cfg["mlp_hidden"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        K = (D, H * Dh, D, F)[matrix]
        N = ((H + 2 * KVH) * Dh, D, 2 * F, D)[matrix]
        codes = torch.empty((K, N), dtype=torch.int8, device=self.device)
        scales = torch.empty(N, dtype=torch.float32, device=self.device)
        B.phx_expert_weight_codes(self.h, layer, matrix, codes.data_ptr(), scales.data_ptr(), self.stream)
        return codes, scales

    def capsule_bytes(self) -> int:
        return B.phx_expert_capsule_bytes(self.h)

    def capsule_regions(self) -> list:
        return B.phx_expert_capsule_regions(self.h)

    def capsule_save(self, capsule=None):
        """Snapshot the state regions into a device uint8 tensor (allocated if
        not given); returns it."""
        torch = self.torch
        n = self.capsule_bytes()
        if capsule is None:
            capsule = torch.empty(n, dtype=torch.uint8, device=self.device)
        B.phx_expert_capsule_save(self.h, capsule.data_ptr(), capsule.numel(), self.stream)
        return capsule

    def capsule_restore(self, capsule):
        B.phx_expert_capsule_restore(self.h, capsule.data_ptr(), capsule.numel(), self.stream)

    def kernels_per_decision(self) -> int:
        return B.phx_expert_kernels_per_decision(self.h)

    def nodes(self) -> list:
        """Every kernel launch of one decision, in replay order."""
        return [B.phx_expert_node_info(self.h, i) for i in range(self.kernels_per_decision())]

    def time_nodes(self, idx: list, reps: int = 20) -> list:
        """Average duration (ms) of each launch in idx, relaunched on its own
        `reps` times, each bracketed by HIP events on the handle's stream."""
        torch = self.torch
        stream = torch.cuda.current_stream(self.device)
        for i in idx:  # warm
            B.phx_expert_launch_node(self.h, i, self.stream)
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
              for _ in idx]
        torch.cuda.synchronize(self.device)
        for r in range(reps):
            for j, i in enumerate(idx):
                a, b = ev[j][r]
                a.record(stream)
                B.phx_expert_launch_node(self.h, i, self.stream)
                b.record(stream)
        torch.cuda.synchronize(self.device)
        return [float(sum(a.elapsed_time(b) for a, b in e) / reps) for e in ev]

    def time_dominant_kernel(self, reps: int = 50) -> dict:
        """Average duration of one launch of the kernel that streams the most
        algorithmic bytes per decision.  Each launch (the first Euler step's
        launches of that kernel, all layers in turn, `reps` rounds) is
        bracketed by HIP events on the handle's stream."""
        torch = self.torch
        nodes = self.nodes()
        per_kind = {}
        for n in nodes:
            per_kind[n["kind"]] = per_kind.get(n["kind"], 0) + n["bytes"]
        kind = max(per_kind, key=per_kind.get)
        first_step = min(n["step"] for n in nodes if n["kind"] == kind)
        idx = [i for i, n in enumerate(nodes) if n["kind"] == kind and n["step"] == first_step]
        stream = torch.cuda.current_stream(self.device)
        for i in idx:  # warm
            B.phx_expert_launch_node(self.h, i, self.stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps * len(idx))]
        torch.cuda.synchronize(self.device)
        j = 0
        for _ in range(reps):
            for i in idx:
                a, b = ev[j]
                a.record(stream)
                B.phx_expert_launch_node(self.h, i, self.stream)
                b.record(stream)
                j += 1
        torch.cuda.synchronize(self.device)
        ms = [a.elapsed_time(b) for a, b in ev]
        return dict(name=nodes[idx[0]]["name"], kind=kind, launches=len(ms),
                    ms_per_launch=float(sum(ms) / len(ms)), bytes_per_launch=nodes[idx[0]]["bytes"])

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
