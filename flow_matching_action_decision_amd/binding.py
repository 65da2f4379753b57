"""ctypes binding of libphx_expert.so, with the C ABI's names.

Argument marshalling only: every step of the decision runs in the library's
HIP kernels.  torch supplies device memory and streams.  There is no CPU
fallback: if the library is missing the import of this module's functions
raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libphx_expert.so")

PHX_ABI_VERSION = 2
PHX_OK, PHX_E_INVALID, PHX_E_VERSION, PHX_E_SHAPE, PHX_E_STATE, PHX_E_NOMEM, PHX_E_HIP = 0, -1, -2, -3, -4, -5, -6
PHX_DTYPE_F32, PHX_DTYPE_BF16 = 0, 1
PHX_FLAG_NO_GRAPH = 1
PHX_FLAG_MULTI_KERNEL = 2
PHX_FLAG_TIMELINE = 4
PHX_FLAG_WEIGHTS_INT8 = 8
PHX_FLAG_PAIRED_ACT = 16
PHX_FLAG_BF16_ACT = 32
PHX_BLOCK_DECODER, PHX_BLOCK_DIT, PHX_BLOCK_PREFILL = 0, 1, 2
_BLOCKS = dict(decoder=PHX_BLOCK_DECODER, dit=PHX_BLOCK_DIT, prefill=PHX_BLOCK_PREFILL)
# launch kinds reported by phx_expert_node_info
PHX_NODE = dict(IN_PROJ=1, NORM_QKV_ROPE=2, ATTENTION=3, ATTN_COMBINE=4, OUT_PROJ_RESID=5, NORM_GATEUP_GEGLU=6,
                DOWN_PROJ_RESID=7, NORM_OUT_EULER=8, DECISION=9, TAG_ADVANCE=10, ROW_NORM=11, QKV=12, GATEUP=13,
                OUT_EULER=14, STATE_CVT=15)
PHX_MASK_FULL, PHX_MASK_CAUSAL = 0, 1

# every function include/phx_expert.h declares
EXPORTED = ("phx_expert_validate_config", "phx_expert_weights_bytes", "phx_expert_create",
            "phx_expert_load_prefix_kv", "phx_expert_decide", "phx_expert_decide_noalloc", "phx_expert_destroy",
            "phx_last_error",
            "phx_expert_kernels_per_decision", "phx_expert_node_info", "phx_expert_launch_node",
            "phx_expert_status", "phx_expert_timeline", "phx_expert_capsule_bytes", "phx_expert_capsule_regions",
            "phx_expert_capsule_save", "phx_expert_capsule_restore", "phx_expert_commit_chunk",
            "phx_expert_prefill", "phx_expert_weight_codes")

NODE_KINDS = {1: "in_proj", 2: "norm_qkv_rope", 3: "attention", 4: "attention_combine", 5: "out_proj_resid",
              6: "norm_gateup_geglu", 7: "down_proj_resid", 8: "norm_out_proj_euler", 9: "decision_kernel",
              10: "tag_advance", 11: "row_norm", 12: "qkv", 13: "gateup", 14: "out_proj_euler", 15: "state_cvt"}


class phx_capsule_region(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 24), ("offset", ctypes.c_uint64), ("bytes", ctypes.c_uint64)]


class phx_expert_config(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32), ("struct_size", ctypes.c_uint32),
        ("layers", ctypes.c_int32), ("width", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("mlp_hidden", ctypes.c_int32),
        ("state_dim", ctypes.c_int32), ("rows", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("prefix_capacity", ctypes.c_int32), ("steps", ctypes.c_int32), ("time_emb_dim", ctypes.c_int32),
        ("tau0", ctypes.c_float), ("dt", ctypes.c_float), ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
        ("weight_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("block_kind", ctypes.c_int32), ("mask_kind", ctypes.c_int32),
    ]


class phx_node_info(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("step", ctypes.c_int32), ("layer", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("bytes", ctypes.c_uint64), ("name", ctypes.c_char * 32)]


class PhxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with flow_matching_action_decision_amd/build.py "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    CP = ctypes.POINTER(phx_expert_config)
    lib.phx_expert_validate_config.argtypes = [CP]
    lib.phx_expert_weights_bytes.argtypes = [CP, ctypes.POINTER(ctypes.c_size_t)]
    lib.phx_expert_create.argtypes = [CP, P, ctypes.c_size_t, P, ctypes.POINTER(P)]
    lib.phx_expert_load_prefix_kv.argtypes = [P, ctypes.c_int32, P, P, ctypes.c_int32, P]
    lib.phx_expert_decide.argtypes = [P, P, P, P]
    lib.phx_expert_decide_noalloc.argtypes = [P, P, P, P]
    lib.phx_expert_destroy.argtypes = [P]
    lib.phx_expert_destroy.restype = None
    lib.phx_last_error.restype = ctypes.c_char_p
    lib.phx_expert_kernels_per_decision.argtypes = [P, ctypes.POINTER(ctypes.c_int)]
    lib.phx_expert_node_info.argtypes = [P, ctypes.c_int32, ctypes.POINTER(phx_node_info)]
    lib.phx_expert_launch_node.argtypes = [P, ctypes.c_int32, P]
    lib.phx_expert_status.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
    lib.phx_expert_timeline.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), ctypes.c_size_t,
                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.phx_expert_capsule_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.phx_expert_capsule_regions.argtypes = [P, ctypes.POINTER(phx_capsule_region), ctypes.c_int32,
                                               ctypes.POINTER(ctypes.c_int32)]
    lib.phx_expert_capsule_save.argtypes = [P, P, ctypes.c_size_t, P]
    lib.phx_expert_capsule_restore.argtypes = [P, P, ctypes.c_size_t, P]
    lib.phx_expert_commit_chunk.argtypes = [P, P, P]
    lib.phx_expert_prefill.argtypes = [P, P, ctypes.c_int32, P, P, P]
    lib.phx_expert_weight_codes.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, P]
    _lib = lib
    return lib


def make_config(cfg: dict, flags: int = 0) -> phx_expert_config:
    """phx_expert_config from a workload dict (phx_inputs naming)."""
    dt = PHX_DTYPE_BF16 if cfg["dtype"] == "bf16" else PHX_DTYPE_F32
    return phx_expert_config(
        abi_version=PHX_ABI_VERSION, struct_size=ctypes.sizeof(phx_expert_config),
        layers=cfg["layers"], width=cfg["width"], n_heads=cfg["n_heads"], head_dim=cfg["head_dim"],
        n_kv_heads=cfg["n_kv_heads"], mlp_hidden=cfg["mlp_hidden"], state_dim=cfg["state_dim"], rows=cfg["rows"],
        batch=cfg["batch"], prefix_capacity=cfg["capacity"], steps=cfg["steps"], time_emb_dim=cfg["time_emb_dim"],
        tau0=cfg["tau0"], dt=cfg["dt"], rms_eps=cfg["rms_eps"], rope_base=cfg["rope_base"],
        weight_dtype=dt, kv_dtype=dt, flags=flags | int(cfg.get("flags", 0)),
        block_kind=_BLOCKS[cfg.get("block", "decoder")],
        mask_kind=PHX_MASK_CAUSAL if cfg.get("block", "decoder") == "prefill" else PHX_MASK_FULL)


def _check(rc: int):
    if rc != PHX_OK:
        raise PhxError(rc, load_library().phx_last_error().decode())


def phx_last_error() -> str:
    return load_library().phx_last_error().decode()


def phx_expert_validate_config(cfg: phx_expert_config) -> int:
    return load_library().phx_expert_validate_config(ctypes.byref(cfg))


def phx_expert_weights_bytes(cfg: phx_expert_config) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().phx_expert_weights_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def phx_expert_create(cfg: phx_expert_config, weights_ptr: int, weights_bytes: int, stream: int = 0) -> int:
    h = ctypes.c_void_p(0)
    _check(load_library().phx_expert_create(ctypes.byref(cfg), ctypes.c_void_p(weights_ptr), weights_bytes,
                                            ctypes.c_void_p(stream), ctypes.byref(h)))
    return h.value


def phx_expert_load_prefix_kv(h: int, request: int, k_ptr: int, v_ptr: int, prefix_len: int, stream: int = 0):
    _check(load_library().phx_expert_load_prefix_kv(ctypes.c_void_p(h), request, ctypes.c_void_p(k_ptr),
                                                    ctypes.c_void_p(v_ptr), prefix_len, ctypes.c_void_p(stream)))


def phx_expert_decide(h: int, noise_ptr: int, actions_ptr: int, stream: int = 0):
    _check(load_library().phx_expert_decide(ctypes.c_void_p(h), ctypes.c_void_p(noise_ptr),
                                            ctypes.c_void_p(actions_ptr), ctypes.c_void_p(stream)))


def phx_expert_decide_noalloc(h: int, noise_ptr: int, actions_ptr: int, stream: int = 0):
    _check(load_library().phx_expert_decide_noalloc(ctypes.c_void_p(h), ctypes.c_void_p(noise_ptr),
                                                    ctypes.c_void_p(actions_ptr), ctypes.c_void_p(stream)))


def phx_expert_destroy(h: int):
    if h:
        load_library().phx_expert_destroy(ctypes.c_void_p(h))


def phx_expert_kernels_per_decision(h: int) -> int:
    n = ctypes.c_int(0)
    _check(load_library().phx_expert_kernels_per_decision(ctypes.c_void_p(h), ctypes.byref(n)))
    return n.value


def phx_expert_node_info(h: int, node: int) -> dict:
    info = phx_node_info()
    _check(load_library().phx_expert_node_info(ctypes.c_void_p(h), node, ctypes.byref(info)))
    return dict(kind=info.kind, step=info.step, layer=info.layer, bytes=int(info.bytes), name=info.name.decode())


def phx_expert_launch_node(h: int, node: int, stream: int = 0):
    _check(load_library().phx_expert_launch_node(ctypes.c_void_p(h), node, ctypes.c_void_p(stream)))


def phx_expert_status(h: int) -> int:
    st = ctypes.c_uint32(0)
    _check(load_library().phx_expert_status(ctypes.c_void_p(h), ctypes.byref(st)))
    return st.value


def phx_expert_timeline(h: int):
    """Per-workgroup phase timeline as a numpy array [workgroups][events] of
    uint32 ticks of the 100 MHz real-time counter."""
    import numpy as np
    lib = load_library()
    n = ctypes.c_size_t(0)
    lib.phx_expert_timeline(ctypes.c_void_p(h), None, 0, ctypes.byref(n))
    if n.value == 0:
        _check(PHX_E_STATE)
    out = np.zeros(n.value, dtype=np.uint32)
    _check(lib.phx_expert_timeline(ctypes.c_void_p(h), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), n.value,
                                   ctypes.byref(n)))
    return out.reshape(256, -1)


def phx_expert_capsule_bytes(h: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().phx_expert_capsule_bytes(ctypes.c_void_p(h), ctypes.byref(n)))
    return n.value


def phx_expert_capsule_regions(h: int) -> list:
    lib = load_library()
    n = ctypes.c_int32(0)
    _check(lib.phx_expert_capsule_regions(ctypes.c_void_p(h), None, 0, ctypes.byref(n)))
    arr = (phx_capsule_region * max(n.value, 1))()
    _check(lib.phx_expert_capsule_regions(ctypes.c_void_p(h), arr, n.value, ctypes.byref(n)))
    return [dict(name=arr[i].name.decode(), offset=int(arr[i].offset), bytes=int(arr[i].bytes)) for i in range(n.value)]


def phx_expert_capsule_save(h: int, capsule: int, nbytes: int, stream: int = 0):
    _check(load_library().phx_expert_capsule_save(ctypes.c_void_p(h), ctypes.c_void_p(capsule), nbytes,
                                                  ctypes.c_void_p(stream)))


def phx_expert_capsule_restore(h: int, capsule: int, nbytes: int, stream: int = 0):
    _check(load_library().phx_expert_capsule_restore(ctypes.c_void_p(h), ctypes.c_void_p(capsule), nbytes,
                                                     ctypes.c_void_p(stream)))


def phx_expert_commit_chunk(h: int, chunk: int, stream: int = 0):
    _check(load_library().phx_expert_commit_chunk(ctypes.c_void_p(h), ctypes.c_void_p(chunk), ctypes.c_void_p(stream)))


def phx_expert_prefill(h: int, x: int, prefix_len: int, k: int, v: int, stream: int = 0):
    _check(load_library().phx_expert_prefill(ctypes.c_void_p(h), ctypes.c_void_p(x), prefix_len, ctypes.c_void_p(k),
                                             ctypes.c_void_p(v), ctypes.c_void_p(stream)))


def phx_expert_weight_codes(h: int, layer: int, matrix: int, codes: int, scales: int, stream: int = 0):
    _check(load_library().phx_expert_weight_codes(ctypes.c_void_p(h), layer, matrix, ctypes.c_void_p(codes),
                                                  ctypes.c_void_p(scales), ctypes.c_void_p(stream)))
