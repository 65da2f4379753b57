"""CPU oracle for one flow-matching action-expert decision (double precision).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and it
imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, fixed-order loops, OpenMP only
across independent outputs); this module builds it with gcc and marshals
numpy arrays through ctypes.  Every function cites, in ``oracle.c``, the
passage of the pages it follows.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(library routines, closed forms, invariants, a tiny brute-force composition
and a mutation sweep); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (-O3, no fast-math, OpenMP)."""
    cmd = ["gcc", "-O3", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-I", _HERE, "-o", out, src, "-lm"]
    subprocess.check_call(cmd)
    return out


class OrcConfig(ctypes.Structure):
    _fields_ = [
        ("layers", ctypes.c_int), ("width", ctypes.c_int), ("n_heads", ctypes.c_int),
        ("head_dim", ctypes.c_int), ("n_kv_heads", ctypes.c_int), ("mlp_hidden", ctypes.c_int),
        ("state_dim", ctypes.c_int), ("rows", ctypes.c_int), ("batch", ctypes.c_int),
        ("capacity", ctypes.c_int), ("steps", ctypes.c_int), ("time_emb_dim", ctypes.c_int),
        ("tau0", ctypes.c_double), ("dt", ctypes.c_double), ("rms_eps", ctypes.c_double),
        ("rope_base", ctypes.c_double),
    ]


_DP = ctypes.POINTER(ctypes.c_double)
_FP = ctypes.POINTER(ctypes.c_float)
_IP = ctypes.POINTER(ctypes.c_int)


def load(path: str = LIB_PATH):
    """Load (building first if absent) and return the ctypes library."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    lib.orc_weight_count.argtypes = [ctypes.POINTER(OrcConfig)]
    lib.orc_weight_count.restype = ctypes.c_size_t
    lib.orc_time_embedding.argtypes = [ctypes.c_int, ctypes.c_double, _DP]
    lib.orc_modulation.argtypes = [ctypes.c_int, ctypes.c_int, _FP, _DP, _DP]
    lib.orc_ada_rmsnorm.argtypes = [ctypes.c_int, ctypes.c_int, _DP, _DP, ctypes.c_double, _DP]
    lib.orc_matmul.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _DP, _FP, _DP]
    lib.orc_rope.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _IP, ctypes.c_double, _DP]
    lib.orc_gelu_tanh.argtypes = [ctypes.c_double]
    lib.orc_gelu_tanh.restype = ctypes.c_double
    lib.orc_attention.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  _DP, _DP, _DP, _FP, _FP, ctypes.c_size_t, _DP]
    lib.orc_attention.restype = ctypes.c_double
    lib.orc_decide.argtypes = [ctypes.POINTER(OrcConfig), _FP, _FP, _FP, _IP, _FP, _DP, _DP, _DP]
    lib.orc_decide.restype = ctypes.c_int
    lib.orc_decide_at.argtypes = [ctypes.POINTER(OrcConfig), _FP, _FP, _FP, _IP, _IP, _FP, _DP, _DP, _DP]
    lib.orc_decide_at.restype = ctypes.c_int
    lib.orc_commit.argtypes = [ctypes.POINTER(OrcConfig), _FP, _FP, _FP, _IP, _IP, _FP, ctypes.c_double, _DP, _DP,
                               _DP]
    lib.orc_commit.restype = ctypes.c_int
    lib.orc_last_softmax_dev.restype = ctypes.c_double
    lib.orc_ada_layernorm.argtypes = [ctypes.c_int, ctypes.c_int, _DP, _DP, _DP, ctypes.c_double, _DP]
    lib.orc_dit.argtypes = [ctypes.POINTER(OrcConfig), _FP, _FP, _DP, _DP]
    lib.orc_dit.restype = ctypes.c_int
    lib.orc_dit_weight_count.argtypes = [ctypes.POINTER(OrcConfig)]
    lib.orc_dit_weight_count.restype = ctypes.c_size_t
    lib.orc_prefill.argtypes = [ctypes.POINTER(OrcConfig), _FP, _FP, ctypes.c_int, _DP, _DP, _DP]
    lib.orc_prefill.restype = ctypes.c_int
    lib.orc_prefill_weight_count.argtypes = [ctypes.POINTER(OrcConfig)]
    lib.orc_prefill_weight_count.restype = ctypes.c_size_t
    lib.orc_quantize_i8.argtypes = [ctypes.c_int, ctypes.c_int, _FP, ctypes.POINTER(ctypes.c_int8), _FP]
    if path == LIB_PATH:
        _lib = lib
    return lib


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_DP)


def _f(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_FP)


def make_config(cfg: dict) -> OrcConfig:
    return OrcConfig(
        layers=cfg["layers"], width=cfg["width"], n_heads=cfg["n_heads"], head_dim=cfg["head_dim"],
        n_kv_heads=cfg["n_kv_heads"], mlp_hidden=cfg["mlp_hidden"], state_dim=cfg["state_dim"],
        rows=cfg["rows"], batch=cfg["batch"], capacity=cfg["capacity"], steps=cfg["steps"],
        time_emb_dim=cfg["time_emb_dim"], tau0=cfg["tau0"], dt=cfg["dt"], rms_eps=cfg["rms_eps"],
        rope_base=cfg["rope_base"])


def weight_count(cfg: dict, lib=None) -> int:
    lib = lib or load()
    c = make_config(cfg)
    if cfg.get("block", "decoder") == "dit":
        return int(lib.orc_dit_weight_count(ctypes.byref(c)))
    if cfg.get("block", "decoder") == "prefill":
        return int(lib.orc_prefill_weight_count(ctypes.byref(c)))
    return int(lib.orc_weight_count(ctypes.byref(c)))


def time_embedding(E: int, tau: float, lib=None) -> np.ndarray:
    lib = lib or load()
    out = np.zeros(E, dtype=np.float64)
    lib.orc_time_embedding(E, tau, out.ctypes.data_as(_DP))
    return out


def modulation(e: np.ndarray, W_mod_n: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    E, D2 = W_mod_n.shape
    out = np.zeros(D2, dtype=np.float64)
    e, pe = _d(e)
    W, pW = _f(W_mod_n)
    lib.orc_modulation(E, D2 // 2, pW, pe, out.ctypes.data_as(_DP))
    return out


def ada_rmsnorm(h: np.ndarray, mod: np.ndarray, eps: float, lib=None) -> np.ndarray:
    lib = lib or load()
    M, D = h.shape
    out = np.zeros((M, D), dtype=np.float64)
    h, ph = _d(h)
    mod, pm = _d(mod)
    lib.orc_ada_rmsnorm(M, D, ph, pm, eps, out.ctypes.data_as(_DP))
    return out


def matmul(x: np.ndarray, W: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    M, K = x.shape
    K2, N = W.shape
    assert K == K2
    out = np.zeros((M, N), dtype=np.float64)
    x, px = _d(x)
    W, pW = _f(W)
    lib.orc_matmul(M, K, N, px, pW, out.ctypes.data_as(_DP))
    return out


def rope(x: np.ndarray, n_heads: int, head_dim: int, pos, base: float, lib=None) -> np.ndarray:
    lib = lib or load()
    M = x.shape[0]
    y = np.array(x, dtype=np.float64, order="C", copy=True).reshape(M, n_heads * head_dim)
    p = np.ascontiguousarray(pos, dtype=np.int32)
    lib.orc_rope(M, n_heads, head_dim, p.ctypes.data_as(_IP), base, y.ctypes.data_as(_DP))
    return y.reshape(x.shape)


def gelu_tanh(z) -> np.ndarray:
    lib = load()
    z = np.asarray(z, dtype=np.float64)
    return np.vectorize(lambda v: lib.orc_gelu_tanh(float(v)))(z) if z.ndim else lib.orc_gelu_tanh(float(z))


def attention(q, ka, va, Kp, Vp, n_heads: int, n_kv_heads: int, head_dim: int, lib=None):
    """q [M][H*Dh], ka/va [M][KVH*Dh] (float64), Kp/Vp [L][KVH*Dh] float32.
    Returns (o [M][H*Dh], largest |sum p - 1|)."""
    lib = lib or load()
    M = q.shape[0]
    L = Kp.shape[0]
    q, pq = _d(q)
    ka, pka = _d(ka)
    va, pva = _d(va)
    if L == 0:  # no prefix rows: pass a dummy row that is never read
        Kp = Vp = np.zeros((1, n_kv_heads * head_dim), np.float32)
    Kp, pK = _f(Kp)
    Vp, pV = _f(Vp)
    o = np.zeros((M, n_heads * head_dim), dtype=np.float64)
    dev = lib.orc_attention(M, n_heads, n_kv_heads, head_dim, L, pq, pka, pva, pK, pV,
                            n_kv_heads * head_dim, o.ctypes.data_as(_DP))
    return o, dev


def decide(cfg: dict, weights: np.ndarray, kv_k, kv_v, lens, noise, trace: bool = False,
           velocity: bool = False, lib=None, pos0=None) -> dict:
    """Run one decision.  weights: float32 blob in the documented order.
    kv_k/kv_v: float32 [B][NL][C][KVH*Dh] (may be None when C == 0).
    pos0: optional [B] base positions (rows of request b at pos0[b] + lens[b] + i).
    Returns {"actions": [B][M][A] float64, "trace": ..., "velocity": ...,
    "softmax_dev": float}."""
    lib = lib or load()
    c = make_config(cfg)
    n_w = int(lib.orc_weight_count(ctypes.byref(c)))
    weights, pw = _f(weights)
    if weights.size != n_w:
        raise ValueError(f"weight blob has {weights.size} values, expected {n_w}")
    B, M, A, NL, D, S = cfg["batch"], cfg["rows"], cfg["state_dim"], cfg["layers"], cfg["width"], cfg["steps"]
    if kv_k is not None:
        kv_k, pk = _f(kv_k)
        kv_v, pv = _f(kv_v)
    else:
        pk = pv = None
    lens_a = np.ascontiguousarray(lens, dtype=np.int32)
    noise, pn = _f(noise)
    actions = np.zeros((B, M, A), dtype=np.float64)
    tr = np.zeros((S, NL + 1, B * M, D), dtype=np.float64) if trace else None
    vel = np.zeros((S, B * M, A), dtype=np.float64) if velocity else None
    if pos0 is None:
        rc = lib.orc_decide(ctypes.byref(c), pw, pk, pv, lens_a.ctypes.data_as(_IP), pn,
                            actions.ctypes.data_as(_DP),
                            tr.ctypes.data_as(_DP) if tr is not None else None,
                            vel.ctypes.data_as(_DP) if vel is not None else None)
    else:
        pos_a = np.ascontiguousarray(pos0, dtype=np.int32)
        rc = lib.orc_decide_at(ctypes.byref(c), pw, pk, pv, lens_a.ctypes.data_as(_IP), pos_a.ctypes.data_as(_IP),
                               pn, actions.ctypes.data_as(_DP),
                               tr.ctypes.data_as(_DP) if tr is not None else None,
                               vel.ctypes.data_as(_DP) if vel is not None else None)
    if rc != 0:
        raise ValueError(f"orc_decide rejected its arguments (rc={rc})")
    return {"actions": actions, "trace": tr, "velocity": vel, "softmax_dev": lib.orc_last_softmax_dev()}


def commit(cfg: dict, weights: np.ndarray, kv_k, kv_v, lens, x, tau: float, pos0=None, trace: bool = False,
           lib=None) -> dict:
    """Commit a decided chunk x [B][M][A] into the history: one pass of the
    layer stack at flow time tau.  Returns {"k", "v": [B][NL][M][KVH*Dh]
    float64 (keys after RoPE), "trace": [1][NL+1][B*M][D] or None}."""
    lib = lib or load()
    c = make_config(cfg)
    weights, pw = _f(weights)
    B, M, NL, D = cfg["batch"], cfg["rows"], cfg["layers"], cfg["width"]
    kvd = cfg["n_kv_heads"] * cfg["head_dim"]
    if kv_k is not None:
        kv_k, pk = _f(kv_k)
        kv_v, pv = _f(kv_v)
    else:
        pk = pv = None
    lens_a = np.ascontiguousarray(lens, dtype=np.int32)
    pos_a = np.ascontiguousarray(np.zeros(B) if pos0 is None else pos0, dtype=np.int32)
    x, px = _f(x)
    k = np.zeros((B, NL, M, kvd), dtype=np.float64)
    v = np.zeros((B, NL, M, kvd), dtype=np.float64)
    tr = np.zeros((1, NL + 1, B * M, D), dtype=np.float64) if trace else None
    rc = lib.orc_commit(ctypes.byref(c), pw, pk, pv, lens_a.ctypes.data_as(_IP), pos_a.ctypes.data_as(_IP), px,
                        float(tau), k.ctypes.data_as(_DP), v.ctypes.data_as(_DP),
                        tr.ctypes.data_as(_DP) if tr is not None else None)
    if rc != 0:
        raise ValueError(f"orc_commit rejected its arguments (rc={rc})")
    return {"k": k, "v": v, "trace": tr}


def ada_layernorm(h: np.ndarray, scale: np.ndarray, shift: np.ndarray, eps: float, lib=None) -> np.ndarray:
    lib = lib or load()
    h, ph = _d(h)
    M, D = h.shape
    scale, ps = _d(scale)
    shift, pb = _d(shift)
    out = np.zeros((M, D), dtype=np.float64)
    lib.orc_ada_layernorm(M, D, ph, ps, pb, eps, out.ctypes.data_as(_DP))
    return out


def dit(cfg: dict, weights: np.ndarray, x, trace: bool = False, lib=None) -> dict:
    """One DiT-style step over the cfg["rows"] tokens of x [T][D] (float32).
    Returns {"out": [T][D] float64, "trace": [NL][T][D] or None,
    "softmax_dev": float}."""
    lib = lib or load()
    c = make_config(cfg)
    n_w = int(lib.orc_dit_weight_count(ctypes.byref(c)))
    weights, pw = _f(weights)
    if weights.size != n_w:
        raise ValueError(f"weight blob has {weights.size} values, expected {n_w}")
    T, D, NL = cfg["rows"], cfg["width"], cfg["layers"]
    x, px = _f(np.asarray(x).reshape(T, D))
    out = np.zeros((T, D), dtype=np.float64)
    tr = np.zeros((NL, T, D), dtype=np.float64) if trace else None
    rc = lib.orc_dit(ctypes.byref(c), pw, px, out.ctypes.data_as(_DP),
                     tr.ctypes.data_as(_DP) if tr is not None else None)
    if rc != 0:
        raise ValueError(f"orc_dit rejected its arguments (rc={rc})")
    return {"out": out, "trace": tr, "softmax_dev": lib.orc_last_softmax_dev()}


def prefill(cfg: dict, weights: np.ndarray, x, length: int, trace: bool = False, lib=None) -> dict:
    """Prefix prefill over the first ``length`` token rows of x [>= length][D]
    (float32).  Returns {"k": [NL][length][KVH*Dh], "v": same (float64),
    "trace": [NL-1][length][D] or None, "softmax_dev": float}."""
    lib = lib or load()
    c = make_config(cfg)
    n_w = int(lib.orc_prefill_weight_count(ctypes.byref(c)))
    weights, pw = _f(weights)
    if weights.size != n_w:
        raise ValueError(f"weight blob has {weights.size} values, expected {n_w}")
    D, NL = cfg["width"], cfg["layers"]
    kvd = cfg["n_kv_heads"] * cfg["head_dim"]
    T = int(length)
    x, px = _f(np.asarray(x, dtype=np.float32).reshape(-1, D)[:T])
    k = np.zeros((NL, T, kvd), dtype=np.float64)
    v = np.zeros((NL, T, kvd), dtype=np.float64)
    tr = np.zeros((max(NL - 1, 1), T, D), dtype=np.float64) if trace else None
    rc = lib.orc_prefill(ctypes.byref(c), pw, px, T, k.ctypes.data_as(_DP), v.ctypes.data_as(_DP),
                         tr.ctypes.data_as(_DP) if tr is not None else None)
    if rc != 0:
        raise ValueError(f"orc_prefill rejected its arguments (rc={rc})")
    return {"k": k, "v": v, "trace": tr, "softmax_dev": lib.orc_last_softmax_dev()}


def quantize_i8(W: np.ndarray, lib=None):
    """Round-to-nearest int8 codes per output channel of W [K][N] (float32):
    returns (q int8 [K][N], s float32 [N]) with W ~ s * q."""
    lib = lib or load()
    W, pw = _f(np.asarray(W).reshape(W.shape[0], -1))
    K, N = W.shape
    q = np.zeros((K, N), dtype=np.int8)
    s = np.zeros(N, dtype=np.float32)
    lib.orc_quantize_i8(K, N, pw, q.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), s.ctypes.data_as(_FP))
    return q, s


# the projection matrices the 8-bit tier quantises: every layer's four matrices
W8_MATRICES = ("W_qkv", "W_o", "W_gu", "W_down")


def w8_weights(cfg: dict, weights: np.ndarray, slices: dict, lib=None) -> np.ndarray:
    """The weight blob the 8-bit tier computes with: every layer's W_qkv,
    W_o, W_gu and W_down replaced by s * q (float64 product rounded to
    float32, a relative change of at most 2^-24); the other matrices as
    given.  `slices` maps names to (offset, shape), as phx_inputs lays the
    blob out."""
    out = np.array(weights, dtype=np.float32, copy=True)
    for l in range(cfg["layers"]):
        for nm in W8_MATRICES:
            off, shape = slices[f"{nm}.{l}"]
            n = int(np.prod(shape))
            W = out[off:off + n].reshape(shape)
            q, s = quantize_i8(W, lib=lib)
            out[off:off + n] = (q.astype(np.float64) * s.astype(np.float64)[None, :]).astype(np.float32).reshape(-1)
    return out
