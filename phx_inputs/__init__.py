"""Seeded synthetic inputs for the action-expert decision.

This module is the only code the oracle side and the HIP side share.  It
holds none of the method's arithmetic: it names the workloads, draws seeded
random tensors and rounds them to bfloat16 storage.

Recipe (stated once, used everywhere):
  * generator: numpy PCG64 via ``default_rng([workload_id, tensor_id, seed])``;
  * weights: one float32 draw of N(0, 0.02) (0.02 is the standard deviation)
    over the whole blob in its documented order, then round-to-nearest-even to
    bfloat16 for the bf16 workloads;
  * prefix K and V: N(0, 1) float32, rounded to bfloat16 for bf16 workloads,
    laid out [B][NL][C][KVH*Dh]; rows past a request's prefix length are drawn
    too (they must never be read);
  * noise: N(0, 1) float32, [B][M][A];
  * prefix lengths: fixed for single-request workloads; for the rollout batch
    drawn uniformly from {512, 640, 768, 800};
  * large-token workloads: the video-action chunk draws its cache like the
    prefix K/V above (4096 of 8192 rows used) and its 256 chunk rows as the
    noise; the DiT-style step draws its 4128 token rows x [T][D] as the noise;
    the prefix prefill draws its token rows x [rows][D] as the noise (its
    norm gains G are part of the one N(0, 0.02) weight draw).

The prefix K/V stands in for the key/value cache a vision-language prefix of
about 500 to 800 tokens would write; random values match its shape and bytes,
not its attention statistics.
"""
from __future__ import annotations

import copy

import numpy as np

# tensor ids for the generator key
T_WEIGHTS, T_KV_K, T_KV_V, T_NOISE, T_LENS = 1, 2, 3, 4, 5

_BASE = dict(width=1024, n_heads=8, head_dim=256, n_kv_heads=1, mlp_hidden=4096, state_dim=32, rows=10,
             time_emb_dim=1024, tau0=1.0, dt=-0.1, rms_eps=1e-6, rope_base=10000.0, weight_std=0.02,
             block="decoder")

WORKLOADS = {
    # one decoder layer, one Euler step, float32 throughout, 64-token prefix
    "single_layer_fp32": dict(_BASE, id=0, layers=1, batch=1, capacity=64, steps=1, dtype="f32",
                              prefix_lens=[64]),
    # pi0.5-shape action expert: 18 layers, 10 steps, 768-token prefix, bf16
    "pi05_expert_bf16": dict(_BASE, id=1, layers=18, batch=1, capacity=768, steps=10, dtype="bf16",
                             prefix_lens=[768]),
    # the pi0.5 shape on the 8-bit weight tier (same inputs as pi05_expert_bf16; flag 8 asks the library
    # to quantise the layer projections to int8 per output column)
    "pi05_expert_w8a16": dict(_BASE, id=1, layers=18, batch=1, capacity=768, steps=10, dtype="bf16",
                              prefix_lens=[768], flags=8),
    # 16 independent requests, ragged prefixes drawn from {512,640,768,800}, capacity 800
    "rollout_b16_bf16": dict(_BASE, id=2, layers=18, batch=16, capacity=800, steps=10, dtype="bf16",
                             prefix_lens="draw"),
    # video-action chunk denoise: 256 new tokens over a 4096-token cache (capacity 8192), width 2048,
    # 16 heads x 128 with full K/V heads, GeGLU 8192, 8 layers, 5 steps of dt = -0.2; the state is the
    # chunk itself (in/out linears 2048 x 2048)
    "va_chunk_bf16": dict(_BASE, id=3, layers=8, width=2048, n_heads=16, head_dim=128, n_kv_heads=16,
                          mlp_hidden=8192, state_dim=2048, rows=256, batch=1, capacity=8192, steps=5, dt=-0.2,
                          dtype="bf16", prefix_lens=[4096]),
    # DiT-style denoise step: 4096 video + 32 action tokens, full bidirectional self-attention, width 3072,
    # 24 heads x 128, GELU MLP 12288, adaLN-Zero modulation (shift, scale, gate) from the tau = 1 embedding,
    # 4 blocks, one step, output = residual stream
    "wam_dit_bf16": dict(_BASE, id=4, block="dit", layers=4, width=3072, n_heads=24, head_dim=128,
                         n_kv_heads=24, mlp_hidden=12288, state_dim=3072, rows=4128, batch=1, capacity=0,
                         steps=1, dt=0.0, dtype="bf16", prefix_lens=[0]),
    # prefix prefill: the 18-layer language model (width 2048, 8 query heads x 256 over one K/V head,
    # GeGLU 16384, causal) over a 768-token prefix in an 800-row bucket; writes the K/V the expert reads.
    # The token rows x [rows][D] are drawn as the noise; prefix_lens holds the prefilled length.
    "prefix_prefill_bf16": dict(_BASE, id=5, block="prefill", layers=18, width=2048, n_heads=8, head_dim=256,
                                n_kv_heads=1, mlp_hidden=16384, state_dim=2048, rows=800, batch=1, capacity=0,
                                steps=1, dt=0.0, dtype="bf16", prefix_lens=[768]),
}

RAGGED_CHOICES = (512, 640, 768, 800)


def workload(name: str, **overrides) -> dict:
    """A copy of a named workload's configuration, with optional overrides."""
    cfg = copy.deepcopy(WORKLOADS[name])
    cfg["name"] = name
    cfg.update(overrides)
    return cfg


def rng(cfg: dict, tensor_id: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(cfg.get("id", 99)), int(tensor_id), int(seed)])


def bf16_round(a: np.ndarray):
    """Round float32 to the nearest bfloat16 (ties to even).

    Returns (values as float32, raw uint16 bits).  Inputs are finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    bits = (r >> np.uint32(16)).astype(np.uint16)
    return r.view(np.float32), bits


def weight_count(cfg: dict) -> int:
    """Number of scalars in the weight blob (documented order)."""
    D, A, F = cfg["width"], cfg["state_dim"], cfg["mlp_hidden"]
    H, KVH, Dh, NL, E = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["layers"], cfg["time_emb_dim"]
    qkv = (H + 2 * KVH) * Dh
    if cfg.get("block", "decoder") == "dit":
        return NL * (D * qkv + H * Dh * D + D * F + F * D) + NL * E * 6 * D
    if cfg.get("block", "decoder") == "prefill":
        return NL * (D * qkv + H * Dh * D + D * 2 * F + F * D) + 2 * NL * D
    per_layer = D * qkv + H * Dh * D + D * 2 * F + F * D
    return A * D + NL * per_layer + D * A + (2 * NL + 1) * E * 2 * D


def prefix_lengths(cfg: dict, seed: int = 0) -> np.ndarray:
    pl = cfg.get("prefix_lens", [cfg["capacity"]] * cfg["batch"])
    if isinstance(pl, str) and pl == "draw":
        g = rng(cfg, T_LENS, seed)
        return g.choice(np.array(RAGGED_CHOICES, dtype=np.int32), size=cfg["batch"]).astype(np.int32)
    arr = np.asarray(pl, dtype=np.int32)
    if arr.size == 1 and cfg["batch"] > 1:
        arr = np.full(cfg["batch"], int(arr[0]), dtype=np.int32)
    return arr


def make_weights(cfg: dict, seed: int = 0):
    """(float32 values, uint16 bf16 bits or None)."""
    g = rng(cfg, T_WEIGHTS, seed)
    w = g.standard_normal(weight_count(cfg), dtype=np.float32)
    w *= np.float32(cfg.get("weight_std", 0.02))
    if cfg["dtype"] == "bf16":
        return bf16_round(w)
    return w, None


def make_kv(cfg: dict, seed: int = 0):
    """K and V caches [B][NL][C][KVH*Dh]: (k values, v values, k bits, v bits)."""
    shape = (cfg["batch"], cfg["layers"], cfg["capacity"], cfg["n_kv_heads"] * cfg["head_dim"])
    k = rng(cfg, T_KV_K, seed).standard_normal(shape, dtype=np.float32)
    v = rng(cfg, T_KV_V, seed).standard_normal(shape, dtype=np.float32)
    if cfg["dtype"] == "bf16":
        kv_, kb = bf16_round(k)
        vv_, vb = bf16_round(v)
        return kv_.reshape(shape), vv_.reshape(shape), kb.reshape(shape), vb.reshape(shape)
    return k, v, None, None


def make_noise(cfg: dict, seed: int = 0) -> np.ndarray:
    return rng(cfg, T_NOISE, seed).standard_normal((cfg["batch"], cfg["rows"], cfg["state_dim"]),
                                                   dtype=np.float32)


def make_inputs(cfg: dict, seed: int = 0) -> dict:
    """All inputs of one decision.  Values are float32 (bf16-representable
    for bf16 workloads); ``*_bits`` hold the raw bfloat16 storage."""
    w, wb = make_weights(cfg, seed)
    k, v, kb, vb = make_kv(cfg, seed)
    return dict(weights=w, weights_bits=wb, kv_k=k, kv_v=v, kv_k_bits=kb, kv_v_bits=vb,
                lens=prefix_lengths(cfg, seed), noise=make_noise(cfg, seed))


def weight_slices(cfg: dict) -> dict:
    """Offsets (start, shape) of every matrix in the blob, by name.  Used by
    tests to plant special weights (zeros, structured values)."""
    D, A, F = cfg["width"], cfg["state_dim"], cfg["mlp_hidden"]
    H, KVH, Dh, NL, E = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["layers"], cfg["time_emb_dim"]
    qkv = (H + 2 * KVH) * Dh
    out = {}
    off = 0

    def put(name, shape):
        nonlocal off
        out[name] = (off, shape)
        off += int(np.prod(shape))

    if cfg.get("block", "decoder") == "dit":
        for l in range(NL):
            put(f"W_qkv.{l}", (D, qkv))
            put(f"W_o.{l}", (H * Dh, D))
            put(f"W_up.{l}", (D, F))
            put(f"W_down.{l}", (F, D))
        put("W_mod", (NL, E, 6 * D))
        assert off == weight_count(cfg)
        return out
    if cfg.get("block", "decoder") == "prefill":
        for l in range(NL):
            put(f"W_qkv.{l}", (D, qkv))
            put(f"W_o.{l}", (H * Dh, D))
            put(f"W_gu.{l}", (D, 2 * F))
            put(f"W_down.{l}", (F, D))
        put("G", (2 * NL, D))
        assert off == weight_count(cfg)
        return out
    put("W_in", (A, D))
    for l in range(NL):
        put(f"W_qkv.{l}", (D, qkv))
        put(f"W_o.{l}", (H * Dh, D))
        put(f"W_gu.{l}", (D, 2 * F))
        put(f"W_down.{l}", (F, D))
    put("W_out", (D, A))
    put("W_mod", (2 * NL + 1, E, 2 * D))
    assert off == weight_count(cfg)
    return out


def view(weights: np.ndarray, cfg: dict, name: str) -> np.ndarray:
    """A writable view of one matrix inside a weight blob."""
    off, shape = weight_slices(cfg)[name]
    return weights[off:off + int(np.prod(shape))].reshape(shape)
