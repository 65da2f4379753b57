"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
compare against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import phx_inputs

# tolerances on the final actions (the accuracy bar of the workloads): bf16 weights and
# activations with fp32 accumulation vs the double-precision oracle
TOL_BF16 = dict(max_abs=2e-2, rel_l2=1e-2)
TOL_F32 = dict(max_abs=1e-4, rel_l2=1e-4)
# The large-token plans return many more values than the expert's actions
# (the DiT-style step returns its residual stream: 12.7M values of standard
# deviation ~1.3 at full size): they are held to the same bar, plus every
# row's cosine similarity, so that no row can hide a local mistake.  The
# DiT-style block meets it with paired GEMM activations (its default), which
# take the bf16 rounding of the QKV, gate/up and down inputs out of the
# residual stream.
TOL_TOKENS = dict(max_abs=2e-2, rel_l2=1e-2, worst_row_cos=0.9999)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_decide(cfg: dict, inp: dict, flags: int = 0, repeats: int = 1, noise=None):
    """Create a handle, load every prefix, run `repeats` decisions; returns
    the list of action arrays (float32 numpy) and the handle's kernel count."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    ex = Expert(cfg, inp["weights"], inp["weights_bits"], flags=flags)
    try:
        keep = ex.load_all(inp)
        nz = torch.from_numpy(np.ascontiguousarray(inp["noise"] if noise is None else noise)).cuda()
        outs = []
        for _ in range(repeats):
            a = ex.decide(nz)
            torch.cuda.synchronize()
            # PHX_OK only means enqueued: the status word says the decision ran to its end
            assert ex.status() == 0, "the decision gave up waiting (persistent kernel status)"
            outs.append(a.cpu().numpy().copy())
        del keep
        return outs, ex.kernels_per_decision()
    finally:
        ex.close()


def oracle_decide(cfg: dict, inp: dict):
    return oracle.decide(cfg, inp["weights"], inp["kv_k"], inp["kv_v"], inp["lens"], inp["noise"])["actions"]


def compare(gpu: np.ndarray, ref: np.ndarray) -> dict:
    g = np.asarray(gpu, dtype=np.float64).reshape(-1)
    r = np.asarray(ref, dtype=np.float64).reshape(-1)
    d = g - r
    rows_g = np.asarray(gpu, dtype=np.float64).reshape(-1, ref.shape[-1])
    rows_r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    cos_rows = np.sum(rows_g * rows_r, 1) / (np.linalg.norm(rows_g, axis=1) * np.linalg.norm(rows_r, axis=1) + 1e-300)
    return dict(max_abs=float(np.max(np.abs(d))), rel_l2=float(np.linalg.norm(d) / (np.linalg.norm(r) + 1e-300)),
                cos_global=float(np.dot(g, r) / (np.linalg.norm(g) * np.linalg.norm(r) + 1e-300)),
                cos_worst_row=float(np.min(cos_rows)), finite=bool(np.all(np.isfinite(g))))


def assert_close(gpu, ref, tol, what=""):
    m = compare(gpu, ref)
    say(f"  {what}: max_abs={m['max_abs']:.3e} rel_l2={m['rel_l2']:.3e} cos={m['cos_global']:.6f} "
        f"worst_row_cos={m['cos_worst_row']:.6f}")
    assert m["finite"], f"{what}: non-finite output"
    assert m["max_abs"] <= tol["max_abs"], f"{what}: max_abs {m['max_abs']:.3e} > {tol['max_abs']}"
    assert m["rel_l2"] <= tol["rel_l2"], f"{what}: rel_l2 {m['rel_l2']:.3e} > {tol['rel_l2']}"
    if "worst_row_cos" in tol:
        assert m["cos_worst_row"] >= tol["worst_row_cos"], f"{what}: worst row cosine {m['cos_worst_row']:.6f}"
    return m


def assert_close_bf16_storage(gpu, ref, tol, what=""):
    """The bar for values the interface stores in bf16 (the prefill's key and
    value cache): rounding a value r to bf16 (round to nearest even) moves it
    by up to half an ulp, 2^-9 |r|, so an exact computation stored in bf16
    already differs from the oracle's double by that much; the max-abs bar
    applies to what remains, |g - r| - 2^-9 |r|.  rel-L2 and the row cosine
    are taken as they are."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    excess = float(np.max(np.abs(g - r) - np.abs(r) * 2.0 ** -9))
    m = compare(gpu, ref)
    say(f"  {what}: max_abs={m['max_abs']:.3e} beyond storage half-ulp={excess:.3e} rel_l2={m['rel_l2']:.3e} "
        f"worst_row_cos={m['cos_worst_row']:.6f}")
    assert m["finite"], f"{what}: non-finite output"
    assert excess <= tol["max_abs"], f"{what}: max-abs beyond the bf16 storage rounding {excess:.3e} > {tol['max_abs']}"
    assert m["rel_l2"] <= tol["rel_l2"], f"{what}: rel_l2 {m['rel_l2']:.3e} > {tol['rel_l2']}"
    return m


def small_cfg(**kw) -> dict:
    """A small shape that still spans several tiles, several key chunks and a
    ragged tail: 2 layers, width 256, 4 heads of 64 over one kv head."""
    cfg = dict(id=50, layers=2, width=256, n_heads=4, head_dim=64, n_kv_heads=1, mlp_hidden=256, state_dim=32,
               rows=10, batch=1, capacity=100, steps=3, time_emb_dim=64, tau0=1.0, dt=-1.0 / 3, rms_eps=1e-6,
               rope_base=10000.0, dtype="bf16", weight_std=0.02, prefix_lens=[77])
    cfg.update(kw)
    return cfg
