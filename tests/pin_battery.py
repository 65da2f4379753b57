"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes a loaded oracle library (ctypes handle) and
raises AssertionError when the oracle disagrees with:
  * a library routine (numpy matmul, torch rms_norm, torch GELU, torch
    scaled-dot-product attention, complex multiplication for RoPE);
  * a closed form or invariant (time embedding at tau = 0, unit pair norms,
    RoPE relative-position property, softmax rows summing to one, uniform
    attention when queries vanish, zero velocity head, dt = 0, ...);
  * a tiny brute-force composition of torch primitives (double precision).

The same battery runs against the real oracle (must pass) and against
deliberately mutated copies of its source (each must fail at least one pin),
which shows that a plausible slip anywhere in the oracle is caught.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import phx_inputs

TIGHT = 1e-10


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol * scale:.3e}"


# ---------------------------------------------------------------- per-op pins

def pin_time_embedding(lib):
    E = 16
    e0 = oracle.time_embedding(E, 0.0, lib)
    assert np.all(e0[:8] == 0.0) and np.all(e0[8:] == 1.0), "tau=0 must give [0..0 | 1..1]"
    tau = 0.7
    e = oracle.time_embedding(E, tau, lib)
    _close(e[0], math.sin(tau), what="lowest frequency is 1")
    _close(e[8], math.cos(tau), what="cos half follows sin half")
    _close(e[:8] ** 2 + e[8:] ** 2, np.ones(8), what="unit pair norm")
    # recover the frequencies at tiny tau: geometric with ratio 10000^(-1/(E/2))
    small = 1e-7
    es = oracle.time_embedding(E, small, lib)
    w = es[:8] / small
    _close(w[1:] / w[:-1], np.full(7, 10000.0 ** (-1.0 / 8)), tol=1e-6, what="geometric frequencies")
    _close(w[0], 1.0, tol=1e-6, what="first frequency")


def pin_modulation(lib):
    g = np.random.default_rng(1)
    E, D = 32, 12
    W = g.standard_normal((E, 2 * D)).astype(np.float32)
    e = g.standard_normal(E)
    _close(oracle.modulation(e, W, lib), e @ W.astype(np.float64), what="modulation vs numpy")


def pin_matmul(lib):
    g = np.random.default_rng(2)
    x = g.standard_normal((5, 7))
    W = g.standard_normal((7, 130)).astype(np.float32)
    _close(oracle.matmul(x, W, lib), x @ W.astype(np.float64), what="matmul vs numpy")


def pin_ada_rmsnorm(lib):
    g = np.random.default_rng(3)
    M, D, eps = 4, 24, 1e-3
    h = g.standard_normal((M, D)) * 3.0
    mod = g.standard_normal(2 * D)
    ref = F.rms_norm(torch.tensor(h), (D,), weight=torch.tensor(1.0 + mod[:D]), eps=eps) + torch.tensor(mod[D:])
    _close(oracle.ada_rmsnorm(h, mod, eps, lib), ref.numpy(), what="AdaRMSNorm vs torch rms_norm")
    zero = np.zeros(2 * D)
    ref0 = F.rms_norm(torch.tensor(h), (D,), eps=eps)
    _close(oracle.ada_rmsnorm(h, zero, eps, lib), ref0.numpy(), what="zero modulation is plain RMSNorm")


def pin_rope(lib):
    g = np.random.default_rng(4)
    M, nh, Dh, base = 5, 3, 8, 10000.0
    half = Dh // 2
    x = g.standard_normal((M, nh * Dh))
    pos = np.array([0, 1, 7, 100, 12345], dtype=np.int32)
    y = oracle.rope(x, nh, Dh, pos, base, lib).reshape(M, nh, Dh)
    xr = x.reshape(M, nh, Dh)
    z = xr[..., :half] + 1j * xr[..., half:]
    theta = base ** (-2.0 * np.arange(half) / Dh)
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    _close(y[..., :half], zr.real, what="RoPE real part vs complex rotation")
    _close(y[..., half:], zr.imag, what="RoPE imaginary part vs complex rotation")
    _close(y[0], xr[0], what="RoPE is the identity at position 0")
    # relative position: <R(m) q, R(n) k> depends only on m - n
    q = g.standard_normal((1, Dh))
    k = g.standard_normal((1, Dh))
    d1 = oracle.rope(q, 1, Dh, [9], base, lib) @ oracle.rope(k, 1, Dh, [4], base, lib).T
    d2 = oracle.rope(q, 1, Dh, [25], base, lib) @ oracle.rope(k, 1, Dh, [20], base, lib).T
    _close(d1, d2, tol=1e-9, what="RoPE relative-position property")


def pin_gelu(lib):
    z = np.linspace(-6, 6, 97)
    ours = np.array([lib.orc_gelu_tanh(float(v)) for v in z])
    ref = F.gelu(torch.tensor(z), approximate="tanh").numpy()
    _close(ours, ref, what="GELU tanh vs torch")
    erf_ref = F.gelu(torch.tensor(z)).numpy()
    assert np.max(np.abs(ours - erf_ref)) < 2e-3, "tanh GELU within 2e-3 of erf GELU"


def _sdpa(q, ka, va, Kp, Vp, H, KVH, Dh):
    M = q.shape[0]
    kfull = np.concatenate([Kp.astype(np.float64), ka], axis=0) if Kp.shape[0] else ka
    vfull = np.concatenate([Vp.astype(np.float64), va], axis=0) if Vp.shape[0] else va
    T = kfull.shape[0]
    group = H // KVH
    qt = torch.tensor(q.reshape(M, H, Dh)).permute(1, 0, 2)            # [H, M, Dh]
    kt = torch.tensor(kfull.reshape(T, KVH, Dh)).permute(1, 0, 2)      # [KVH, T, Dh]
    vt = torch.tensor(vfull.reshape(T, KVH, Dh)).permute(1, 0, 2)
    kt = kt.repeat_interleave(group, dim=0).contiguous()
    vt = vt.repeat_interleave(group, dim=0).contiguous()
    o = F.scaled_dot_product_attention(qt[None], kt[None], vt[None])[0]  # [H, M, Dh]
    return o.permute(1, 0, 2).reshape(M, H * Dh).numpy()


def pin_attention(lib):
    g = np.random.default_rng(5)
    for (H, KVH, Dh) in [(2, 1, 4), (4, 2, 8), (8, 1, 16)]:
        for L in (0, 1, 3, 37):
            for M in (1, 3, 10):
                q = g.standard_normal((M, H * Dh)) * 2.0
                ka = g.standard_normal((M, KVH * Dh))
                va = g.standard_normal((M, KVH * Dh))
                Kp = g.standard_normal((L, KVH * Dh)).astype(np.float32)
                Vp = g.standard_normal((L, KVH * Dh)).astype(np.float32)
                o, dev = oracle.attention(q, ka, va, Kp, Vp, H, KVH, Dh, lib)
                _close(o, _sdpa(q, ka, va, Kp, Vp, H, KVH, Dh), tol=1e-9, what=f"attention H{H} KVH{KVH} L{L} M{M}")
                assert dev < 1e-12, "softmax rows must sum to one"
    # values identically one give outputs identically one
    H, KVH, Dh, L, M = 4, 1, 8, 11, 3
    q = g.standard_normal((M, H * Dh))
    o, _ = oracle.attention(q, g.standard_normal((M, Dh)), np.ones((M, Dh)),
                            g.standard_normal((L, Dh)).astype(np.float32), np.ones((L, Dh), np.float32), H, KVH, Dh, lib)
    _close(o, np.ones_like(o), what="V == 1 gives o == 1")
    # zero queries: uniform weights, o = mean of all value rows
    va = g.standard_normal((M, Dh))
    Vp = g.standard_normal((L, Dh)).astype(np.float32)
    o, _ = oracle.attention(np.zeros((M, H * Dh)), g.standard_normal((M, Dh)), va,
                            g.standard_normal((L, Dh)).astype(np.float32), Vp, H, KVH, Dh, lib)
    mean = np.concatenate([Vp.astype(np.float64), va]).mean(axis=0)
    _close(o, np.tile(mean, (M, H)), what="q == 0 gives the mean of the values")


# ---------------------------------------------------------- whole-decision pins

def tiny_cfg(**kw):
    cfg = dict(id=97, layers=2, width=8, n_heads=2, head_dim=4, n_kv_heads=1, mlp_hidden=8, state_dim=3,
               rows=3, batch=2, capacity=5, steps=2, time_emb_dim=8, tau0=1.0, dt=-0.5, rms_eps=1e-6,
               rope_base=10000.0, dtype="f32", weight_std=0.5, prefix_lens=[0, 5])
    cfg.update(kw)
    return cfg


def torch_decide(cfg, inp, pos0=None, capture=None):
    """Brute force: the decision composed from torch double-precision
    primitives (sin/cos, matmul, rms_norm, complex rotation, scaled dot
    product attention, tanh GELU).  pos0: base positions per request;
    capture: a dict that receives every layer's rotated keys and values of
    the rows of the last step, "k"/"v" [B][NL][M][KVH*Dh]."""
    W = inp["weights"]
    NL, D, H, Dh, KVH = cfg["layers"], cfg["width"], cfg["n_heads"], cfg["head_dim"], cfg["n_kv_heads"]
    F_, A, M, B, S, E = cfg["mlp_hidden"], cfg["state_dim"], cfg["rows"], cfg["batch"], cfg["steps"], cfg["time_emb_dim"]
    t = lambda name: torch.tensor(phx_inputs.view(W, cfg, name).astype(np.float64))
    Wmod = t("W_mod")
    x = torch.tensor(inp["noise"].astype(np.float64)).reshape(B * M, A)
    half = Dh // 2
    theta = torch.pow(torch.tensor(cfg["rope_base"], dtype=torch.float64), -2.0 * torch.arange(half, dtype=torch.float64) / Dh)
    freqs = torch.pow(torch.tensor(10000.0, dtype=torch.float64), -torch.arange(E // 2, dtype=torch.float64) / (E // 2))

    def rot(v, pos, nh):
        v = v.reshape(-1, nh, Dh)
        z = torch.complex(v[..., :half], v[..., half:])
        ang = pos[:, None, None].to(torch.float64) * theta[None, None, :]
        z = z * torch.polar(torch.ones_like(ang), ang)
        return torch.cat([z.real, z.imag], dim=-1).reshape(-1, nh * Dh)

    def norm(hh, m):
        return F.rms_norm(hh, (D,), weight=1.0 + m[:D], eps=cfg["rms_eps"]) + m[D:]

    for k in range(S):
        tau = cfg["tau0"] + k * cfg["dt"]
        e = torch.cat([torch.sin(tau * freqs), torch.cos(tau * freqs)])
        mods = [e @ Wmod[n] for n in range(2 * NL + 1)]
        h = x @ t("W_in")
        for l in range(NL):
            n1 = norm(h, mods[2 * l])
            qkv = n1 @ t(f"W_qkv.{l}")
            o_all = []
            for b in range(B):
                L = int(inp["lens"][b])
                rows = slice(b * M, (b + 1) * M)
                base = 0 if pos0 is None else int(pos0[b])
                pos = torch.arange(base + L, base + L + M)
                q = rot(qkv[rows, :H * Dh], pos, H)
                ka = rot(qkv[rows, H * Dh:(H + KVH) * Dh], pos, KVH)
                va = qkv[rows, (H + KVH) * Dh:]
                if capture is not None:
                    capture.setdefault("k", np.zeros((B, NL, M, KVH * Dh)))[b, l] = ka.numpy()
                    capture.setdefault("v", np.zeros((B, NL, M, KVH * Dh)))[b, l] = va.numpy()
                Kp = torch.tensor(inp["kv_k"][b, l, :L].astype(np.float64))
                Vp = torch.tensor(inp["kv_v"][b, l, :L].astype(np.float64))
                kf = torch.cat([Kp, ka]).reshape(L + M, KVH, Dh).permute(1, 0, 2).repeat_interleave(H // KVH, 0)
                vf = torch.cat([Vp, va]).reshape(L + M, KVH, Dh).permute(1, 0, 2).repeat_interleave(H // KVH, 0)
                qh = q.reshape(M, H, Dh).permute(1, 0, 2)
                o = F.scaled_dot_product_attention(qh[None], kf.contiguous()[None], vf.contiguous()[None])[0]
                o_all.append(o.permute(1, 0, 2).reshape(M, H * Dh))
            h = h + torch.cat(o_all) @ t(f"W_o.{l}")
            n2 = norm(h, mods[2 * l + 1])
            gu = n2 @ t(f"W_gu.{l}")
            h = h + (F.gelu(gu[:, :F_], approximate="tanh") * gu[:, F_:]) @ t(f"W_down.{l}")
        v = norm(h, mods[2 * NL]) @ t("W_out")
        x = x + cfg["dt"] * v
    return x.reshape(B, M, A).numpy()


def _run(cfg, inp, lib, **kw):
    return oracle.decide(cfg, inp["weights"], inp["kv_k"], inp["kv_v"], inp["lens"], inp["noise"], lib=lib, **kw)


def pin_decide_brute_force(lib):
    for kw in [dict(), dict(n_heads=4, n_kv_heads=2, prefix_lens=[3, 1]), dict(batch=1, prefix_lens=[5], steps=1),
               dict(rows=1, prefix_lens=[2, 0]), dict(layers=1, steps=3, dt=-1.0 / 3)]:
        cfg = tiny_cfg(**kw)
        inp = phx_inputs.make_inputs(cfg, seed=3)
        out = _run(cfg, inp, lib)
        _close(out["actions"], torch_decide(cfg, inp), tol=1e-9, what=f"decision vs torch composition {kw}")
        assert out["softmax_dev"] < 1e-12


def pin_decide_at_brute_force(lib):
    """Rows at shifted base positions (the window of a history cache)."""
    for kw in [dict(), dict(n_heads=4, n_kv_heads=2, prefix_lens=[3, 1])]:
        cfg = tiny_cfg(**kw)
        inp = phx_inputs.make_inputs(cfg, seed=5)
        pos0 = [4, 9]
        out = oracle.decide(cfg, inp["weights"], inp["kv_k"], inp["kv_v"], inp["lens"], inp["noise"], lib=lib,
                            pos0=pos0)
        _close(out["actions"], torch_decide(cfg, inp, pos0=pos0), tol=1e-9, what=f"decision at base positions {kw}")


def pin_commit_brute_force(lib):
    """Commit of a chunk: the per-layer keys (after RoPE) and values of the
    chunk rows from one pass at flow time tau, against the torch composition
    run as a one-step decision at tau that records them."""
    cfg = tiny_cfg()
    inp = phx_inputs.make_inputs(cfg, seed=6)
    x = np.random.default_rng(6).standard_normal((cfg["batch"], cfg["rows"], cfg["state_dim"])).astype(np.float32)
    tau, pos0 = 0.25, [2, 7]
    got = oracle.commit(cfg, inp["weights"], inp["kv_k"], inp["kv_v"], inp["lens"], x, tau, pos0=pos0, lib=lib)
    cap = {}
    torch_decide(dict(cfg, steps=1, tau0=tau), dict(inp, noise=x), pos0=pos0, capture=cap)
    _close(got["k"], cap["k"], tol=1e-9, what="committed keys vs torch composition")
    _close(got["v"], cap["v"], tol=1e-9, what="committed values vs torch composition")


def pin_decide_invariants(lib):
    cfg = tiny_cfg()
    inp = phx_inputs.make_inputs(cfg, seed=4)
    base = _run(cfg, inp, lib, velocity=True)
    # zero velocity head: actions are the noise, bit for bit
    w0 = inp["weights"].copy()
    phx_inputs.view(w0, cfg, "W_out")[:] = 0.0
    out = _run(cfg, dict(inp, weights=w0), lib)
    assert np.array_equal(out["actions"], inp["noise"].astype(np.float64)), "W_out == 0 must return the noise"
    # dt == 0 leaves the state unchanged
    out = _run(dict(cfg, dt=0.0), inp, lib)
    assert np.array_equal(out["actions"], inp["noise"].astype(np.float64)), "dt == 0 must return the noise"
    # one step: x1 = x0 + dt * v(x0, tau0), v reported by the same run
    one = _run(dict(cfg, steps=1), inp, lib, velocity=True)
    _close(one["actions"].reshape(-1, cfg["state_dim"]),
           inp["noise"].reshape(-1, cfg["state_dim"]) + cfg["dt"] * one["velocity"][0], what="single Euler step")
    _close(one["velocity"][0], base["velocity"][0], what="first-step velocity independent of step count")
    # zero up-projection: the MLP adds nothing, same as a zero down-projection
    wu = inp["weights"].copy()
    wd = inp["weights"].copy()
    for l in range(cfg["layers"]):
        phx_inputs.view(wu, cfg, f"W_gu.{l}")[:, cfg["mlp_hidden"]:] = 0.0
        phx_inputs.view(wd, cfg, f"W_down.{l}")[:] = 0.0
    _close(_run(cfg, dict(inp, weights=wu), lib)["actions"], _run(cfg, dict(inp, weights=wd), lib)["actions"],
           what="zero up-projection == zero down-projection")
    # poison beyond the prefix length is never read
    kp = inp["kv_k"].copy()
    vp = inp["kv_v"].copy()
    for b, L in enumerate(inp["lens"]):
        kp[b, :, L:] = np.nan
        vp[b, :, L:] = 1e30
    out = _run(cfg, dict(inp, kv_k=kp, kv_v=vp), lib)
    assert np.array_equal(out["actions"], base["actions"]), "rows past the prefix length must not matter"
    # requests are independent: request 1 alone equals request 1 in the batch
    one_cfg = dict(cfg, batch=1, prefix_lens=[int(inp["lens"][1])])
    single = dict(weights=inp["weights"], kv_k=inp["kv_k"][1:2], kv_v=inp["kv_v"][1:2], lens=inp["lens"][1:2],
                  noise=inp["noise"][1:2])
    _close(_run(one_cfg, single, lib)["actions"][0], base["actions"][1], tol=1e-12, what="batch independence")
    # swapping two requests swaps their results
    sw = dict(weights=inp["weights"], kv_k=inp["kv_k"][::-1].copy(), kv_v=inp["kv_v"][::-1].copy(),
              lens=inp["lens"][::-1].copy(), noise=inp["noise"][::-1].copy())
    _close(_run(cfg, sw, lib)["actions"][::-1], base["actions"], tol=1e-12, what="request permutation")
    # no layers: v = AdaRMS(x W_in) W_out with the final modulation
    c0 = dict(cfg, layers=0, steps=1)
    inp0 = phx_inputs.make_inputs(c0, seed=5)
    out0 = _run(c0, inp0, lib, velocity=True)
    W = inp0["weights"]
    x = inp0["noise"].reshape(-1, c0["state_dim"]).astype(np.float64)
    e = np.concatenate([np.sin(1.0 * 10000.0 ** (-np.arange(4) / 4)), np.cos(1.0 * 10000.0 ** (-np.arange(4) / 4))])
    mod = e @ phx_inputs.view(W, c0, "W_mod")[0].astype(np.float64)
    h = torch.tensor(x @ phx_inputs.view(W, c0, "W_in").astype(np.float64))
    n = (F.rms_norm(h, (c0["width"],), weight=torch.tensor(1.0 + mod[:8]), eps=c0["rms_eps"]) + torch.tensor(mod[8:])).numpy()
    _close(out0["velocity"][0], n @ phx_inputs.view(W, c0, "W_out").astype(np.float64), what="zero-layer velocity")


# ---------------------------------------------------------------- DiT-style step

def pin_ada_layernorm(lib):
    g = np.random.default_rng(11)
    h = g.standard_normal((5, 12)) * 3.0 + 1.5
    scale = g.standard_normal(12) * 0.3
    shift = g.standard_normal(12) * 0.3
    got = oracle.ada_layernorm(h, scale, shift, 1e-6, lib=lib)
    ref = F.layer_norm(torch.tensor(h), (12,), eps=1e-6).numpy() * (1.0 + scale) + shift
    _close(got, ref, what="adaptive LayerNorm vs torch layer_norm")
    # closed form: a row (1, 3) has mean 2, variance 1
    two = oracle.ada_layernorm(np.array([[1.0, 3.0]]), np.zeros(2), np.zeros(2), 0.0, lib=lib)
    _close(two, np.array([[-1.0, 1.0]]), what="LayerNorm of (1, 3)")


def tiny_dit_cfg(**kw):
    cfg = dict(id=96, block="dit", layers=2, width=8, n_heads=2, head_dim=4, n_kv_heads=2, mlp_hidden=12,
               state_dim=8, rows=5, batch=1, capacity=0, steps=1, time_emb_dim=8, tau0=1.0, dt=0.0, rms_eps=1e-6,
               rope_base=10000.0, dtype="f32", weight_std=0.5, prefix_lens=[0])
    cfg.update(kw)
    return cfg


def torch_dit(cfg, W, x):
    """Brute force: the DiT-style step composed from torch double-precision
    primitives (sin/cos, matmul, layer_norm, scaled dot product attention,
    tanh GELU)."""
    NL, D, H, Dh, F_, E = cfg["layers"], cfg["width"], cfg["n_heads"], cfg["head_dim"], cfg["mlp_hidden"], cfg["time_emb_dim"]
    T = cfg["rows"]
    t = lambda name: torch.tensor(phx_inputs.view(W, cfg, name).astype(np.float64))
    freqs = torch.pow(torch.tensor(10000.0, dtype=torch.float64), -torch.arange(E // 2, dtype=torch.float64) / (E // 2))
    tau = cfg["tau0"]
    e = torch.cat([torch.sin(tau * freqs), torch.cos(tau * freqs)])
    x = torch.tensor(np.asarray(x, dtype=np.float64).reshape(T, D))
    Wmod = t("W_mod")
    for b in range(NL):
        m = e @ Wmod[b]
        sh_a, sc_a, g_a, sh_m, sc_m, g_m = [m[i * D:(i + 1) * D] for i in range(6)]
        n = F.layer_norm(x, (D,), eps=cfg["rms_eps"]) * (1 + sc_a) + sh_a
        qkv = n @ t(f"W_qkv.{b}")
        q, k, v = [qkv[:, i * H * Dh:(i + 1) * H * Dh].reshape(T, H, Dh).permute(1, 0, 2).contiguous() for i in range(3)]
        o = F.scaled_dot_product_attention(q[None], k[None], v[None])[0].permute(1, 0, 2).reshape(T, H * Dh)
        x = x + g_a * (o @ t(f"W_o.{b}"))
        n = F.layer_norm(x, (D,), eps=cfg["rms_eps"]) * (1 + sc_m) + sh_m
        x = x + g_m * (F.gelu(n @ t(f"W_up.{b}"), approximate="tanh") @ t(f"W_down.{b}"))
    return x.numpy()


def _dit(cfg, W, x, lib):
    return oracle.dit(cfg, W, x, lib=lib)["out"]


def pin_dit_brute_force(lib):
    for kw in [dict(), dict(rows=1), dict(n_heads=4, head_dim=2, n_kv_heads=4), dict(layers=1, rows=7)]:
        cfg = tiny_dit_cfg(**kw)
        inp = phx_inputs.make_inputs(cfg, seed=6)
        x = inp["noise"].reshape(cfg["rows"], cfg["width"])
        r = oracle.dit(cfg, inp["weights"], x, lib=lib)
        _close(r["out"], torch_dit(cfg, inp["weights"], x), tol=1e-9, what=f"DiT step vs torch composition {kw}")
        assert r["softmax_dev"] < 1e-12


def pin_dit_invariants(lib):
    cfg = tiny_dit_cfg()
    D, T = cfg["width"], cfg["rows"]
    inp = phx_inputs.make_inputs(cfg, seed=7)
    W = inp["weights"]
    x = inp["noise"].reshape(T, D)
    xd = x.astype(np.float64)
    base = _dit(cfg, W, x, lib)
    assert not np.allclose(base, xd), "the random step must change its input"
    # zero gates: both residual branches vanish, the step is the identity, bit for bit
    wg = W.copy()
    wm = phx_inputs.view(wg, cfg, "W_mod")
    wm[:, :, 2 * D:3 * D] = 0.0
    wm[:, :, 5 * D:6 * D] = 0.0
    assert np.array_equal(_dit(cfg, wg, x, lib), xd), "zero gates must give the identity"
    # zero output projections of both branches: the identity as well
    wz = W.copy()
    for b in range(cfg["layers"]):
        phx_inputs.view(wz, cfg, f"W_o.{b}")[:] = 0.0
        phx_inputs.view(wz, cfg, f"W_down.{b}")[:] = 0.0
    assert np.array_equal(_dit(cfg, wz, x, lib), xd), "zero branch outputs must give the identity"
    # no positions and no mask: permuting the tokens permutes the result
    perm = np.array([3, 0, 4, 1, 2])
    _close(_dit(cfg, W, x[perm], lib), base[perm], tol=1e-12, what="token permutation equivariance")
    # one block, MLP off, zero queries: every token attends uniformly, so the
    # attention branch adds gate_a * (mean over tokens of v) . W_o to every row
    c1 = dict(cfg, layers=1)
    in1 = phx_inputs.make_inputs(c1, seed=8)
    W1 = in1["weights"].copy()
    phx_inputs.view(W1, c1, "W_qkv.0")[:, :D] = 0.0
    phx_inputs.view(W1, c1, "W_down.0")[:] = 0.0
    x1 = in1["noise"].reshape(T, D)
    E = c1["time_emb_dim"]
    e = oracle.time_embedding(E, c1["tau0"], lib=lib)
    m = e @ phx_inputs.view(W1, c1, "W_mod")[0].astype(np.float64)
    n = oracle.ada_layernorm(x1.astype(np.float64), m[D:2 * D], m[:D], c1["rms_eps"], lib=lib)
    v = n @ phx_inputs.view(W1, c1, "W_qkv.0")[:, 2 * D:].astype(np.float64)
    want = x1 + m[2 * D:3 * D] * (v.mean(axis=0) @ phx_inputs.view(W1, c1, "W_o.0").astype(np.float64))
    _close(_dit(c1, W1, x1, lib), want, what="uniform attention closed form")
    # a single token attends only to itself: attention returns its own v
    c2 = dict(c1, rows=1)
    x2 = x1[:1]
    n2 = n[:1]
    v2 = n2 @ phx_inputs.view(W1, c2, "W_qkv.0")[:, 2 * D:].astype(np.float64)
    W2 = in1["weights"].copy()
    phx_inputs.view(W2, c2, "W_down.0")[:] = 0.0
    want2 = x2 + m[2 * D:3 * D] * (v2 @ phx_inputs.view(W2, c2, "W_o.0").astype(np.float64))
    _close(_dit(c2, W2, x2, lib), want2, what="single-token attention is the identity on v")


# ---------------------------------------------------------------- prefix prefill

def tiny_prefill_cfg(**kw):
    cfg = dict(id=95, block="prefill", layers=3, width=16, n_heads=4, head_dim=8, n_kv_heads=2, mlp_hidden=12,
               state_dim=16, rows=7, batch=1, capacity=0, steps=1, time_emb_dim=2, tau0=0.0, dt=0.0, rms_eps=1e-6,
               rope_base=10000.0, dtype="f32", weight_std=0.3, prefix_lens=[7])
    cfg.update(kw)
    return cfg


def torch_prefill(cfg, W, x, T):
    """Brute force: the causal prefill composed from torch double-precision
    primitives (rms_norm, matmul, rotate-half RoPE from cos/sin, scaled dot
    product attention with is_causal and the kv heads repeated, tanh GELU).
    Returns (keys, values) [NL][T][KVH*Dh]."""
    NL, D, H, Dh, KVH, F_ = (cfg["layers"], cfg["width"], cfg["n_heads"], cfg["head_dim"], cfg["n_kv_heads"],
                             cfg["mlp_hidden"])
    t = lambda name: torch.tensor(phx_inputs.view(W, cfg, name).astype(np.float64))
    G = t("G")
    x = torch.tensor(np.asarray(x, dtype=np.float64).reshape(-1, D)[:T])
    half = Dh // 2
    theta = torch.pow(torch.tensor(cfg["rope_base"], dtype=torch.float64), -2.0 * torch.arange(half, dtype=torch.float64) / Dh)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * theta[None, :]
    cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]

    def rope(y):  # y [T][nh][Dh]
        a, b = y[..., :half], y[..., half:]
        return torch.cat([a * cos - b * sin, b * cos + a * sin], dim=-1)

    ks, vs = [], []
    for l in range(NL):
        n = F.rms_norm(x, (D,), eps=cfg["rms_eps"]) * (1 + G[2 * l])
        qkv = n @ t(f"W_qkv.{l}")
        q = rope(qkv[:, :H * Dh].reshape(T, H, Dh))
        k = rope(qkv[:, H * Dh:(H + KVH) * Dh].reshape(T, KVH, Dh))
        v = qkv[:, (H + KVH) * Dh:].reshape(T, KVH, Dh)
        ks.append(k.reshape(T, KVH * Dh).numpy().copy())
        vs.append(v.reshape(T, KVH * Dh).numpy().copy())
        if l + 1 == NL:
            break
        rep = H // KVH
        kk = k.repeat_interleave(rep, dim=1).permute(1, 0, 2).contiguous()
        vv = v.repeat_interleave(rep, dim=1).permute(1, 0, 2).contiguous()
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], kk[None], vv[None], is_causal=True)[0]
        x = x + o.permute(1, 0, 2).reshape(T, H * Dh) @ t(f"W_o.{l}")
        n = F.rms_norm(x, (D,), eps=cfg["rms_eps"]) * (1 + G[2 * l + 1])
        gu = n @ t(f"W_gu.{l}")
        x = x + (F.gelu(gu[:, :F_], approximate="tanh") * gu[:, F_:]) @ t(f"W_down.{l}")
    return np.stack(ks), np.stack(vs)


def pin_prefill_brute_force(lib):
    for kw in [dict(), dict(rows=1, prefix_lens=[1]), dict(n_kv_heads=1, layers=2), dict(n_kv_heads=4, rows=5)]:
        cfg = tiny_prefill_cfg(**kw)
        inp = phx_inputs.make_inputs(cfg, seed=9)
        x = inp["noise"].reshape(cfg["rows"], cfg["width"])
        for T in sorted({cfg["rows"], max(1, cfg["rows"] - 2)}):
            r = oracle.prefill(cfg, inp["weights"], x, T, lib=lib)
            k, v = torch_prefill(cfg, inp["weights"], x, T)
            _close(r["k"], k, tol=1e-9, what=f"prefill keys vs torch composition {kw} T={T}")
            _close(r["v"], v, tol=1e-9, what=f"prefill values vs torch composition {kw} T={T}")
            assert r["softmax_dev"] < 1e-12


def pin_prefill_incremental(lib):
    """One causal pass over T tokens equals decoding them one at a time with a
    key/value cache: token t's keys and values, in every layer, are what a
    one-row commit of the expert's layer stack produces over the t cached
    rows, when the expert's in-projection is the identity and its modulation
    at flow time 0 is the prefill's gains (with E = 2 the sinusoid at tau = 0
    is exactly [0, 1], so the modulation is row 1 of W_mod)."""
    cfg = tiny_prefill_cfg(layers=2)
    inp = phx_inputs.make_inputs(cfg, seed=10)
    D, NL, T = cfg["width"], cfg["layers"], cfg["rows"]
    x = inp["noise"].reshape(T, D)
    ref = oracle.prefill(cfg, inp["weights"], x, T, lib=lib)
    ecfg = dict(cfg, block="decoder", state_dim=D, rows=1, capacity=T, time_emb_dim=2, steps=1)
    we = np.zeros(phx_inputs.weight_count(ecfg), dtype=np.float32)
    phx_inputs.view(we, ecfg, "W_in")[:] = np.eye(D, dtype=np.float32)
    for l in range(NL):
        for name in ("W_qkv", "W_o", "W_gu", "W_down"):
            phx_inputs.view(we, ecfg, f"{name}.{l}")[:] = phx_inputs.view(inp["weights"], cfg, f"{name}.{l}")
    wm = phx_inputs.view(we, ecfg, "W_mod")
    wm[:2 * NL, 1, :D] = phx_inputs.view(inp["weights"], cfg, "G")
    kvd = cfg["n_kv_heads"] * cfg["head_dim"]
    kc = np.zeros((1, NL, T, kvd), dtype=np.float32)
    vc = np.zeros((1, NL, T, kvd), dtype=np.float32)
    kc[0] = ref["k"].astype(np.float32)
    vc[0] = ref["v"].astype(np.float32)
    for t in range(T):
        got = oracle.commit(ecfg, we, kc, vc, np.array([t], dtype=np.int32), x[t].reshape(1, 1, D), 0.0,
                            pos0=[0], lib=lib)
        _close(got["k"][0, :, 0], ref["k"][:, t], tol=1e-6, what=f"prefill keys of token {t} vs one-row commit")
        _close(got["v"][0, :, 0], ref["v"][:, t], tol=1e-6, what=f"prefill values of token {t} vs one-row commit")


def pin_prefill_invariants(lib):
    cfg = tiny_prefill_cfg()
    inp = phx_inputs.make_inputs(cfg, seed=11)
    D, NL, T, H, Dh, KVH = (cfg["width"], cfg["layers"], cfg["rows"], cfg["n_heads"], cfg["head_dim"],
                            cfg["n_kv_heads"])
    W = inp["weights"]
    x = inp["noise"].reshape(T, D)
    base = oracle.prefill(cfg, W, x, T, lib=lib)
    # causal: changing token j leaves every earlier token's keys and values unchanged, bit for bit
    j = 4
    xp = x.copy()
    xp[j:] = -xp[j:] + 1.0
    pert = oracle.prefill(cfg, W, xp, T, lib=lib)
    assert np.array_equal(pert["k"][:, :j], base["k"][:, :j]) and np.array_equal(pert["v"][:, :j], base["v"][:, :j]), \
        "tokens before a change must keep their cache"
    assert not np.allclose(pert["k"][1:, j:], base["k"][1:, j:]), "tokens from the change on must move"
    # a shorter prefill is the head of a longer one, bit for bit
    short = oracle.prefill(cfg, W, x, 3, lib=lib)
    assert np.array_equal(short["k"], base["k"][:, :3]) and np.array_equal(short["v"], base["v"][:, :3])
    # zero residual branches: the stream stays x, so layer l's cache is the projection of
    # RMSNorm(x) * (1 + G[2l]) with rotate-half RoPE at positions 0..T-1 on the keys
    wz = W.copy()
    for l in range(NL):
        phx_inputs.view(wz, cfg, f"W_o.{l}")[:] = 0.0
        phx_inputs.view(wz, cfg, f"W_down.{l}")[:] = 0.0
    z = oracle.prefill(cfg, wz, x, T, lib=lib)
    xd = x.astype(np.float64)
    rms = np.sqrt(np.mean(xd * xd, axis=1, keepdims=True) + cfg["rms_eps"])
    G = phx_inputs.view(wz, cfg, "G").astype(np.float64)
    half = Dh // 2
    for l in range(NL):
        n = xd / rms * (1.0 + G[2 * l])
        Wq = phx_inputs.view(wz, cfg, f"W_qkv.{l}").astype(np.float64)
        k = (n @ Wq[:, H * Dh:(H + KVH) * Dh]).reshape(T, KVH, Dh)
        v = n @ Wq[:, (H + KVH) * Dh:]
        # RoPE as a complex rotation of (k_j + i k_{j+half}) by angle p * base^(-2j/Dh)
        zc = (k[..., :half] + 1j * k[..., half:]) * np.exp(
            1j * np.arange(T)[:, None, None] * cfg["rope_base"] ** (-2.0 * np.arange(half) / Dh))
        kr = np.concatenate([zc.real, zc.imag], axis=-1).reshape(T, KVH * Dh)
        _close(z["k"][l], kr, tol=1e-12, what=f"zero-branch keys, layer {l}")
        _close(z["v"][l], v, tol=1e-12, what=f"zero-branch values, layer {l}")
    # the first token attends only to itself: with one layer of queries zeroed the result is unchanged
    wq = W.copy()
    phx_inputs.view(wq, cfg, "W_qkv.0")[:, :H * Dh] = 0.0
    one = oracle.prefill(cfg, wq, x, 1, lib=lib)
    ref1 = oracle.prefill(cfg, W, x, 1, lib=lib)
    _close(one["k"], ref1["k"], tol=1e-12, what="a single token's cache does not depend on its queries")


# ---------------------------------------------------------------- 8-bit weight tier

def pin_quantize_i8(lib):
    """Round-to-nearest int8 codes per output channel: the column maximum
    maps to +-127, every weight is within half a step of s*q, ties go to the
    even code, a zero column gives zeros, signs and column order carry
    through, codes are monotone within a column."""
    rng = np.random.default_rng(12)
    K, N = 64, 24
    W = phx_inputs.bf16_round((rng.standard_normal((K, N)) * 0.02).astype(np.float32))[0].reshape(K, N)
    W[:, 5] = 0.0                                   # zero column
    W[:, 6] = 0.0
    W[3, 6] = -0.75                                 # a single (negative) weight
    # a column with step exactly 2^-10 (its maximum is 127 * 2^-10) and weights on half steps
    step = 2.0 ** -10
    W[:, 7] = 0.0
    W[0, 7] = 127 * step
    halves = np.array([0.5, 1.5, 2.5, 3.5, 4.5, -0.5, -1.5, -2.5, -3.5, 126.5, -126.5], dtype=np.float64)
    W[1:1 + halves.size, 7] = (halves * step).astype(np.float32)
    q, sc = oracle.quantize_i8(W, lib=lib)
    assert q.dtype == np.int8 and sc.dtype == np.float32
    assert int(np.max(np.abs(q.astype(np.int32)))) <= 127
    for n in range(N):
        col = W[:, n].astype(np.float64)
        m = float(np.max(np.abs(col)))
        if m == 0.0:
            assert sc[n] == 0.0 and not np.any(q[:, n]), "a zero column has zero scale and codes"
            continue
        assert abs(float(sc[n]) * 127.0 - m) <= 1e-6 * m, f"column {n}: scale is not max/127"
        k = int(np.argmax(np.abs(col)))
        assert int(q[k, n]) == (127 if col[k] > 0 else -127), f"column {n}: its maximum must map to +-127"
        # nearest code of the float32 quotient, which is within 127 * 2^-24 of a step of the exact one
        err = np.abs(col - float(sc[n]) * q[:, n].astype(np.float64))
        assert float(np.max(err)) <= (0.5 + 1e-5) * float(sc[n]), f"column {n}: not rounded to nearest"
        order = np.argsort(col, kind="stable")
        assert np.all(np.diff(q[order, n].astype(np.int32)) >= 0), f"column {n}: codes not monotone"
    assert sc[7] == np.float32(step)
    want = np.array([0, 2, 2, 4, 4, 0, -2, -2, -4, 126, -126])
    assert np.array_equal(q[1:1 + halves.size, 7].astype(np.int32), want), "ties must go to the even code"
    assert int(q[3, 6]) == -127 and np.count_nonzero(q[:, 6]) == 1
    # signs and column order carry through
    qn, sn = oracle.quantize_i8(-W, lib=lib)
    assert np.array_equal(qn, -q) and np.array_equal(sn, sc)
    perm = rng.permutation(N)
    qp, sp = oracle.quantize_i8(np.ascontiguousarray(W[:, perm]), lib=lib)
    assert np.array_equal(qp, q[:, perm]) and np.array_equal(sp, sc[perm])


def pin_w8_weights(lib):
    """The 8-bit tier's blob: exactly the four layer matrices change, each to
    s * q within half a quantisation step; everything else is untouched."""
    cfg = tiny_cfg()
    inp = phx_inputs.make_inputs(cfg, seed=13)
    sl = phx_inputs.weight_slices(cfg)
    w8 = oracle.w8_weights(cfg, inp["weights"], sl, lib=lib)
    for nm, (off, shape) in sl.items():
        n = int(np.prod(shape))
        a, b = inp["weights"][off:off + n].reshape(shape), w8[off:off + n].reshape(shape)
        if nm.split(".")[0] in oracle.W8_MATRICES:
            step = np.max(np.abs(a.astype(np.float64)), axis=0) / 127.0
            assert np.all(np.abs(b - a.astype(np.float64)) <= 0.5 * step[None, :] * (1 + 1e-5) + 1e-12), nm
            assert not np.array_equal(a, b), f"{nm}: not quantised"
        else:
            assert np.array_equal(a, b), f"{nm} must not change"


ALL_PINS = [pin_time_embedding, pin_modulation, pin_matmul, pin_ada_rmsnorm, pin_rope, pin_gelu, pin_attention,
            pin_decide_brute_force, pin_decide_invariants, pin_ada_layernorm, pin_dit_brute_force, pin_dit_invariants,
            pin_decide_at_brute_force, pin_commit_brute_force, pin_prefill_brute_force, pin_prefill_incremental,
            pin_prefill_invariants, pin_quantize_i8, pin_w8_weights]


def run_all(lib):
    """Run every pin; return the names of the pins that failed."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
        except (ValueError, FloatingPointError, RuntimeError):
            failed.append(pin.__name__)
    return failed
