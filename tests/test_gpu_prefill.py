"""Prefix prefill through the C ABI against the oracle.

The prefill is the language-model pass that reads the prefix tokens and
writes the key/value cache the action expert attends to ("FlashRT-PAI",
section 2.1, Figure 1a).  Cases:
  * small shapes (several GEMM tiles, several 64-key blocks and 128-query
    blocks, ragged lengths, head_dim 256 with one kv head and 128 with two);
  * the cache of a shorter prefix is the head of a longer one (causal mask),
    bit for bit when the cut falls on a 32-query boundary;
  * replays are bit-identical;
  * the full-width shape (width 2048, 8 x 256 over one kv head, GeGLU 16384,
    an 800-row bucket, 768 tokens) with two layers, sampled: layer 0 on every
    token, both layers on the first 64 tokens (under the causal mask the
    first tokens' cache does not depend on later ones);
  * the benchmarked shape itself (18 layers): layer 0 on every token, every
    layer on the first 64 tokens, and the first 640 tokens' cache of every
    layer bit-identical when the later tokens change;
  * prefill -> load_prefix_kv -> decide matches the oracle's prefill feeding
    the oracle's decision;
  * a prefill handle rejects decide, load_prefix_kv and out-of-range lengths.
"""
import numpy as np
import pytest

import oracle
import phx_inputs
from gpu_util import TOL_BF16, assert_close, assert_close_bf16_storage, say

pytestmark = pytest.mark.gpu


def prefill_small(**kw):
    cfg = dict(id=70, name="prefill_small", block="prefill", layers=3, width=256, n_heads=2, head_dim=256,
               n_kv_heads=1, mlp_hidden=512, state_dim=256, rows=200, batch=1, capacity=0, steps=1,
               time_emb_dim=64, tau0=1.0, dt=0.0, rms_eps=1e-6, rope_base=10000.0, dtype="bf16", weight_std=0.02,
               prefix_lens=[200])
    cfg.update(kw)
    if "state_dim" not in kw:
        cfg["state_dim"] = cfg["width"]
    return cfg


def _bf16_to_f32(t):
    """Raw bfloat16 bits (int16 tensor) -> float32 numpy."""
    u = t.cpu().numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def _gpu_prefill(cfg, inp, lengths):
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    try:
        x = torch.from_numpy(np.ascontiguousarray(inp["noise"][0])).cuda()
        out = []
        for n in lengths:
            k, v = ex.prefill(x, n)
            torch.cuda.synchronize()
            out.append((_bf16_to_f32(k), _bf16_to_f32(v)))
        return out, ex.kernels_per_decision()
    finally:
        ex.close()


def _case(cfg, lengths, seed=0, tol=TOL_BF16):
    say(f"case {cfg['name']} seed={seed} bucket={cfg['rows']} lengths={lengths} width={cfg['width']} "
        f"heads={cfg['n_heads']}x{cfg['head_dim']}/{cfg['n_kv_heads']} layers={cfg['layers']}")
    inp = phx_inputs.make_inputs(cfg, seed)
    got, nk = _gpu_prefill(cfg, inp, lengths)
    x = inp["noise"][0]
    for n, (k, v) in zip(lengths, got):
        ref = oracle.prefill(cfg, inp["weights"], x, n)
        kvd = cfg["n_kv_heads"] * cfg["head_dim"]
        assert k.shape == (cfg["layers"], n, kvd) and v.shape == k.shape
        assert_close_bf16_storage(k, ref["k"], tol, what=f"{cfg['name']} keys, {n} tokens")
        assert_close_bf16_storage(v, ref["v"], tol, what=f"{cfg['name']} values, {n} tokens")
    return inp, got, nk


def test_prefill_small():
    _, _, nk = _case(prefill_small(), [200, 137, 1])
    # per layer: 2 norms, QKV, attention (+ combine), O, gate/up, down, where a norm after a residual GEMM
    # with k splits runs inside that GEMM's reduction launch; the last layer stops after its QKV
    assert nk >= 2 * 5 + 2


def test_prefill_head_dim_128_two_kv_heads():
    _case(prefill_small(n_heads=4, head_dim=128, n_kv_heads=2, name="prefill_dh128_gqa"), [200, 77])


def test_prefill_long_bucket():
    """Six 128-query blocks and eleven 64-key blocks per head (key splits meet the causal mask)."""
    _case(prefill_small(layers=2, rows=700, width=512, name="prefill_700"), [700, 333])


def test_prefill_shorter_prefix_is_the_head_of_a_longer_one():
    cfg = prefill_small(name="prefill_heads")
    inp = phx_inputs.make_inputs(cfg, 1)
    say("case prefill_heads lengths 200, 96, 200 (replay)")
    (k2, v2), (k1, v1), (k3, v3) = _gpu_prefill(cfg, inp, [200, 96, 200])[0]
    # rows past 96 are zeros in the second call; the first 96 tokens' cache is the same, bit for bit
    assert np.array_equal(k1, k2[:, :96]) and np.array_equal(v1, v2[:, :96])
    assert np.array_equal(k2, k3) and np.array_equal(v2, v3), "replays must be bit-identical"


def test_prefill_full_width_sampled():
    """The full-width prefill shape with two layers (the kernels and their launches are per layer)."""
    cfg = phx_inputs.workload("prefix_prefill_bf16", layers=2)
    cfg["name"] = "prefill_full_width"
    n = int(cfg["prefix_lens"][0])
    say(f"case prefill_full_width bucket={cfg['rows']} tokens={n} layers=2")
    inp = phx_inputs.make_inputs(cfg, 0)
    (k, v), = _gpu_prefill(cfg, inp, [n])[0]
    x = inp["noise"][0]
    # layer 0 on every token: the cache of layer 0 is the same in a one-layer stack
    one = dict(cfg, layers=1)
    w1 = inp["weights"][:phx_inputs.weight_count(one)].copy()
    phx_inputs.view(w1, one, "G")[:] = phx_inputs.view(inp["weights"], cfg, "G")[:2]
    r0 = oracle.prefill(one, w1, x, n)
    assert_close_bf16_storage(k[:1], r0["k"], TOL_BF16, what="full width, layer 0 keys, all tokens")
    assert_close_bf16_storage(v[:1], r0["v"], TOL_BF16, what="full width, layer 0 values, all tokens")
    # both layers on the first 64 tokens
    r = oracle.prefill(cfg, inp["weights"], x, 64)
    assert_close_bf16_storage(k[:, :64], r["k"], TOL_BF16, what="full width, both layers, first 64 tokens")
    assert_close_bf16_storage(v[:, :64], r["v"], TOL_BF16, what="full width, both layers, first 64 tokens")


def test_prefill_feeds_the_expert():
    """The prefill's cache loaded into an action expert: the decision matches the oracle's prefill feeding
    the oracle's decision (the expert's K/V head is the prefill's)."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    pcfg = prefill_small(layers=2, name="prefill_pipeline")
    pin = phx_inputs.make_inputs(pcfg, 2)
    n = 150
    ecfg = dict(id=71, layers=2, width=256, n_heads=2, head_dim=256, n_kv_heads=1, mlp_hidden=256, state_dim=32,
                rows=10, batch=1, capacity=200, steps=3, time_emb_dim=64, tau0=1.0, dt=-1.0 / 3, rms_eps=1e-6,
                rope_base=10000.0, dtype="bf16", weight_std=0.02, prefix_lens=[n])
    ein = phx_inputs.make_inputs(ecfg, 2)
    say(f"case prefill_pipeline: prefill {n} tokens -> expert decision")
    pre = Expert(pcfg, pin["weights"], pin["weights_bits"])
    ex = Expert(ecfg, ein["weights"], ein["weights_bits"])
    try:
        x = torch.from_numpy(np.ascontiguousarray(pin["noise"][0])).cuda()
        k, v = pre.prefill(x, n)
        ex.load_prefix_kv(0, k, v, n)
        nz = torch.from_numpy(ein["noise"]).cuda()
        act = ex.decide(nz)
        torch.cuda.synchronize()
        act = act.cpu().numpy().copy()
    finally:
        pre.close()
        ex.close()
    ref = oracle.prefill(pcfg, pin["weights"], pin["noise"][0], n)
    kc = np.zeros((1, 2, 200, 256), dtype=np.float32)
    vc = np.zeros_like(kc)
    kc[0, :, :n] = phx_inputs.bf16_round(ref["k"].astype(np.float32))[0]
    vc[0, :, :n] = phx_inputs.bf16_round(ref["v"].astype(np.float32))[0]
    want = oracle.decide(ecfg, ein["weights"], kc, vc, np.array([n], dtype=np.int32), ein["noise"])["actions"]
    assert_close(act, want, TOL_BF16, what="prefill -> expert decision")


def test_prefill_handle_rejects_other_calls():
    import torch
    from flow_matching_action_decision_amd.binding import PhxError
    from flow_matching_action_decision_amd.expert import Expert
    cfg = prefill_small(layers=1, name="prefill_errors")
    inp = phx_inputs.make_inputs(cfg, 0)
    say("case prefill_errors")
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    try:
        x = torch.zeros((200, 256), dtype=torch.float32, device="cuda")
        k = torch.zeros((1, 200, 256), dtype=torch.int16, device="cuda")
        with pytest.raises(PhxError):
            ex.decide(torch.zeros((1, 200, 256), dtype=torch.float32, device="cuda"))
        with pytest.raises(PhxError):
            ex.load_prefix_kv(0, k, k, 10)
        with pytest.raises(PhxError):
            ex.prefill(x, 201)
        with pytest.raises(PhxError):
            ex.prefill(x, 10, k=torch.zeros((1, 10, 256), dtype=torch.int16), v=k)  # host k
        k0, v0 = ex.prefill(x, 0)  # nothing to do
        assert k0.numel() == 0 and v0.numel() == 0
        torch.cuda.synchronize()
    finally:
        ex.close()


def test_prefill_full_shape_properties():
    """The benchmarked prefill (18 layers, width 2048, 800-row bucket, 768 tokens): layer 0's cache on every
    token and every layer's cache of the first 64 tokens against the oracle, the first 640 tokens' cache of every layer unchanged, bit for bit, when the
    tokens after them change (causal mask; 640 is a multiple of the 32 queries of a wave), and every layer's
    cache finite."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    cfg = phx_inputs.workload("prefix_prefill_bf16")
    n, cut = int(cfg["prefix_lens"][0]), 640
    say(f"case prefill_full_shape: {cfg['layers']} layers, bucket {cfg['rows']}, {n} tokens, cut {cut}")
    inp = phx_inputs.make_inputs(cfg, 0)
    x0 = np.ascontiguousarray(inp["noise"][0])
    x1 = x0.copy()
    x1[cut:] = -x1[cut:] + 0.5
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    try:
        outs = []
        for xx in (x0, x1):
            k, v = ex.prefill(torch.from_numpy(xx).cuda(), n)
            torch.cuda.synchronize()
            outs.append((_bf16_to_f32(k), _bf16_to_f32(v)))
    finally:
        ex.close()
    (k0, v0), (k1, v1) = outs
    assert np.all(np.isfinite(k0)) and np.all(np.isfinite(v0))
    assert np.array_equal(k0[:, :cut], k1[:, :cut]) and np.array_equal(v0[:, :cut], v1[:, :cut])
    assert not np.array_equal(k0[1:, cut:], k1[1:, cut:]), "tokens after the change must move"
    one = dict(cfg, layers=1)
    w1 = inp["weights"][:phx_inputs.weight_count(one)].copy()
    phx_inputs.view(w1, one, "G")[:] = phx_inputs.view(inp["weights"], cfg, "G")[:2]
    r0 = oracle.prefill(one, w1, x0, n)
    assert_close_bf16_storage(k0[:1], r0["k"], TOL_BF16, what="full shape, layer 0 keys, all tokens")
    assert_close_bf16_storage(v0[:1], r0["v"], TOL_BF16, what="full shape, layer 0 values, all tokens")
    # every layer on the first 64 tokens: under the causal mask their cache is that of a 64-token prefill
    r64 = oracle.prefill(cfg, inp["weights"], x0, 64)
    assert_close_bf16_storage(k0[:, :64], r64["k"], TOL_BF16, what="full shape, all 18 layers' keys, first 64 tokens")
    assert_close_bf16_storage(v0[:, :64], r64["v"], TOL_BF16, what="full shape, all 18 layers' values, first 64 tokens")
