"""HIP path vs the oracle, element by element, on the same seeded inputs.

Every test here calls the library through its C ABI (ctypes binding) on
cuda:0.  Sizes range from small shapes that still span several tiles, key
chunks and a ragged tail, to the full pi0.5-shape and rollout workloads.
"""
import numpy as np
import pytest

import phx_inputs
from gpu_util import TOL_BF16, TOL_F32, assert_close, compare, gpu_decide, oracle_decide, say, small_cfg

pytestmark = pytest.mark.gpu


def _case(cfg, seed=0, tol=None):
    say(f"case {cfg.get('name', 'custom')} seed={seed} dtype={cfg['dtype']} L={cfg.get('prefix_lens')}")
    inp = phx_inputs.make_inputs(cfg, seed)
    outs, _ = gpu_decide(cfg, inp)
    ref = oracle_decide(cfg, inp)
    tol = tol or (TOL_BF16 if cfg["dtype"] == "bf16" else TOL_F32)
    return assert_close(outs[0], ref, tol, what=f"{cfg.get('name', 'small')}"), inp, outs[0]


def test_small_bf16():
    _case(small_cfg())


def test_small_f32():
    _case(small_cfg(dtype="f32"))


@pytest.mark.parametrize("heads", [(4, 2, 128), (2, 2, 64), (8, 1, 256)], ids=["gqa", "mha", "mqa256"])
def test_head_layouts(heads):
    H, KVH, Dh = heads
    _case(small_cfg(n_heads=H, n_kv_heads=KVH, head_dim=Dh, width=256 if H * Dh <= 512 else 512))


@pytest.mark.parametrize("L", [0, 1, 54, 55, 100])
def test_prefix_length_edges(L):
    # 54 + 10 action rows end exactly on a 64-key chunk; 55 spills one key
    _case(small_cfg(prefix_lens=[L]))


def test_ragged_batch():
    _case(small_cfg(batch=4, prefix_lens=[0, 17, 100, 54]))


@pytest.mark.parametrize("shape", [(4, 1, 64, 256), (4, 2, 128, 256), (8, 1, 256, 512)],
                         ids=["mqa64", "gqa128", "mqa256"])
def test_batched_plan(shape):
    """8 requests x 10 rows (80 rows, bf16): the batched plan (large-token
    GEMMs over all rows, per-request caches, batched attention), ragged
    prefixes.  Kernel count identifies the plan: per step the input
    projection, per layer 8 launches, the final norm and velocity projection;
    a norm that follows a residual GEMM with k splits runs inside that GEMM's
    reduction launch, so per layer 6 to 8 nodes."""
    H, KVH, Dh, D = shape
    cfg = small_cfg(batch=8, prefix_lens=[0, 17, 100, 54, 64, 1, 99, 33], n_heads=H, n_kv_heads=KVH, head_dim=Dh,
                    width=D)
    m, inp, out = _case(cfg)
    _, nk = gpu_decide(cfg, inp)
    L, S = cfg["layers"], cfg["steps"]
    assert nk % S == 0 and S * (3 + 6 * L) <= nk <= S * (3 + 8 * L)


def test_ragged_batch_f32():
    _case(small_cfg(batch=3, prefix_lens=[100, 3, 64], dtype="f32"))


def test_single_layer_fp32_workload():
    cfg = phx_inputs.workload("single_layer_fp32")
    _case(cfg)


def test_pi05_expert_bf16_workload():
    """The full pi0.5-shape decision (18 layers, 10 steps, 768-token prefix),
    in the launch configuration the benchmark times."""
    cfg = phx_inputs.workload("pi05_expert_bf16")
    m, inp, first = _case(cfg)
    outs, nk = gpu_decide(cfg, inp, repeats=3)
    for o in outs:
        assert np.array_equal(o, outs[0]), "replays must be bit-identical"
    say(f"  kernels per decision: {nk}")
    assert nk == 2, "the pi0.5 shape runs as one persistent decision kernel plus its tag advance"


def test_pi05_expert_bf16_multi_kernel_path():
    """The same workload through the multi-kernel graph (forced by flag)."""
    from flow_matching_action_decision_amd import PHX_FLAG_MULTI_KERNEL
    cfg = phx_inputs.workload("pi05_expert_bf16")
    inp = phx_inputs.make_inputs(cfg, 0)
    outs, nk = gpu_decide(cfg, inp, flags=PHX_FLAG_MULTI_KERNEL)
    assert nk == cfg["steps"] * (2 + 6 * cfg["layers"])
    assert_close(outs[0], oracle_decide(cfg, inp), TOL_BF16, what="pi05 multi-kernel")


@pytest.mark.slow
@pytest.mark.timeout(400)
def test_rollout_b16_every_request():
    """The full rollout batch (16 requests, ragged prefixes drawn from {512,
    640, 768, 800}) in the launch configuration the benchmark times; every
    request's actions against the oracle's decision of the same batch."""
    cfg = phx_inputs.workload("rollout_b16_bf16")
    inp = phx_inputs.make_inputs(cfg, 0)
    say(f"case rollout_b16 lens={list(inp['lens'])}")
    outs, _ = gpu_decide(cfg, inp)
    ref = oracle_decide(cfg, inp)
    for r in range(cfg["batch"]):
        assert_close(outs[0][r:r + 1], ref[r:r + 1], TOL_BF16, what=f"request {r} (L={inp['lens'][r]})")
    assert_close(outs[0], ref, TOL_BF16, what="whole batch")


def test_zero_velocity_head_is_bit_exact():
    cfg = small_cfg()
    inp = phx_inputs.make_inputs(cfg, 1)
    w = inp["weights"].copy()
    phx_inputs.view(w, cfg, "W_out")[:] = 0.0
    bits = phx_inputs.bf16_round(w)[1]
    outs, _ = gpu_decide(cfg, dict(inp, weights=w, weights_bits=bits))
    assert np.array_equal(outs[0], inp["noise"]), "W_out == 0 must return the noise bit for bit"


def test_graph_replay_matches_direct_launches():
    from flow_matching_action_decision_amd import PHX_FLAG_NO_GRAPH
    cfg = small_cfg(batch=2, prefix_lens=[77, 12])
    inp = phx_inputs.make_inputs(cfg, 2)
    g, _ = gpu_decide(cfg, inp, repeats=2)
    d, _ = gpu_decide(cfg, inp, flags=PHX_FLAG_NO_GRAPH)
    assert np.array_equal(g[0], g[1])
    assert np.array_equal(g[0], d[0])


def test_restore_is_bit_exact():
    """decide -> overwrite the context -> decide -> reload the original -> decide:
    the first and last actions agree bit for bit."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    cfg = small_cfg(batch=2, prefix_lens=[77, 40])
    a = phx_inputs.make_inputs(cfg, 3)
    b = phx_inputs.make_inputs(cfg, 4)
    ex = Expert(cfg, a["weights"], a["weights_bits"])
    try:
        keep = ex.load_all(a)
        nz = torch.from_numpy(a["noise"]).cuda()
        first = ex.decide(nz).cpu().numpy()
        keep2 = ex.load_all(dict(b, weights=a["weights"]))
        other = ex.decide(nz).cpu().numpy()
        keep3 = ex.load_all(a)
        again = ex.decide(nz).cpu().numpy()
        del keep, keep2, keep3
    finally:
        ex.close()
    assert not np.array_equal(first, other)
    assert np.array_equal(first, again)


def test_shorter_reload_ignores_stale_rows():
    """A request reloaded with a shorter prefix gives the same bits as a fresh
    handle loaded only with the shorter prefix."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    cfg = small_cfg(prefix_lens=[100])
    inp = phx_inputs.make_inputs(cfg, 5)
    short = dict(inp, lens=np.array([30], np.int32))
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    try:
        keep = ex.load_all(inp)
        keep2 = ex.load_all(short)
        nz = torch.from_numpy(inp["noise"]).cuda()
        reused = ex.decide(nz).cpu().numpy()
        del keep, keep2
    finally:
        ex.close()
    fresh, _ = gpu_decide(cfg, short)
    assert np.array_equal(reused, fresh[0])


def test_batch_request_matches_single_request():
    cfg = small_cfg(batch=4, prefix_lens=[0, 17, 100, 54])
    inp = phx_inputs.make_inputs(cfg, 6)
    outs, _ = gpu_decide(cfg, inp)
    for r in range(4):
        one = dict(cfg, batch=1, prefix_lens=[int(inp["lens"][r])])
        sub = dict(inp, kv_k=inp["kv_k"][r:r + 1], kv_v=inp["kv_v"][r:r + 1], kv_k_bits=inp["kv_k_bits"][r:r + 1],
                   kv_v_bits=inp["kv_v_bits"][r:r + 1], lens=inp["lens"][r:r + 1], noise=inp["noise"][r:r + 1])
        single, _ = gpu_decide(one, sub)
        m = compare(outs[0][r], single[0][0])
        say(f"  request {r}: batch vs single max_abs={m['max_abs']:.3e}")
        assert m["max_abs"] <= 1e-5


def test_error_paths_on_gpu():
    import torch
    import flow_matching_action_decision_amd as p
    from flow_matching_action_decision_amd.expert import Expert
    cfg = small_cfg(batch=2, prefix_lens=[10, 10])
    inp = phx_inputs.make_inputs(cfg, 7)
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    try:
        nz = torch.from_numpy(inp["noise"]).cuda()
        with pytest.raises(p.PhxError) as e:
            ex.decide(nz)
        assert e.value.code == -4
        k = torch.zeros((cfg["layers"], 101, 64), dtype=torch.int16, device="cuda")
        with pytest.raises(p.PhxError) as e:
            ex.load_prefix_kv(0, k, k, 101)
        assert e.value.code == -3
        with pytest.raises(p.PhxError) as e:
            ex.load_prefix_kv(2, k, k, 10)
        assert e.value.code == -3
        ex.load_prefix_kv(0, k, k, 10)
        with pytest.raises(p.PhxError) as e:
            ex.decide(nz)  # request 1 still has no prefix
        assert e.value.code == -4
    finally:
        ex.close()
    c = p.make_config(cfg)
    with pytest.raises(p.PhxError) as e:
        p.phx_expert_create(c, 0, 0, 0)
    assert e.value.code == -1


@pytest.mark.parametrize("plan", ["graph", "batched", "persistent"])
def test_nan_prefix_tail_is_never_read(plan):
    """Each request is first loaded with a full-capacity prefix of NaN and then
    with its real, shorter prefix.  The decision must give the same bits as a
    fresh handle loaded only with the real prefixes, and be finite: no key or
    value row at or past a request's length may reach the result (masked
    probabilities are zero, and 0 * NaN would still be NaN)."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    if plan == "graph":
        cfg = small_cfg(name="nan_tail_graph", prefix_lens=[45])
    elif plan == "batched":
        cfg = small_cfg(name="nan_tail_batched", batch=8, prefix_lens=[0, 17, 100, 54, 64, 1, 99, 33])
    else:
        cfg = phx_inputs.workload("pi05_expert_bf16", prefix_lens=[500])
    say(f"case {cfg['name']}: NaN prefixes of {cfg['capacity']} rows, then L={cfg['prefix_lens']}")
    inp = phx_inputs.make_inputs(cfg, 7)
    C, kvd = cfg["capacity"], cfg["n_kv_heads"] * cfg["head_dim"]
    nan_bits = np.full((cfg["layers"], C, kvd), 0x7FC0, dtype=np.uint16).view(np.int16)
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    try:
        nk = torch.from_numpy(nan_bits).cuda()
        for b in range(cfg["batch"]):
            ex.load_prefix_kv(b, nk, nk, C)
        keep = ex.load_all(inp)
        nz = torch.from_numpy(inp["noise"]).cuda()
        reloaded = ex.decide(nz).cpu().numpy()
        del keep, nk
    finally:
        ex.close()
    fresh, _ = gpu_decide(cfg, inp)
    assert np.all(np.isfinite(reloaded))
    assert np.array_equal(reloaded, fresh[0])
