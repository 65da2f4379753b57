"""Large-token plan vs the oracle: the video-action chunk (decoder block, a
chunk of hundreds of rows over a prefix cache) and the DiT-style step
(adaLN-Zero block over thousands of tokens).

Element-by-element parity runs at reduced sizes that still span several
GEMM tiles, several 64-key attention blocks, attention key splits and a
ragged row tail (rows not a multiple of the 128-row padding).  At the full
workload sizes the checks are the ones that hold at any size: zero velocity
head gives back the noise bit for bit, zero gates give back the tokens bit
for bit, token permutation commutes with the DiT step, and a one-layer,
one-step slice at full width, heads, rows and cache length matches the
oracle.
"""
import numpy as np
import pytest

import oracle
import phx_inputs
from gpu_util import TOL_BF16, TOL_TOKENS, assert_close, gpu_decide, oracle_decide, say

pytestmark = pytest.mark.gpu


def va_small(**kw) -> dict:
    """Decoder block through the large-token plan: 200 rows (> 160, and not a
    multiple of 128), 2 layers, width 256, 2 heads of 128, a 250-row prefix."""
    cfg = dict(id=60, name="va_small", block="decoder", layers=2, width=256, n_heads=2, head_dim=128,
               n_kv_heads=2, mlp_hidden=512, state_dim=128, rows=200, batch=1, capacity=300, steps=2,
               time_emb_dim=64, tau0=1.0, dt=-0.5, rms_eps=1e-6, rope_base=10000.0, dtype="bf16",
               weight_std=0.02, prefix_lens=[250])
    cfg.update(kw)
    return cfg


def dit_small(**kw) -> dict:
    """DiT-style block at 300 tokens (ragged), 2 blocks, width 256, 2 heads of 128."""
    cfg = dict(id=61, name="dit_small", block="dit", layers=2, width=256, n_heads=2, head_dim=128, n_kv_heads=2,
               mlp_hidden=1024, state_dim=256, rows=300, batch=1, capacity=0, steps=1, time_emb_dim=64, tau0=1.0,
               dt=0.0, rms_eps=1e-6, rope_base=10000.0, dtype="bf16", weight_std=0.02, prefix_lens=[0])
    cfg.update(kw)
    return cfg


def _va_case(cfg, seed=0, tol=TOL_BF16):
    say(f"case {cfg['name']} seed={seed} rows={cfg['rows']} L={cfg['prefix_lens']} heads={cfg['n_heads']}/"
        f"{cfg['n_kv_heads']} layers={cfg['layers']} steps={cfg['steps']}")
    inp = phx_inputs.make_inputs(cfg, seed)
    outs, nk = gpu_decide(cfg, inp)
    ref = oracle_decide(cfg, inp)
    return assert_close(outs[0], ref, tol, what=cfg["name"]), inp, outs[0], nk


def _dit_gpu(cfg, inp, x=None, repeats=1, flags=0):
    return gpu_decide(cfg, inp, noise=inp["noise"] if x is None else x, repeats=repeats, flags=flags)


def _dit_case(cfg, seed=0, tol=TOL_TOKENS, flags=0):
    say(f"case {cfg['name']} seed={seed} tokens={cfg['rows']} width={cfg['width']} blocks={cfg['layers']} "
        f"flags={flags}")
    inp = phx_inputs.make_inputs(cfg, seed)
    outs, nk = _dit_gpu(cfg, inp, flags=flags)
    ref = oracle.dit(cfg, inp["weights"], inp["noise"][0])["out"]
    return assert_close(outs[0][0], ref, tol, what=cfg["name"]), inp, outs[0], nk


# ------------------------------------------------------------ decoder block

def test_va_small():
    _, _, _, nk = _va_case(va_small())
    # per step: convert, in-proj, 2 layers x (2 norms, 4 GEMMs, attention [+ combine]), final norm, out-proj
    assert nk >= 2 * (2 + 2 * 7 + 2)


def test_va_small_gqa():
    _va_case(va_small(n_heads=4, n_kv_heads=2, name="va_small_gqa"))


def test_va_head_dim_256():
    """Heads of 256 (MQA: two query heads over one kv head), width 512."""
    _va_case(va_small(n_heads=2, head_dim=256, n_kv_heads=1, width=512, name="va_dh256"))


def test_va_many_rows():
    """1030 rows: the GEMMs take the register-fed kernel (1024 rows or more)."""
    _va_case(va_small(rows=1030, prefix_lens=[100], name="va_1030"))


@pytest.mark.parametrize("L", [0, 1, 63, 300])
def test_va_prefix_edges(L):
    # 161 rows: the smallest chunk the large-token plan takes; 300 = the full capacity
    _va_case(va_small(rows=161, prefix_lens=[L], name=f"va_L{L}"))


def test_va_reload_and_replay_bit_identical():
    """Decide, load another prefix, decide, reload the original, decide: the
    first and last runs agree bit for bit; replays are bit-identical."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    cfg = va_small(name="va_reload")
    a = phx_inputs.make_inputs(cfg, 0)
    b = phx_inputs.make_inputs(cfg, 1)
    say("case va_reload: prefix seed 0, then 1, then 0")
    ex = Expert(cfg, a["weights"], a["weights_bits"])
    try:
        nz = torch.from_numpy(a["noise"]).cuda()
        keep = ex.load_all(a)
        r0 = ex.decide(nz).cpu().numpy().copy()
        r0b = ex.decide(nz).cpu().numpy().copy()
        keep_b = ex.load_all(b)
        r1 = ex.decide(nz).cpu().numpy().copy()
        keep = ex.load_all(a)
        r2 = ex.decide(nz).cpu().numpy().copy()
        del keep, keep_b
    finally:
        ex.close()
    assert np.array_equal(r0, r0b)
    assert np.array_equal(r0, r2)
    assert not np.array_equal(r0, r1)


def test_va_poisoned_cache_tail_is_never_read():
    cfg = va_small(name="va_poison", prefix_lens=[130])
    inp = phx_inputs.make_inputs(cfg, 0)
    clean, _ = gpu_decide(cfg, inp)
    # the loader copies only the first L rows, so poison the caller's rows past L and
    # also load a longer prefix first so the handle's rows past L hold other values
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    say("case va_poison: load 300 rows of NaN, then the real 130-row prefix")
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    try:
        nan_bits = np.full((cfg["layers"], 300, 256), 0x7FC0, dtype=np.uint16).view(np.int16)
        kt = torch.from_numpy(nan_bits).cuda()
        ex.load_prefix_kv(0, kt, kt, 300)
        keep = ex.load_all(inp)
        out = ex.decide(torch.from_numpy(inp["noise"]).cuda()).cpu().numpy()
        del keep
    finally:
        ex.close()
    assert np.array_equal(out, clean[0])


def test_va_chunk_full_zero_velocity_head_returns_noise():
    """The full video-action chunk workload (8 layers, 5 steps, 256 rows over a
    4096-row cache of capacity 8192) with W_out = 0: every Euler step adds
    dt * 0, so the actions equal the noise bit for bit."""
    cfg = phx_inputs.workload("va_chunk_bf16")
    say("case va_chunk_bf16 W_out=0 (full size)")
    inp = phx_inputs.make_inputs(cfg, 0)
    phx_inputs.view(inp["weights"], cfg, "W_out")[:] = 0
    off, shape = phx_inputs.weight_slices(cfg)["W_out"]
    inp["weights_bits"][off:off + int(np.prod(shape))] = 0
    outs, nk = gpu_decide(cfg, inp)
    say(f"  kernels per decision: {nk}")
    assert np.array_equal(outs[0], inp["noise"])


def test_va_chunk_full_width_one_layer_one_step():
    """One layer and one Euler step of the video-action chunk at full width,
    heads, rows, cache length and capacity, element by element."""
    cfg = phx_inputs.workload("va_chunk_bf16", layers=1, steps=1)
    cfg["name"] = "va_chunk_1x1"
    _va_case(cfg)


@pytest.mark.slow
@pytest.mark.timeout(400)
def test_va_chunk_full_every_layer_one_step():
    """Every layer of the video-action chunk (8 layers at full width, heads,
    rows, cache length and capacity) for one Euler step, element by element."""
    cfg = phx_inputs.workload("va_chunk_bf16", steps=1)
    cfg["name"] = "va_chunk_8x1"
    _va_case(cfg)


# ------------------------------------------------------------ DiT-style block

def test_dit_small():
    _dit_case(dit_small())


def test_dit_small_rows_multiple_of_padding():
    _dit_case(dit_small(rows=256, name="dit_256"))


def test_dit_head_dim_256():
    _dit_case(dit_small(n_heads=2, head_dim=256, n_kv_heads=2, width=512, state_dim=512, name="dit_dh256"))


def test_dit_many_rows():
    """1100 tokens (ragged): the GEMMs take the register-fed kernel."""
    _dit_case(dit_small(rows=1100, name="dit_1100"))


def test_dit_uniform_attention_closed_form():
    """W_q = 0 makes every attention row uniform, so o is the mean of the value
    rows; the oracle is pinned to that closed form, and here the GPU follows."""
    cfg = dit_small(name="dit_wq0")
    inp = phx_inputs.make_inputs(cfg, 0)
    hd = cfg["n_heads"] * cfg["head_dim"]
    off, shape = phx_inputs.weight_slices(cfg)["W_qkv.0"]
    w = inp["weights"][off:off + int(np.prod(shape))].reshape(shape)
    wb = inp["weights_bits"][off:off + int(np.prod(shape))].reshape(shape)
    w[:, :hd] = 0
    wb[:, :hd] = 0
    say("case dit_wq0")
    outs, _ = _dit_gpu(cfg, inp)
    ref = oracle.dit(cfg, inp["weights"], inp["noise"][0])["out"]
    assert_close(outs[0][0], ref, TOL_TOKENS, what="dit_wq0")


def test_dit_full_zero_gates_identity():
    """The full DiT-style step (4 blocks, 4128 tokens, width 3072) with zero
    gate rows of W_mod: every residual update is multiplied by 0, so the
    output is the input bit for bit (and every kernel ran at full size without
    producing a non-finite value, which 0 * NaN would expose)."""
    cfg = phx_inputs.workload("wam_dit_bf16")
    say("case wam_dit_bf16 zero gates (full size)")
    inp = phx_inputs.make_inputs(cfg, 0)
    D = cfg["width"]
    wm = phx_inputs.view(inp["weights"], cfg, "W_mod")
    off, shape = phx_inputs.weight_slices(cfg)["W_mod"]
    wmb = inp["weights_bits"][off:off + int(np.prod(shape))].reshape(shape)
    for g0 in (2 * D, 5 * D):
        wm[:, :, g0:g0 + D] = 0
        wmb[:, :, g0:g0 + D] = 0
    outs, nk = _dit_gpu(cfg, inp)
    say(f"  kernels per decision: {nk}")
    assert np.array_equal(outs[0], inp["noise"])


def test_dit_full_permutation_equivariance():
    """Full DiT-style step: permuting the tokens permutes the output (no
    positions, no mask).  Only the order of the attention sums changes, so
    the two runs agree to rounding."""
    cfg = phx_inputs.workload("wam_dit_bf16")
    say("case wam_dit_bf16 permutation (full size)")
    inp = phx_inputs.make_inputs(cfg, 0)
    perm = np.random.default_rng(7).permutation(cfg["rows"])
    outs, _ = _dit_gpu(cfg, inp, repeats=2)
    assert np.array_equal(outs[0], outs[1]), "replays must be bit-identical"
    outs_p, _ = _dit_gpu(cfg, inp, x=np.ascontiguousarray(inp["noise"][:, perm]))
    # Both runs carry their own bf16 rounding of the attention operands and of
    # the probabilities (rounded against a running maximum that depends on the
    # key order): the bar doubled on max-abs for the difference of two such
    # runs, and rel-L2 at half the bar.
    assert_close(outs_p[0][0], outs[0][0][perm], dict(max_abs=4e-2, rel_l2=5e-3, worst_row_cos=0.9999),
                 what="permuted")


@pytest.mark.parametrize("rows", [528, 1100])
def test_dit_full_width_one_block(rows):
    """One block at full width, heads and MLP, element by element: 528 tokens
    (four 128-row tiles and a ragged 16-row tail, LDS-ring GEMMs) and 1100
    tokens (register-fed GEMMs, ragged 76-row tail)."""
    cfg = phx_inputs.workload("wam_dit_bf16", layers=1, rows=rows)
    cfg["name"] = f"dit_1block_{rows}"
    _dit_case(cfg)


@pytest.mark.slow
@pytest.mark.timeout(400)
def test_dit_full_tokens_one_block():
    """One block of the DiT-style step at its full size (4128 tokens, width
    3072, 24 heads of 128, MLP 12288), every value against the oracle."""
    cfg = phx_inputs.workload("wam_dit_bf16", layers=1)
    cfg["name"] = "dit_1block_4128"
    _dit_case(cfg)


def test_dit_paired_activations_beat_plain_bf16():
    """The paired GEMM activations (the DiT-style block's default) against
    plain bf16 ones (PHX_FLAG_BF16_ACT), one full-width block of 528 tokens:
    both against the oracle, the paired run at the bar and closer than the
    plain run, which carries the bf16 rounding of the QKV, gate/up and down inputs."""
    from flow_matching_action_decision_amd import PHX_FLAG_BF16_ACT
    cfg = phx_inputs.workload("wam_dit_bf16", layers=1, rows=528)
    cfg["name"] = "dit_1block_528_pairing"
    inp = phx_inputs.make_inputs(cfg, 0)
    ref = oracle.dit(cfg, inp["weights"], inp["noise"][0])["out"]
    say("case dit paired vs plain bf16 GEMM activations (528 tokens, one block)")
    paired, nk_p = _dit_gpu(cfg, inp)
    plain, nk_b = _dit_gpu(cfg, inp, flags=PHX_FLAG_BF16_ACT)
    assert nk_p == nk_b
    mp = assert_close(paired[0][0], ref, TOL_TOKENS, what="paired GEMM activations")
    mb = assert_close(plain[0][0], ref, dict(max_abs=1.0, rel_l2=1e-2), what="plain bf16 GEMM activations")
    assert mp["max_abs"] < mb["max_abs"] and mp["rel_l2"] < mb["rel_l2"]


def test_dit_small_plain_bf16_act():
    """The plain-bf16 opt-out on the small DiT shape (small modulation, so the
    bf16 rounding of the MLP stays within the bar there)."""
    from flow_matching_action_decision_amd import PHX_FLAG_BF16_ACT
    _dit_case(dit_small(name="dit_small_bf16_act"), flags=PHX_FLAG_BF16_ACT)


def test_va_paired_activations():
    """The decoder plan with paired GEMM activations (opt-in): the same
    oracle bar, and the chunk's QKV, gate/up and down GEMMs at twice the k-steps."""
    from flow_matching_action_decision_amd import PHX_FLAG_PAIRED_ACT
    cfg = va_small(name="va_small_paired")
    inp = phx_inputs.make_inputs(cfg, 0)
    say("case va_small paired GEMM activations")
    outs, _ = gpu_decide(cfg, inp, flags=PHX_FLAG_PAIRED_ACT)
    assert_close(outs[0], oracle_decide(cfg, inp), TOL_BF16, what="va_small paired")


# ------------------------------------------------------------ history update

def _history_case(cfg, name, commits=1):
    """Decide, commit the decided chunk, decide the next chunk (repeat), and
    compare every decision with the oracle on the same history: the oracle
    commits the same chunk (the GPU's decided actions), appends its keys and
    values, drops the oldest rows past the window, and decides at the
    window's base position."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    say(f"case history {name} rows={cfg['rows']} C={cfg['capacity']} L={cfg['prefix_lens']} commits={commits}")
    inp = phx_inputs.make_inputs(cfg, 0)
    NL, C, M = cfg["layers"], cfg["capacity"], cfg["rows"]
    L = int(inp["lens"][0])
    k_hist = inp["kv_k"][0, :, :L].astype(np.float64)
    v_hist = inp["kv_v"][0, :, :L].astype(np.float64)
    base = 0
    tau_end = cfg["tau0"] + cfg["steps"] * cfg["dt"]
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    try:
        keep = ex.load_all(inp)
        noise = inp["noise"]
        for r in range(commits + 1):
            out = ex.decide(torch.from_numpy(noise).cuda()).cpu().numpy()
            kk = np.zeros((1, NL, C, k_hist.shape[-1]), dtype=np.float32)
            vv = np.zeros_like(kk)
            kk[0, :, :k_hist.shape[1]] = k_hist
            vv[0, :, :v_hist.shape[1]] = v_hist
            ref = oracle.decide(cfg, inp["weights"], kk, vv, [k_hist.shape[1]], noise, pos0=[base])["actions"]
            assert_close(out, ref, TOL_BF16, what=f"{name} decision {r} (history {k_hist.shape[1]}, base {base})")
            if r == commits:
                last_ref = ref
                break
            ex.commit_chunk(torch.from_numpy(out[0]).cuda())
            got = oracle.commit(cfg, inp["weights"], kk, vv, [k_hist.shape[1]], out, tau_end, pos0=[base])
            k_hist = np.concatenate([k_hist, got["k"][0]], axis=1)
            v_hist = np.concatenate([v_hist, got["v"][0]], axis=1)
            if k_hist.shape[1] > C:
                d = k_hist.shape[1] - C
                k_hist, v_hist, base = k_hist[:, d:], v_hist[:, d:], base + d
            noise = np.random.default_rng(100 + r).standard_normal(noise.shape).astype(np.float32)
        cap = ex.capsule_save()
        nz = torch.from_numpy(noise).cuda()
        first = ex.decide(nz).cpu().numpy().copy()
        ex.load_all(inp)  # overwrite the history
        ex.capsule_restore(cap)
        again = ex.decide(nz).cpu().numpy().copy()
        del keep
    finally:
        ex.close()
    assert np.array_equal(first, again), "a capsule must carry the history and its window position"
    # the restored decision is the oracle's decision on its own committed history and window base
    assert_close(again, last_ref, TOL_BF16, what=f"{name} after restore vs oracle")


def test_history_commit_grows_the_cache():
    _history_case(va_small(capacity=700, prefix_lens=[150], name="history"), "grow", commits=2)


def test_history_window_drops_oldest_rows():
    # 250 + 200 rows pass the 300-row window: the 150 oldest are dropped, then 200 more
    _history_case(va_small(capacity=300, prefix_lens=[250], name="window"), "window", commits=2)


def test_history_rejects_other_plans():
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    from flow_matching_action_decision_amd.binding import PhxError
    from gpu_util import small_cfg
    cfg = small_cfg()
    inp = phx_inputs.make_inputs(cfg, 0)
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    try:
        keep = ex.load_all(inp)
        with pytest.raises(PhxError):
            ex.commit_chunk(torch.zeros(cfg["rows"], cfg["state_dim"], device="cuda"))
        del keep
    finally:
        ex.close()
