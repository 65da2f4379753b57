"""The persistent decision kernel (pi0.5 widths, one request) against the
oracle, element by element on the same seeded inputs.

The persistent path applies to width 1024, 8 query heads of 256 over one
key/value head, GeGLU hidden 4096, action dim 32, bf16, one request of up to
16 rows.  These cases keep those widths and vary what the kernel's indexing
depends on: layers, steps, rows, prefix length (64-key chunk edges, empty
prefix, full capacity) and capacity.
"""
import numpy as np
import pytest

import phx_inputs
from gpu_util import TOL_BF16, assert_close, compare, gpu_decide, oracle_decide, say

pytestmark = pytest.mark.gpu


def pcfg(**kw):
    cfg = phx_inputs.workload("pi05_expert_bf16", id=60, layers=2, steps=2, dt=-0.5, prefix_lens=[768])
    cfg.update(kw)
    return cfg


def _run(cfg, seed=0, flags=0, repeats=1):
    say(f"case persistent layers={cfg['layers']} steps={cfg['steps']} rows={cfg['rows']} "
        f"C={cfg['capacity']} L={cfg['prefix_lens']} seed={seed}")
    inp = phx_inputs.make_inputs(cfg, seed)
    outs, nk = gpu_decide(cfg, inp, flags=flags, repeats=repeats)
    return inp, outs, nk


def test_uses_the_persistent_kernel():
    cfg = pcfg()
    inp, outs, nk = _run(cfg)
    assert nk == 2, "the pi0.5 shape must run as one decision kernel plus its tag advance"
    assert_close(outs[0], oracle_decide(cfg, inp), TOL_BF16, what="2 layers x 2 steps, L=768")


@pytest.mark.parametrize("L", [0, 1, 63, 64, 65, 700, 767])
def test_prefix_length_edges(L):
    cfg = pcfg(layers=1, steps=1, dt=-0.1, prefix_lens=[L])
    inp, outs, _ = _run(cfg)
    assert_close(outs[0], oracle_decide(cfg, inp), TOL_BF16, what=f"L={L}")


@pytest.mark.parametrize("L", [897, 960])
def test_largest_capacity(L):
    """Capacity 960 (15 prefix chunks, the most the kernel takes): the fewest
    workgroups are free of prefix attention, so some also take a QKV role."""
    cfg = pcfg(layers=2, steps=2, capacity=960, prefix_lens=[L])
    inp, outs, nk = _run(cfg)
    assert nk == 2
    assert_close(outs[0], oracle_decide(cfg, inp), TOL_BF16, what=f"C=960 L={L}")


@pytest.mark.parametrize("C,L", [(0, 0), (1, 1), (64, 64), (65, 33)])
def test_small_capacities(C, L):
    """No prefix chunk at all (capacity 0: the action rows attend to
    themselves only), one chunk (capacities 1 and 64) and two chunks with the
    second empty: the merge and the ring schedule with the fewest roles."""
    cfg = pcfg(capacity=C, prefix_lens=[L])
    inp, outs, nk = _run(cfg, repeats=2)
    assert nk == 2
    assert np.array_equal(outs[0], outs[1]), "replays must be bit-identical"
    assert_close(outs[0], oracle_decide(cfg, inp), TOL_BF16, what=f"C={C} L={L}")


@pytest.mark.parametrize("rows", [1, 7, 16])
def test_row_counts(rows):
    cfg = pcfg(rows=rows, capacity=320, prefix_lens=[300])
    inp, outs, _ = _run(cfg)
    assert_close(outs[0], oracle_decide(cfg, inp), TOL_BF16, what=f"rows={rows}")


def test_small_capacity_and_three_steps():
    cfg = pcfg(layers=3, steps=3, dt=-1.0 / 3, capacity=100, prefix_lens=[77])
    inp, outs, _ = _run(cfg, seed=1)
    assert_close(outs[0], oracle_decide(cfg, inp), TOL_BF16, what="C=100 L=77, 3 layers x 3 steps")


def test_replays_are_bit_identical_and_tags_advance():
    """Many decisions on one handle: exchange tags advance every decision and
    the buffers are never cleared, so stale words of earlier decisions must
    never be mistaken for fresh ones."""
    cfg = pcfg()
    inp, outs, _ = _run(cfg, repeats=6)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_replays_many_steps_are_bit_identical():
    """Ten Euler steps, three decisions in a row: every exchange buffer's uses
    (per layer-step, per norm input, per state hand-off between steps) run on
    from one decision to the next without a gap."""
    cfg = pcfg(layers=2, steps=10, dt=-0.1)
    inp, outs, _ = _run(cfg, repeats=3)
    assert_close(outs[0], oracle_decide(cfg, inp), TOL_BF16, what="2 layers x 10 steps")
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_zero_velocity_head_is_bit_exact():
    cfg = pcfg(layers=1, steps=2)
    inp = phx_inputs.make_inputs(cfg, 2)
    w = inp["weights"].copy()
    phx_inputs.view(w, cfg, "W_out")[:] = 0.0
    outs, _ = gpu_decide(cfg, dict(inp, weights=w, weights_bits=phx_inputs.bf16_round(w)[1]))
    assert np.array_equal(outs[0], inp["noise"]), "W_out == 0 must return the noise bit for bit"


def test_matches_multi_kernel_path():
    from flow_matching_action_decision_amd import PHX_FLAG_MULTI_KERNEL
    cfg = pcfg()
    inp = phx_inputs.make_inputs(cfg, 3)
    p, nk_p = gpu_decide(cfg, inp)
    m, nk_m = gpu_decide(cfg, inp, flags=PHX_FLAG_MULTI_KERNEL)
    assert nk_p == 2 and nk_m > 2
    d = compare(p[0], m[0])
    say(f"  persistent vs multi-kernel: max_abs={d['max_abs']:.3e}")
    assert d["max_abs"] <= 2e-2


def test_restore_is_bit_exact():
    """decide -> overwrite the prefix -> decide -> reload the original -> decide."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    cfg = pcfg(layers=1, steps=2, capacity=256, prefix_lens=[200])
    a = phx_inputs.make_inputs(cfg, 4)
    b = phx_inputs.make_inputs(cfg, 5)
    ex = Expert(cfg, a["weights"], a["weights_bits"])
    try:
        assert ex.kernels_per_decision() == 2
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


@pytest.mark.slow
@pytest.mark.timeout(400)
def test_every_rollout_request_on_the_decision_kernel():
    """Each request of the 16-request rollout batch (prefix lengths drawn from
    {512, 640, 768, 800}) decided alone on the persistent kernel, against the
    oracle's decision of the whole batch (requests are independent)."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    rcfg = phx_inputs.workload("rollout_b16_bf16")
    rin = phx_inputs.make_inputs(rcfg, 0)
    ref = oracle_decide(rcfg, rin)
    cfg = pcfg(layers=rcfg["layers"], steps=rcfg["steps"], dt=rcfg["dt"], rows=rcfg["rows"],
               capacity=rcfg["capacity"], prefix_lens=[int(rin["lens"][0])])
    ex = Expert(cfg, rin["weights"], rin["weights_bits"])
    try:
        assert ex.kernels_per_decision() == 2
        worst = 0.0
        for r in range(rcfg["batch"]):
            L = int(rin["lens"][r])
            say(f"case rollout request {r} on the decision kernel, L={L}")
            one = dict(rin, kv_k=rin["kv_k"][r:r + 1], kv_v=rin["kv_v"][r:r + 1], kv_k_bits=rin["kv_k_bits"][r:r + 1],
                       kv_v_bits=rin["kv_v_bits"][r:r + 1], lens=rin["lens"][r:r + 1], noise=rin["noise"][r:r + 1])
            keep = ex.load_all(one)
            out = ex.decide(torch.from_numpy(np.ascontiguousarray(one["noise"])).cuda())
            torch.cuda.synchronize()
            assert ex.status() == 0
            m = assert_close(out.cpu().numpy(), ref[r:r + 1], TOL_BF16, what=f"request {r} (L={L})")
            worst = max(worst, m["max_abs"])
            del keep
        say(f"  worst max_abs over the 16 requests: {worst:.3e}")
    finally:
        ex.close()
