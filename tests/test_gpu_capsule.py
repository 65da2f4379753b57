"""Execution-state capsules through the C ABI: snapshot, restore and fork of
the declared state regions ("FlashRT-PAI", section 3.4 and Table 6).

For every execution path (the persistent decision kernel, the multi-kernel
graph, the large-token plan, the DiT-style step): decide on context A, save a
capsule, overwrite the context with B and decide, restore the capsule and
decide again -- bit-identical to the first decision; restore the capsule
into a second handle of the same plan that never loaded a context (fork) --
bit-identical again; the first, restored and forked decisions also match the
oracle's decision on context A; a handle of another plan rejects the capsule.
"""
import numpy as np
import pytest

import oracle
import phx_inputs
from gpu_util import TOL_BF16, TOL_TOKENS, assert_close, oracle_decide, say, small_cfg

pytestmark = pytest.mark.gpu


def _plans():
    return {
        "persistent": phx_inputs.workload("pi05_expert_bf16", layers=2, steps=2, dt=-0.5),
        "multi_kernel": small_cfg(batch=3, prefix_lens=[100, 3, 64]),
        "large_token": dict(id=62, name="va_capsule", block="decoder", layers=2, width=256, n_heads=2, head_dim=128,
                            n_kv_heads=2, mlp_hidden=512, state_dim=128, rows=200, batch=1, capacity=300, steps=2,
                            time_emb_dim=64, tau0=1.0, dt=-0.5, rms_eps=1e-6, rope_base=10000.0, dtype="bf16",
                            weight_std=0.02, prefix_lens=[250]),
        "dit": dict(id=63, name="dit_capsule", block="dit", layers=2, width=256, n_heads=2, head_dim=128,
                    n_kv_heads=2, mlp_hidden=512, state_dim=256, rows=300, batch=1, capacity=0, steps=1,
                    time_emb_dim=64, tau0=1.0, dt=0.0, rms_eps=1e-6, rope_base=10000.0, dtype="bf16",
                    weight_std=0.02, prefix_lens=[0]),
    }


@pytest.mark.parametrize("plan", ["persistent", "multi_kernel", "large_token", "dit"])
def test_capsule_restore_and_fork_bit_exact(plan):
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    cfg = _plans()[plan]
    say(f"case capsule {plan}")
    a = phx_inputs.make_inputs(cfg, 0)
    b = phx_inputs.make_inputs(cfg, 1)
    nz = torch.from_numpy(a["noise"]).cuda()
    ex = Expert(cfg, a["weights"], a["weights_bits"])
    fork = Expert(cfg, a["weights"], a["weights_bits"])
    try:
        regions = ex.capsule_regions()
        say(f"  regions: {[(r['name'], r['bytes']) for r in regions]}, capsule {ex.capsule_bytes()} bytes")
        assert ex.capsule_bytes() >= sum(r["bytes"] for r in regions)
        if plan != "dit":
            assert {r["name"] for r in regions} >= {"prefix_lengths", "position_table"}
        keep_a = ex.load_all(a)
        first = ex.decide(nz).cpu().numpy().copy()
        cap = ex.capsule_save()
        keep_b = ex.load_all(b)
        other = ex.decide(nz).cpu().numpy().copy()
        ex.capsule_restore(cap)
        again = ex.decide(nz).cpu().numpy().copy()
        fork.capsule_restore(cap)
        forked = fork.decide(nz).cpu().numpy().copy()
        torch.cuda.synchronize()
        del keep_a, keep_b
    finally:
        ex.close()
        fork.close()
    assert np.all(np.isfinite(first))
    if plan != "dit":  # the DiT-style step has no context to overwrite
        assert not np.array_equal(first, other)
    assert np.array_equal(first, again), "restore must reproduce the decision bit for bit"
    assert np.array_equal(first, forked), "fork must reproduce the decision bit for bit"
    # the restored and forked decisions are the decision on context A, not only the handle's own first run
    if plan == "dit":
        ref = oracle.dit(cfg, a["weights"], a["noise"][0])["out"]
        assert_close(again[0], ref, TOL_TOKENS, what="dit restored vs oracle")
        assert_close(forked[0], ref, TOL_TOKENS, what="dit forked vs oracle")
    else:
        ref = oracle_decide(cfg, a)
        assert_close(again, ref, TOL_BF16, what=f"{plan} restored vs oracle on context A")
        assert_close(forked, ref, TOL_BF16, what=f"{plan} forked vs oracle on context A")


def test_capsule_rejects_another_plan():
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    from flow_matching_action_decision_amd.binding import PhxError
    cfg = small_cfg()
    say("case capsule plan mismatch")
    a = phx_inputs.make_inputs(cfg, 0)
    other_cfg = small_cfg(capacity=120)
    o = phx_inputs.make_inputs(other_cfg, 0)
    ex = Expert(cfg, a["weights"], a["weights_bits"])
    other = Expert(other_cfg, o["weights"], o["weights_bits"])
    try:
        keep = ex.load_all(a)
        cap = ex.capsule_save()
        torch.cuda.synchronize()
        with pytest.raises(PhxError):
            other.capsule_restore(cap)
        junk = torch.zeros_like(cap)
        with pytest.raises(PhxError):
            ex.capsule_restore(junk)
        # the handle is unchanged by the failed restores
        nz = torch.from_numpy(a["noise"]).cuda()
        r1 = ex.decide(nz).cpu().numpy().copy()
        ex.capsule_restore(cap)
        r2 = ex.decide(nz).cpu().numpy().copy()
        del keep
    finally:
        ex.close()
        other.close()
    assert np.array_equal(r1, r2)
