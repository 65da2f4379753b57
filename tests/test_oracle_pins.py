"""The oracle against library routines, closed forms, invariants and a tiny
brute-force composition (see pin_battery).  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
import phx_inputs
import pin_battery

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


@pytest.mark.parametrize("pin", pin_battery.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, orc):
    pin(orc)


def test_pages_facts_match_the_pi05_workload():
    """Shapes and counts the pages print, checked against the pi0.5-shape
    workload definition and the oracle's own weight layout."""
    facts = json.load(open(GOLDEN))
    cfg = phx_inputs.workload("pi05_expert_bf16")
    assert cfg["layers"] == facts["expert_layers"]["value"]
    assert cfg["rows"] == facts["action_rows"]["value"]
    assert cfg["steps"] == facts["flow_steps"]["value"]
    assert cfg["head_dim"] == facts["head_dim"]["value"]
    # one modulation projection per norm: two per layer plus the final one
    slices = phx_inputs.weight_slices(cfg)
    assert slices["W_mod"][1][0] == facts["modulation_projections"]["value"]
    assert facts["prefix_tokens_min"]["value"] <= cfg["capacity"] <= facts["prefix_tokens_max"]["value"]
    for L in phx_inputs.RAGGED_CHOICES:
        assert facts["prefix_tokens_min"]["value"] <= L <= facts["prefix_tokens_max"]["value"]
    # the prefix K/V of this shape fits inside the pages' 14.40 MB pi0.5 capsule
    kv_bytes = 2 * cfg["layers"] * cfg["capacity"] * cfg["n_kv_heads"] * cfg["head_dim"] * 2
    assert kv_bytes / 1e6 <= facts["capsule_megabytes"]["value"]
    assert kv_bytes / 1e6 > 0.95 * facts["capsule_megabytes"]["value"]


def test_weight_count_agrees_with_input_layout(orc):
    for name in phx_inputs.WORKLOADS:
        cfg = phx_inputs.workload(name)
        assert oracle.weight_count(cfg, orc) == phx_inputs.weight_count(cfg)


def test_oracle_rejects_bad_arguments(orc):
    cfg = pin_battery.tiny_cfg()
    inp = phx_inputs.make_inputs(cfg)
    with pytest.raises(ValueError):
        oracle.decide(cfg, inp["weights"][:-1], inp["kv_k"], inp["kv_v"], inp["lens"], inp["noise"], lib=orc)
    with pytest.raises(ValueError):
        oracle.decide(cfg, inp["weights"], inp["kv_k"], inp["kv_v"], np.array([0, 6]), inp["noise"], lib=orc)


def test_thread_count_does_not_change_results(orc, monkeypatch):
    """OpenMP only splits independent outputs: one thread and many agree bit for bit."""
    import subprocess, sys
    code = ("import sys; sys.path[:0]=[%r, %r]; import numpy as np, oracle, phx_inputs, pin_battery;"
            "cfg=pin_battery.tiny_cfg(width=64, mlp_hidden=128, n_heads=4, head_dim=16, time_emb_dim=32);"
            "inp=phx_inputs.make_inputs(cfg, seed=9);"
            "out=oracle.decide(cfg, inp['weights'], inp['kv_k'], inp['kv_v'], inp['lens'], inp['noise']);"
            "sys.stdout.write(out['actions'].tobytes().hex())") % (os.path.dirname(os.path.dirname(__file__)),
                                                                     os.path.dirname(__file__))
    res = []
    for n in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        res.append(subprocess.check_output([sys.executable, "-c", code], env=env))
    assert res[0] == res[1]
