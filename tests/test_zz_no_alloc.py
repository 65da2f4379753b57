"""phx_expert_decide_noalloc against phx_expert_decide.

The allocation-free decision runs the same decision kernel with its exchange
and control words in the device's static scratch instead of the handle's
arena, so on the same inputs it must return the same actions bit for bit.
Two handles share the scratch here: the larger request first, then a smaller
one (fewer rows, a shorter prefix, fewer layers and steps), then the larger
one again, twice, so each call starts from what the previous one left in the
shared words and counter.
"""
import numpy as np
import pytest

import phx_inputs
from gpu_util import TOL_BF16, assert_close, oracle_decide, say

pytestmark = pytest.mark.gpu


def _handle(cfg, inp):
    from flow_matching_action_decision_amd.expert import Expert
    ex = Expert(cfg, inp["weights"], inp["weights_bits"])
    keep = ex.load_all(inp)
    return ex, keep


def _both(ex, inp):
    """(phx_expert_decide, phx_expert_decide_noalloc) actions of one handle."""
    import torch
    nz = torch.from_numpy(np.ascontiguousarray(inp["noise"])).cuda()
    ref = ex.decide(nz)
    torch.cuda.synchronize()
    assert ex.status() == 0
    out = torch.full_like(nz, float("nan"))
    ex.decide_noalloc(nz, out)
    torch.cuda.synchronize()
    assert ex.status() == 0, "the allocation-free decision gave up waiting"
    return ref.cpu().numpy(), out.cpu().numpy()


def test_noalloc_matches_decide_twice_second_smaller():
    import torch
    big = phx_inputs.workload("pi05_expert_bf16", id=70, layers=2, steps=3, dt=-1.0 / 3, prefix_lens=[768])
    # fewer rows, fewer prefix chunks, fewer layers and steps: every part of the shape changes
    small = phx_inputs.workload("pi05_expert_bf16", id=71, layers=1, steps=2, dt=-0.5, rows=5,
                                capacity=320, prefix_lens=[300])
    a = phx_inputs.make_inputs(big, 0)
    b = phx_inputs.make_inputs(small, 1)
    say(f"case noalloc: rows {big['rows']} L {big['prefix_lens']} then rows {small['rows']} L {small['prefix_lens']}")
    ea, ka = _handle(big, a)
    eb, kb = _handle(small, b)
    try:
        assert ea.kernels_per_decision() == 2 and eb.kernels_per_decision() == 2
        ref_a, out_a = _both(ea, a)
        assert np.array_equal(out_a, ref_a), "first call: allocation-free actions differ from phx_expert_decide"
        assert_close(out_a, oracle_decide(big, a), TOL_BF16, what="noalloc, 10 rows, L=768")
        ref_b, out_b = _both(eb, b)
        assert np.array_equal(out_b, ref_b), "second (smaller) call differs from phx_expert_decide"
        assert_close(out_b, oracle_decide(small, b), TOL_BF16, what="noalloc, 5 rows, L=300")
        # the scratch keeps the last call's words and counter; the larger handle again, twice
        nz = torch.from_numpy(np.ascontiguousarray(a["noise"])).cuda()
        out = torch.empty_like(nz)
        free0 = torch.cuda.mem_get_info()[0]
        for _ in range(2):
            out.fill_(float("nan"))
            ea.decide_noalloc(nz, out)
            torch.cuda.synchronize()
            assert ea.status() == 0
            assert np.array_equal(out.cpu().numpy(), ref_a)
        assert torch.cuda.mem_get_info()[0] == free0, "device memory changed across allocation-free decisions"
        # a third handle of the larger one's shape takes over the words without a clear
        c = phx_inputs.make_inputs(big, 3)
        ec, kc = _handle(big, c)
        try:
            ref_c, out_c = _both(ec, c)
            assert np.array_equal(out_c, ref_c), "same-shape handle on the shared words differs"
            assert not np.array_equal(out_c, ref_a)
        finally:
            del kc
            ec.close()
    finally:
        del ka, kb
        ea.close()
        eb.close()


def test_noalloc_rejects_handles_off_the_decision_kernel():
    from flow_matching_action_decision_amd import PHX_FLAG_MULTI_KERNEL
    from flow_matching_action_decision_amd.binding import PhxError
    from flow_matching_action_decision_amd.expert import Expert
    import torch
    cfg = phx_inputs.workload("pi05_expert_bf16", id=72, layers=1, steps=1, prefix_lens=[64], capacity=64)
    inp = phx_inputs.make_inputs(cfg, 2)
    ex = Expert(cfg, inp["weights"], inp["weights_bits"], flags=PHX_FLAG_MULTI_KERNEL)
    try:
        keep = ex.load_all(inp)
        nz = torch.from_numpy(np.ascontiguousarray(inp["noise"])).cuda()
        with pytest.raises(PhxError, match="static scratch"):
            ex.decide_noalloc(nz, torch.empty_like(nz))
        del keep
    finally:
        ex.close()
