"""The C-ABI library on the host: it loads without a GPU, exports every
function include/phx_expert.h declares, and its pure-host calls (config
validation, blob size) behave as documented.  No compute calls."""
import ctypes
import os
import re

import pytest

import phx_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "phx_expert.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"PHX_API\s+[\w\s\*]+?\b(phx_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from flow_matching_action_decision_amd import binding
    return binding.load_library()


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("phx_expert_create", "phx_expert_load_prefix_kv", "phx_expert_decide", "phx_expert_destroy"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from flow_matching_action_decision_amd import binding
    names = _declared()
    assert set(names) == set(binding.EXPORTED), "binding and header disagree"
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_struct_layout_matches_header(lib):
    from flow_matching_action_decision_amd import binding
    # 14 int32-sized fields + 4 floats + 5 int32 = 23 * 4 bytes
    assert ctypes.sizeof(binding.phx_expert_config) == 92
    assert ctypes.sizeof(binding.phx_node_info) == 56


def _cfg(**kw):
    from flow_matching_action_decision_amd import binding
    c = binding.make_config(phx_inputs.workload("pi05_expert_bf16"))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_validate_accepts_the_workloads(lib):
    from flow_matching_action_decision_amd import binding
    for name in phx_inputs.WORKLOADS:
        c = binding.make_config(phx_inputs.workload(name))
        assert binding.phx_expert_validate_config(c) == 0, binding.phx_last_error()


@pytest.mark.parametrize("field,value,code", [
    ("abi_version", 99, -2), ("struct_size", 12, -2), ("layers", 0, -3), ("width", 1000, -3),
    ("head_dim", 96, -3), ("n_kv_heads", 3, -3), ("mlp_hidden", 100, -3), ("state_dim", 7, -3),
    ("rows", 0, -3), ("batch", 17, -3), ("prefix_capacity", -1, -3), ("steps", 0, -3),
    ("time_emb_dim", 3, -3), ("rms_eps", 0.0, -1), ("rope_base", -1.0, -1), ("weight_dtype", 7, -1),
    ("kv_dtype", 0, -3), ("flags", 0x80, -1), ("block_kind", 5, -1), ("mask_kind", 7, -1),
    ("mask_kind", 1, -3),  # the causal mask belongs to the prefix prefill only
])
def test_validate_rejects(lib, field, value, code):
    from flow_matching_action_decision_amd import binding
    c = _cfg(**{field: value})
    assert binding.phx_expert_validate_config(c) == code
    assert binding.phx_last_error()


@pytest.mark.parametrize("field,value", [
    ("mask_kind", 0), ("state_dim", 1024), ("prefix_capacity", 64), ("steps", 2), ("batch", 2), ("head_dim", 64),
    ("weight_dtype", 0),
])
def test_validate_rejects_prefill_shapes(lib, field, value):
    """The prefix prefill: causal mask, token rows as wide as the stack, no cache of its own, one pass,
    one request, bf16 and head_dim 128 or 256 (the large-token kernels)."""
    from flow_matching_action_decision_amd import binding
    c = binding.make_config(phx_inputs.workload("prefix_prefill_bf16"))
    assert binding.phx_expert_validate_config(c) == 0, binding.phx_last_error()
    setattr(c, field, value)
    if field == "weight_dtype":
        c.kv_dtype = value
    assert binding.phx_expert_validate_config(c) == -3
    assert binding.phx_last_error()


def test_validate_mlp_pairing_flags(lib):
    """Paired MLP activations (opt-in) and plain bf16 ones (opt-out) are each a valid choice, not both."""
    from flow_matching_action_decision_amd import binding
    for name in ("wam_dit_bf16", "va_chunk_bf16", "prefix_prefill_bf16"):
        for fl in (binding.PHX_FLAG_PAIRED_ACT, binding.PHX_FLAG_BF16_ACT):
            c = binding.make_config(phx_inputs.workload(name), flags=fl)
            assert binding.phx_expert_validate_config(c) == 0, binding.phx_last_error()
        c = binding.make_config(phx_inputs.workload(name),
                                flags=binding.PHX_FLAG_PAIRED_ACT | binding.PHX_FLAG_BF16_ACT)
        assert binding.phx_expert_validate_config(c) == -1
        assert "exclude" in binding.phx_last_error()


@pytest.mark.parametrize("workload", ["single_layer_fp32", "va_chunk_bf16", "wam_dit_bf16", "prefix_prefill_bf16"])
def test_validate_rejects_the_int8_tier_off_its_path(lib, workload):
    """The 8-bit weight tier: bf16 weights, the decoder block, at most 160 rows."""
    from flow_matching_action_decision_amd import binding
    c = binding.make_config(phx_inputs.workload(workload), flags=binding.PHX_FLAG_WEIGHTS_INT8)
    assert binding.phx_expert_validate_config(c) == -3
    c = binding.make_config(phx_inputs.workload("pi05_expert_w8a16"))
    assert c.flags == binding.PHX_FLAG_WEIGHTS_INT8
    assert binding.phx_expert_validate_config(c) == 0, binding.phx_last_error()


def test_weight_codes_null_handle_without_a_gpu(lib):
    assert lib.phx_expert_weight_codes(None, 0, 0, None, None, None) == -1


def test_prefill_null_arguments_without_a_gpu(lib):
    assert lib.phx_expert_prefill(None, None, 0, None, None, None) == -1


def test_validate_null(lib):
    assert lib.phx_expert_validate_config(None) == -1


def test_weights_bytes_matches_the_input_layout(lib):
    from flow_matching_action_decision_amd import binding
    for name in phx_inputs.WORKLOADS:
        cfg = phx_inputs.workload(name)
        esz = 2 if cfg["dtype"] == "bf16" else 4
        assert binding.phx_expert_weights_bytes(binding.make_config(cfg)) == phx_inputs.weight_count(cfg) * esz


def test_null_handles_are_rejected_without_a_gpu(lib):
    assert lib.phx_expert_load_prefix_kv(None, 0, None, None, 0, None) == -1
    assert lib.phx_expert_decide(None, None, None, None) == -1
    assert lib.phx_expert_decide_noalloc(None, None, None, None) == -1
    n = ctypes.c_int(0)
    assert lib.phx_expert_kernels_per_decision(None, ctypes.byref(n)) == -1
    assert lib.phx_expert_launch_node(None, 0, None) == -1
    lib.phx_expert_destroy(None)  # NULL-safe
    out = ctypes.c_void_p(0)
    from flow_matching_action_decision_amd import binding
    c = _cfg()
    assert lib.phx_expert_create(ctypes.byref(c), None, 0, None, ctypes.byref(out)) == -1
    assert out.value is None


@pytest.mark.parametrize("name,field,value", [
    ("wam_dit_bf16", "state_dim", 1024), ("wam_dit_bf16", "n_kv_heads", 8), ("wam_dit_bf16", "prefix_capacity", 64),
    ("wam_dit_bf16", "steps", 2), ("wam_dit_bf16", "head_dim", 64), ("wam_dit_bf16", "weight_dtype", 0),
    ("va_chunk_bf16", "batch", 2), ("va_chunk_bf16", "state_dim", 2000), ("va_chunk_bf16", "rows", 20000),
])
def test_validate_rejects_large_token_shapes(lib, name, field, value):
    from flow_matching_action_decision_amd import binding
    c = binding.make_config(phx_inputs.workload(name))
    setattr(c, field, value)
    if field == "weight_dtype":
        c.kv_dtype = value
    assert binding.phx_expert_validate_config(c) == -3, f"{name}: {field}={value} accepted"
