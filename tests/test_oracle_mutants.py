"""Mutation sweep over the oracle: each planted mistake must fail a pin.

A copy of ``oracle/oracle.c`` with one plausible slip (a dropped term, a
wrong sign, a wrong index, a transposed operand, a swapped operand) is built
into a temporary library, and the pin battery is run against it.  The real
oracle passes the battery (test_oracle_pins), so a mutant that also passed
would mean the pins cannot tell the slip from the method.  CPU only; the
mistakes are planted in the oracle, never in GPU code.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import pin_battery

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = [
    ("time embedding: cos half replaced by sin", "e[half + j] = cos(tau * w);", "e[half + j] = sin(tau * w);"),
    ("time embedding: wrong frequency exponent", "-(double)j / (double)half", "-(double)j / (double)E"),
    ("modulation: transposed operand", "Wmod_n[(size_t)j * n2 + c]", "Wmod_n[(size_t)c * E + j]"),
    ("norm: eps dropped", "ss / (double)D + eps", "ss / (double)D"),
    ("norm: 1+scale replaced by scale", "* (1.0 + scale[d]) + shift[d]", "* scale[d] + shift[d]"),
    ("norm: shift sign", "* (1.0 + scale[d]) + shift[d]", "* (1.0 + scale[d]) - shift[d]"),
    ("norm: mean replaced by sum", "sqrt(ss / (double)D + eps)", "sqrt(ss + eps)"),
    ("matmul: accumulation dropped", "yr[n] += xv * (double)wr[n];", "yr[n] = xv * (double)wr[n];"),
    ("rope: sign of first output", "v[j] = a * c - b * s;", "v[j] = a * c + b * s;"),
    ("rope: sign of second output", "v[j + half] = b * c + a * s;", "v[j + half] = b * c - a * s;"),
    ("rope: wrong frequency", "pow(base, -2.0 * (double)j / (double)Dh)", "pow(base, -1.0 * (double)j / (double)Dh)"),
    ("gelu: wrong constant", "sqrt(2.0 / M_PI)", "sqrt(1.0 / M_PI)"),
    ("gelu: cubic term dropped", "(z + 0.044715 * z * z * z)", "(z)"),
    ("attention: scale dropped", "logit[t] = s * scale;", "logit[t] = s;"),
    ("attention: wrong kv head mapping", "int m = mh / H, hh = mh % H, g = hh / group;",
     "int m = mh / H, hh = mh % H, g = hh % KVH;"),
    ("attention: action keys left out", "int T = L + M;", "int T = L;"),
    ("decide: action position offset dropped", "pos[m] = base + L + m;", "pos[m] = base + m;"),
    ("decide: position base dropped", "pos[m] = base + L + m;", "pos[m] = L + m;"),
    ("commit: values captured as keys",
     "memcpy(vout + (((size_t)b * NL + l) * M) * kvd, va,", "memcpy(vout + (((size_t)b * NL + l) * M) * kvd, ka,"),
    ("commit: nothing captured", "        if (kout && vout) {", "        if (0) {"),
    ("commit: flow time ignored", "  one.tau0 = tau;", "  one.tau0 = c->tau0;"),
    ("decide: Euler sign", "x[i] += c->dt * proj[i];", "x[i] -= c->dt * proj[i];"),
    ("decide: tau schedule sign", "double tau = c->tau0 + (double)k * c->dt;", "double tau = c->tau0 - (double)k * c->dt;"),
    ("decide: gate and up swapped", "act[(size_t)r * F + f] = orc_gelu_tanh(g) * u;",
     "act[(size_t)r * F + f] = orc_gelu_tanh(u) * g;"),
    ("decide: MLP norm uses attention modulation", "mod + (size_t)(2 * l + 1) * 2 * D", "mod + (size_t)(2 * l) * 2 * D"),
    ("decide: value rows taken from keys", "memcpy(va + (size_t)m * kvd, src + hd + kvd,", "memcpy(va + (size_t)m * kvd, src + hd,"),
    ("decide: attention residual dropped", "orc_matmul(BM, hd, D, o, W_o, proj);\n      for (int i = 0; i < BM * D; ++i) h[i] += proj[i];",
     "orc_matmul(BM, hd, D, o, W_o, proj);\n      for (int i = 0; i < BM * D; ++i) h[i] = proj[i];"),
    ("decide: RoPE not applied to keys", "orc_rope(M, KVH, Dh, pos, c->rope_base, ka);", ""),
    ("decide: final norm uses first modulation", "mod + (size_t)(2 * NL) * 2 * D", "mod"),
    ("layernorm: mean not subtracted", "var += (r[d] - mean) * (r[d] - mean);", "var += r[d] * r[d];"),
    ("layernorm: eps dropped", "1.0 / sqrt(var + eps);", "1.0 / sqrt(var);"),
    ("dit: scale and shift swapped", "const double *shift_a = mod, *scale_a = mod + D, *gate_a = mod + 2 * D;",
     "const double *scale_a = mod, *shift_a = mod + D, *gate_a = mod + 2 * D;"),
    ("dit: MLP gate dropped", "x[(size_t)t * D + d] += gate_m[d] * proj[(size_t)t * D + d];",
     "x[(size_t)t * D + d] += proj[(size_t)t * D + d];"),
    ("dit: MLP uses attention modulation", "const double *shift_m = mod + 3 * D, *scale_m = mod + 4 * D, *gate_m = mod + 5 * D;",
     "const double *shift_m = mod, *scale_m = mod + D, *gate_m = mod + 5 * D;"),
    ("dit: value rows taken from keys", "memcpy(v + (size_t)t * hd, src + 2 * hd, sizeof(double) * hd);",
     "memcpy(v + (size_t)t * hd, src + hd, sizeof(double) * hd);"),
    ("dit: GELU left out", "for (size_t i = 0; i < (size_t)T * F; ++i) up[i] = orc_gelu_tanh(up[i]);", ""),
    ("dit: modulation from the wrong block", "const float* Wm = W_mod + (size_t)b * E * 6 * D;", "const float* Wm = W_mod;"),
    ("prefill: wrong kv head mapping", "const int i = ih / H, hh = ih % H, g = hh / group;",
     "const int i = ih / H, hh = ih % H, g = hh % KVH;"),
    ("prefill: MLP norm uses the attention gains", "mod[d] = (double)G[(size_t)(2 * l + 1) * D + d];",
     "mod[d] = (double)G[(size_t)(2 * l) * D + d];"),
    ("prefill: positions start at one", "for (int i = 0; i < T; ++i) pos[i] = i;",
     "for (int i = 0; i < T; ++i) pos[i] = i + 1;"),
    ("prefill: values captured as keys", "memcpy(vout + (size_t)l * T * kvd, v,", "memcpy(vout + (size_t)l * T * kvd, k,"),
    ("prefill: RoPE not applied to keys", "orc_rope(T, KVH, Dh, pos, c->rope_base, k);", ""),
    ("prefill: attention residual replaced", "x[i] += proj[i];\n\n    for (int d = 0; d < D; ++d) mod[d]",
     "x[i] = proj[i];\n\n    for (int d = 0; d < D; ++d) mod[d]"),
    ("prefill: gate and up swapped",
     "orc_gelu_tanh(gu[(size_t)t * 2 * F + f]) * gu[(size_t)t * 2 * F + F + f]",
     "orc_gelu_tanh(gu[(size_t)t * 2 * F + F + f]) * gu[(size_t)t * 2 * F + f]"),
    ("prefill: softmax scale dropped", "      p[t] = s * scale;", "      p[t] = s;"),
    ("quantize: ties away from zero", "rintf(W[(size_t)k * N + n] / sc)", "roundf(W[(size_t)k * N + n] / sc)"),
    ("quantize: truncation", "rintf(W[(size_t)k * N + n] / sc)", "truncf(W[(size_t)k * N + n] / sc)"),
    ("quantize: 128 levels", "const float sc = m / 127.0f;", "const float sc = m / 128.0f;"),
    ("quantize: scale from the first row", "      if (a > m) m = a;", "      if (k == 0) m = a;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique in oracle.c: {old!r}"
    mut = src.replace(old, new)
    c_path = tmp_path / "oracle_mut.c"
    c_path.write_text(mut)
    so_path = str(tmp_path / "liboracle_mut.so")
    oracle.build(src=str(c_path), out=so_path)
    lib = oracle.load(so_path)
    failed = pin_battery.run_all(lib)
    assert failed, f"planted mistake '{name}' passed every pin"
