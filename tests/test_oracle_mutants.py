"""The pins catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a copy of ``oracle/oracle.c`` (a dropped term,
a wrong sign, a wrong operand or index, a read before the write, a decay on the
wrong step), builds it with gcc into a temporary directory, and runs every pin
against it in a subprocess.  At least one pin must fail; the unmodified source
must pass them all.  The copy is made on the CPU only; nothing here touches a
GPU.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
RUNNER = os.path.join(ROOT, "tests", "oracle_pins.py")

MUTANTS = {
    "la_feature_map_drops_plus_one": (
        "return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x : exp(x);"),
    "la_key_feature_from_query": (
        "fk[i] = elu_plus_one(rd(k, qk_row + i, dt));",
        "fk[i] = elu_plus_one(rd(q, qk_row + i, dt));"),
    "la_normaliser_not_accumulated": ("z[i] += fk[i];", "z[i] += 0.0 * fk[i];"),
    "la_reads_state_before_write": (
        "den += fq[i] * z[i];", "den += fq[i] * (z[i] - fk[i]) + 1e-300;"),
    "la_numerator_with_key_feature": (
        "num[j] += fq[i] * S[(size_t)i * dv + j];", "num[j] += fk[i] * S[(size_t)i * dv + j];"),
    "delta_sign_of_correction": (
        "u[j] = b * (rd(v, v_row + j, dt) - r[j]);",
        "u[j] = b * (rd(v, v_row + j, dt) + r[j]);"),
    "delta_beta_applied_twice": (
        "S[(size_t)i * dv + j] += kt[i] * u[j];",
        "S[(size_t)i * dv + j] += kt[i] * u[j] * b;"),
    "delta_read_with_query": (
        "r[j] += kt[i] * S[(size_t)i * dv + j];",
        "r[j] += qt[i] * S[(size_t)i * dv + j];"),
    "delta_output_with_key": (
        "o[v_row + j] += qt[i] * S[(size_t)i * dv + j];",
        "o[v_row + j] += kt[i] * S[(size_t)i * dv + j];"),
    "delta_state_transposed_write": (
        "S[(size_t)i * dv + j] += kt[i] * u[j];",
        "S[(size_t)i * dv + j] += kt[j % dk] * u[i % dv];"),
    "gate_sign": (
        "? exp(rd(g, qk_row + i, dt))", "? exp(-rd(g, qk_row + i, dt))"),
    "gate_uses_previous_token": (
        "? exp(rd(g, qk_row + i, dt))",
        "? exp(rd(g, (t > 0 ? qk_row - dk : qk_row) + i, dt))"),
    "gate_same_for_all_channels": (
        "? exp(rd(g, qk_row + i, dt))", "? exp(rd(g, qk_row, dt))"),
    "scalar_gate_sign": (
        ": exp(rd(g, (size_t)bh * T + t, dt));", ": exp(-rd(g, (size_t)bh * T + t, dt));"),
    "scalar_gate_uses_previous_token": (
        ": exp(rd(g, (size_t)bh * T + t, dt));",
        ": exp(rd(g, (size_t)bh * T + (t > 0 ? t - 1 : t), dt));"),
    "gla_decay_applied_twice": ("S[i] *= a;", "S[i] *= a * a;"),
    "gla_decay_uses_next_token": (
        "const double a = exp(rd(g, (size_t)bh * T + t, dt));",
        "const double a = exp(rd(g, (size_t)bh * T + (t + 1 < T ? t + 1 : t), dt));"),
    "gla_write_with_wrong_value_column": (
        "vt[j] = rd(v, v_row + j, dt);", "vt[j] = rd(v, v_row + (j + 1) % dv, dt);"),
    "bwd_output_gradient_not_added": (
        "dS[(size_t)i * dv + j] += qa * dov[j];", "dS[(size_t)i * dv + j] += 0.0 * qa * dov[j];"),
    "bwd_key_gradient_drops_read_term": (
        "acc += dS[(size_t)i * dv + j] * u[j] - b * S[(size_t)i * dv + j] * du[j];",
        "acc += dS[(size_t)i * dv + j] * u[j];"),
    "bwd_beta_gradient_without_read": (
        "db += du[j] * (rd(v, v_row + j, dt) - r[j]);", "db += du[j] * rd(v, v_row + j, dt);"),
    "bwd_state_gradient_sign": (
        "dS[(size_t)i * dv + j] -= b * kt[i] * du[j];", "dS[(size_t)i * dv + j] += b * kt[i] * du[j];"),
    "bwd_value_gradient_without_beta": ("dvv[v_row + j] = b * du[j];", "dvv[v_row + j] = du[j];"),
    "prologue_silu_without_gate": (
        "const double y = apply_silu ? xi / (1.0 + exp(-xi)) : xi;",
        "const double y = apply_silu ? xi / (1.0 + exp(xi)) : xi;"),
    "prologue_normalised_by_squared_norm": ("double nrm = sqrt(ss);", "double nrm = ss;"),
    "beta_broadcast_wrong_head": (
        "const int hs = Hb == 1 ? 0 : h;", "const int hs = Hb == 1 ? 0 : (h + 1) % Hb;"),
    "gla_read_with_key": (
        "const double qi = rd(q, qk_row + i, dt);", "const double qi = rd(k, qk_row + i, dt);"),
    "bf16_widening_wrong_shift": (
        "uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;",
        "uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 15;"),
    "gated_bwd_state_gradient_not_decayed": (
        "dS[(size_t)i * dv + j] *= ga[i];", "dS[(size_t)i * dv + j] *= 1.0;"),
    "gated_bwd_dg_against_undecayed_state": (
        "gi += dS[(size_t)i * dv + j] * Sa[(size_t)i * dv + j];",
        "gi += dS[(size_t)i * dv + j] * Sall[(size_t)t * ss + (size_t)i * dv + j];"),
    "gated_bwd_dg_before_the_erase_term": (
        "if (g) {\n                double gsum = 0.0;",
        "if (g) {\n                for (int i = 0; i < dk; i++) for (int j = 0; j < dv; j++)\n"
        "                    dS[(size_t)i * dv + j] += b * kt[i] * du[j];\n"
        "                double gsum = 0.0;"),
}


def _build_and_run(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = tmp_path / f"lib{name}.so"
    oracle.build(out_path=str(lib), src=str(src))
    env = dict(os.environ, OMP_NUM_THREADS="2",
               PYTHONPATH=os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]))
    return subprocess.run([sys.executable, RUNNER, str(lib)], capture_output=True,
                          text=True, timeout=300, env=env, cwd=ROOT)


def test_unmodified_oracle_passes_all_pins(tmp_path):
    r = _build_and_run(tmp_path, "original", open(SRC).read())
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"pattern for {name} must occur exactly once"
    r = _build_and_run(tmp_path, name, text.replace(old, new))
    assert r.returncode != 0, f"no pin caught {name}: {r.stdout}"
    # a crash would also be non-zero; require that a pin reported the failure
    assert "FAILED:" in r.stdout and r.stdout.strip() != "FAILED:", r.stdout + r.stderr
