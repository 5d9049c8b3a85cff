"""The oracle's pins have teeth: each planted mistake below, a plausible slip
in one of oracle.c's recursions or boundary rules, makes at least one pin of
tests/test_oracle_pins.py fail.

Each case writes oracle.c with one edit to a temporary directory, builds it
with the oracle's own compiler flags (warnings off: a mutant may leave a
parameter unused), and runs the pin suite against that build in a fresh
process (RLCA_ORACLE_LIB points the oracle's loader at it).  The suite must
end with failed tests (pytest exit status 1), not with a collection or usage
error.  A control case builds the unmodified source the same way and must
pass, so a failure below is the mistake's doing and not the harness's.
All of it runs on the CPU; nothing here touches the HIP library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in oracle.c, replacement); each text occurs exactly once.
MUTATIONS = [
    ("gae_drops_lambda",
     "adv = delta + carried(gamma * lam, next_adv);", "adv = delta + carried(gamma, next_adv);"),
    ("gae_next_value_index",
     "delta = (double)r[t] + gamma * (double)v[t + 1] - (double)v[t];",
     "delta = (double)r[t] + gamma * (double)v[t] - (double)v[t];"),
    ("gae_returns_without_values",
     "returns[n * T + t] = adv + (double)v[t];", "returns[n * T + t] = adv;"),
    ("td_lambda_drops_one_minus_lambda",
     "gamma * (1.0 - lam) * (double)v[t + 1] +", "gamma * (double)v[t + 1] +"),
    ("discounted_continues_with_gamma_squared",
     "g = (double)r[t] + carried(gamma, next_g);",
     "g = (double)r[t] + carried(gamma * gamma, next_g);"),
    ("edge_ignores_bootstrap",
     "*next_value = bootstrap;", "*next_value = 0.0;"),
    ("truncation_ignored",
     "if (trunc != NULL && trunc[t]) {", "if (0 && trunc != NULL && trunc[t]) {"),
    ("truncation_wins_over_termination",
     "if (term[t]) {", "if (term[t] && !(trunc != NULL && trunc[t])) {"),
    ("truncation_successor_is_zero",
     "*next_value = (double)trunc_values[t];", "*next_value = 0.0;"),
    ("log_ratio_not_clipped_below",
     "if (l < -ORACLE_LOG_RATIO_CLIP) l = -ORACLE_LOG_RATIO_CLIP;", ""),
    ("vtrace_trace_weight_uses_rho",
     "carried(gamma * c, next_vs", "carried(gamma * rho, next_vs"),
    ("vtrace_c_drops_lambda",
     "double c = lam * min_d(c_bar, ratio);", "double c = min_d(c_bar, ratio);"),
    ("vtrace_pg_target_is_value",
     "carried(rho * gamma, next_vs", "carried(0.0 * rho * gamma, next_vs"),
    ("retrace_uses_current_trace_weight",
     "clipped_ratio(pi[t + 1], mu[t + 1])", "clipped_ratio(pi[t], mu[t])"),
    ("retrace_expected_q_replaced_by_q",
     "gamma * (double)eq[t + 1] +", "gamma * (double)q[t + 1] +"),
    ("eligibility_drops_lambda",
     "e = (double)x[t] + carried(gamma * lam, e);", "e = (double)x[t] + carried(gamma, e);"),
    ("reset_after_done_reads_current_flag",
     "return flags[t - 1] != 0;", "return flags[t] != 0;"),
    ("prefix_sum_exclusive",
     "s += (double)x[n * T + t];\n            out[n * T + t] = s;",
     "out[n * T + t] = s;\n            s += (double)x[n * T + t];"),
    ("prefix_sum_i32_saturates",
     "(int64_t)low - 0x100000000LL", "(int64_t)0x7fffffff"),
    ("affine_direction_swapped",
     "if (direction == 0) {", "if (direction != 0) {"),
    ("affine_carry_ignored",
     "double A = carry != NULL ? (double)carry[n] : 0.0;", "double A = 0.0;"),
    ("std_population_divisor",
     "sqrt(ss / (double)(M - 1))", "sqrt(ss / (double)M)"),
    ("ppo_takes_the_larger_term",
     "const int take_unclipped = unclipped <= clipped;",
     "const int take_unclipped = unclipped >= clipped;"),
    ("ppo_no_upper_clip",
     "if (clipped_rho > 1.0 + clip_eps) clipped_rho = 1.0 + clip_eps;", ""),
    ("ppo_gradient_sign",
     "grad[i] = take_unclipped ? -unclipped / (double)M : 0.0;",
     "grad[i] = take_unclipped ? unclipped / (double)M : 0.0;"),
    ("gae_boundary_drops_successor",
     "delta = (double)r[t] + gamma * nv - (double)v[t];", "delta = (double)r[t] - (double)v[t];"),
    ("log_ratio_not_clipped_above",
     "if (l > ORACLE_LOG_RATIO_CLIP) l = ORACLE_LOG_RATIO_CLIP;", ""),
    ("vtrace_rho_clipped_at_c_bar",
     "double rho = min_d(rho_bar, ratio);", "double rho = min_d(c_bar, ratio);"),
    ("vtrace_delta_without_rho",
     "double delta = rho * ((double)r[t] + gamma * (double)v[t + 1] - (double)v[t]);",
     "double delta = ((double)r[t] + gamma * (double)v[t + 1] - (double)v[t]);"),
    ("vtrace_boundary_delta_without_rho",
     "double delta = rho * ((double)r[t] + gamma * nv - (double)v[t]);",
     "double delta = ((double)r[t] + gamma * nv - (double)v[t]);"),
    ("retrace_correction_sign",
     "carried(gamma * c_next, next_qret - (double)q[t + 1])",
     "carried(gamma * c_next, (double)q[t + 1] - next_qret)"),
    ("retrace_ignores_c_bar",
     "double c_next = lam * min_d(c_bar,", "double c_next = lam * min_d(1.0,"),
    ("eligibility_never_resets",
     "if (starts_episode(f, convention, t)) e = 0.0;", ""),
    ("prefix_sum_i32_never_resets",
     "if (starts_episode(f, convention, t)) s = 0;", ""),
    ("mean_with_sample_divisor",
     "s / (double)M : 0.0;", "s / (double)(M - 1) : 0.0;"),
    ("zero_coefficient_does_not_cut",
     "return coef == 0.0 ? 0.0 : coef * value;", "return coef * value;"),
    ("ppo_no_lower_clip",
     "if (clipped_rho < 1.0 - clip_eps) clipped_rho = 1.0 - clip_eps;", ""),
    ("ppo_loss_sign",
     "*loss = M > 0 ? -total / (double)M : 0.0;", "*loss = M > 0 ? total / (double)M : 0.0;"),
    ("ppo_ratio_inverted",
     "exp((double)logp_new[i] - (double)logp_old[i])",
     "exp((double)logp_old[i] - (double)logp_new[i])"),
    ("ppo_normalization_without_eps",
     "((double)adv[i] - mean) / (std + norm_eps)", "((double)adv[i] - mean) / std"),
]


def _build(src_text, tmp_path):
    src = tmp_path / "oracle.c"
    src.write_text(src_text)
    lib = tmp_path / "liboracle_variant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-w",
                    "-fPIC", "-shared", "-I", os.path.join(ROOT, "oracle"), "-o", str(lib),
                    str(src), "-lm"], check=True)
    return str(lib)


def _run_pins(lib, stop_at_first=True):
    env = dict(os.environ, RLCA_ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", PINS, "-q", "-p", "no:cacheprovider",
           "-p", "no:randomly", "-m", "not gpu"]
    if stop_at_first:
        cmd.append("-x")
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_unmodified_build_passes_the_pins(tmp_path):
    with open(SRC) as f:
        r = _run_pins(_build(f.read(), tmp_path), stop_at_first=False)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(name, old, new, tmp_path):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"{name}: the text to mutate must occur exactly once"
    r = _run_pins(_build(text.replace(old, new), tmp_path))
    assert r.returncode == 1, (f"{name}: the pins did not catch it (pytest exit status "
                               f"{r.returncode})\n" + r.stdout[-2000:] + r.stderr[-2000:])
