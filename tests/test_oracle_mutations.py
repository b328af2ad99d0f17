"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of oracle.c (a dropped term, a
wrong sign, a wrong index, a transposed operand, an off-by-one mask, a wrong
pairing), builds it with gcc into a temporary library, and runs the pin suite
against it in a subprocess.  The suite must fail for every mutant.  Only the
CPU is involved.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "dropped_score_scale": ("s1[j] = dot1 * inv_sqrt_d;", "s1[j] = dot1;"),
    "scale_uses_value_width": ("1.0 / sqrt((double)r->d)", "1.0 / sqrt((double)(r->d + r->dv))"),
    "difference_sign": ("double w = w1 - r->lambda * w2;", "double w = w1 + r->lambda * w2;"),
    "second_map_uses_first_key": (
        "elem(r->k2, r->dtype, r->k_off + (int64_t)j * r->ldk + c);",
        "elem(r->k1, r->dtype, r->k_off + (int64_t)j * r->ldk + c);"),
    "second_map_normalised_by_first": ("double w2 = s2[j] / z2;", "double w2 = s2[j] / z1;"),
    "causal_sees_next_key": ("r.nkeys = c->causal ? i + 1 : c->N;",
                             "r.nkeys = c->causal ? (i + 2 < c->N ? i + 2 : c->N) : c->N;"),
    "lambda_of_wrong_head": ("r.lambda = (double)c->lambda[h];", "r.lambda = (double)c->lambda[0];"),
    "lambda_init_wrong_sign": ("exp(-0.3 * (double)(layer - 1))", "exp(0.3 * (double)(layer - 1))"),
    "lambda_init_off_by_one_layer": ("exp(-0.3 * (double)(layer - 1))", "exp(-0.3 * (double)layer)"),
    "lambda_dot_mispaired": ("* (double)lk1[(int64_t)h * dim + i];",
                             "* (double)lq2[(int64_t)h * dim + i];"),
    "lambda_second_term_sign": ("exp(d1) - exp(d2) + init", "exp(d1) + exp(d2) + init"),
    "rmsnorm_sum_not_mean": ("ms /= (double)dv;", "ms /= 1.0;"),
    "rmsnorm_eps_dropped": ("1.0 / sqrt(ms + eps)", "1.0 / sqrt(ms)"),
    "decode_pair_maps_to_wrong_kv_head": ("int g = (2 * p) / group;", "int g = p / group;"),
    "decode_second_head_is_first": ("(size_t)c->D * (c->dtype == ORACLE_FP32 ? 4 : 2)", "(size_t)0"),
    "bf16_widening_wrong_shift": ("[idx] << 16;", "[idx] << 15;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found: %r" % old
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                           str(mutated), "-o", str(lib), "-lm"])
    env = dict(os.environ, DIFFATTN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
