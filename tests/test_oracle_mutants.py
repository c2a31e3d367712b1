"""The pins catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (on the CPU, in the
copy), builds it, and runs the pin suite against that build in a child process:
the suite must fail.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "round_half_away": ("float r = rintf(t);", "float r = roundf(t);"),
    "k3_wrong_short_slot": ("return (c % 11 == 10) ? 3 : 7;", "return (c % 11 == 0) ? 3 : 7;"),
    "dropped_softmax_scale": ("e[t] = acc * scale;", "e[t] = acc;"),
    "k_zero_wrong_channel": ("(double)L->k_zero[g * L->d + c];", "(double)L->k_zero[g * L->d];"),
    "early_flush": ("L->N - L->Tq == L->R)", "L->N - L->Tq == L->R - 1)"),
    "v_zero_from_scale": ("(double)L->v_zero[tt];", "(double)L->v_scale[tt];"),
    "reversed_offset": ("float t = (x[(long)i * stride] - mn) / s;",
                        "float t = (mx - x[(long)i * stride]) / s;"),
    "prefill_causal_off_by_one": ("const int p = N - n_q + j;", "const int p = N - n_q + j - 1;"),
    "prefill_no_causal_mask": ("const int p = N - n_q + j;", "const int p = N - 1;"),
    "prefill_query_of_wrong_head": ("const double *qv = q + (((size_t)s * g + h) * n_q + j) * d;",
                                    "const double *qv = q + (((size_t)s * g) * n_q + j) * d;"),
    "rpc_flush_rounded_up": ("n_flush = (current - keep) / L->G * L->G;",
                             "n_flush = (current - keep + L->G - 1) / L->G * L->G;"),
    "rpc_ratio_inverted": ("const int keep = (int)(((long long)current * L->rpc_permille) / 1000);",
                           "const int keep = (int)(((long long)current * (1000 - L->rpc_permille)) / 1000);"),
    "pack_msb_first": ("*shift = bits * (c % per_word);",
                       "*shift = 32 - bits * (1 + c % per_word);"),
    # per-token Key
    "k_tok_qmax_of_value_bits": ("kvqo_quantize(x, d, 1, (1 << L->k_bits) - 1, codes, 1,",
                                 "kvqo_quantize(x, d, 1, (1 << L->v_bits) - 1, codes, 1,"),
    "k_tok_dequant_zero_as_scale": (
        "return (double)row_codes[c] * (double)L->k_scale[tt] + (double)L->k_zero[tt];",
        "return (double)row_codes[c] * (double)L->k_scale[tt] + (double)L->k_scale[tt];"),
    "k_tok_dequant_other_token": (
        "return (double)row_codes[c] * (double)L->k_scale[tt] + (double)L->k_zero[tt];",
        "return (double)row_codes[c] * (double)L->k_scale[tt ^ 1] + (double)L->k_zero[tt ^ 1];"),
    # live byte count
    "bytes_k_tok_meta_per_channel": ("long long kmeta = k_tok ? Tq * 8LL : (Tq / G) * 8LL * d;",
                                     "long long kmeta = (Tq / G) * 8LL * d;"),
    "bytes_v_meta_dropped": ("long long vmeta = Tq * 8LL;", "long long vmeta = 0;"),
    "bytes_recent_one_tensor": ("return code_bytes + kmeta + vmeta + Tr * 4LL * d;",
                                "return code_bytes + kmeta + vmeta + Tr * 2LL * d;"),
}

# pin suites run against each mutant
PIN_FILES = ["test_oracle_pins.py", "test_oracle_key_per_token.py"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "kvq_oracle.c")).read()
    assert src.count(old) >= 1, "mutation site moved: " + old  # every occurrence is mutated
    (tmp_path / "kvq_oracle.c").write_text(src.replace(old, new))
    shutil.copy(os.path.join(ROOT, "oracle", "kvq_oracle.h"), tmp_path / "kvq_oracle.h")
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off",
                           "-fPIC", "-shared", str(tmp_path / "kvq_oracle.c"), "-o", str(so), "-lm"])
    env = dict(os.environ, KVQ_ORACLE_SO=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        ] + [os.path.join(ROOT, "tests", f) for f in PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "pins did not catch mutant %s\n%s" % (name, r.stdout[-2000:])
