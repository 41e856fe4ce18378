"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks that
the oracle's pins catch every one: a dropped term, a flipped sign, a wrong index,
an off-by-one window, a wrong rounding mode, a missed cache rewrite."""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dory_oracle.c")
PINS = [os.path.join(ROOT, "tests", f) for f in
        ("test_oracle_primitives.py", "test_oracle_attention.py", "test_oracle_forward.py")]

# name: (text in the oracle, its mistaken replacement)
MUTANTS = {
    "rope_sign": ("row[j + half] = (float)(y * cs + x * sn);", "row[j + half] = (float)(y * cs - x * sn);"),
    "slerp_direction": ("(double)alpha[i] * ((double)oh[i] - (double)x[i])",
                        "(double)alpha[i] * ((double)x[i] - (double)oh[i])"),
    "no_score_scale": ("            s[e] = d * scale;\n        }\n        softmax(s, n);\n        for (int i = 0; i < hd; i++) {\n            double acc = 0.0;\n            for (int64_t e = 0; e < n; e++) acc +=",
                       "            s[e] = d;\n        }\n        softmax(s, n);\n        for (int i = 0; i < hd; i++) {\n            double acc = 0.0;\n            for (int64_t e = 0; e < n; e++) acc +="),
    "gate_sign": ("(1.0 + exp(-((double)g * (double)sg)))", "(1.0 + exp(((double)g * (double)sg)))"),
    "gqa_index": ("        int kh = h / rep;\n        for (int64_t e = 0; e < n; e++) {\n            const float *key",
                  "        int kh = h % nk;\n        for (int64_t e = 0; e < n; e++) {\n            const float *key"),
    "window_off_by_one": ("int64_t first = p + 1 - win > 0 ? p + 1 - win : 0;", "int64_t first = p - win > 0 ? p - win : 0;"),
    "round_half_even": ("float c = roundf(r[d] / s);", "float c = rintf(r[d] / s);"),
    "freeze_one_row_early": ("if (s->rows >= ORA_WARMUP && !s->frozen)", "if (s->rows >= ORA_WARMUP - 1 && !s->frozen)"),
    "mix_drops_input": ("for (size_t j = 0; j < (size_t)t * H; j++) h[j] = state[j] + input[j];",
                        "for (size_t j = 0; j < (size_t)t * H; j++) h[j] = state[j];"),
    "silu_sign": ("return (float)(x / (1.0 + exp(-x)) * ((double)b * (double)su));",
                  "return (float)(x / (1.0 + exp(x)) * ((double)b * (double)su));"),
    "no_q_scale": ("for (int i = 0; i < hd; i++) row[i] *= L->sq[hh * hd + i];", ";"),
    "no_renorm_before_o": ("        ora_justnorm(yr, Q);\n", "\n"),
    "no_logit_scale": ("i++) lg[i] *= m->w.logit_scale[i];", "i++) ;"),
    "field_without_sqrt": ("float c = sqrtf(col[d] / (float)rows);", "float c = col[d] / (float)rows;"),
    "key_not_normed": ("            ora_rope_rotate(row, hd, inv, pos0 + r);\n            ora_justnorm(row, hd);\n        }\n    }",
                       "            ora_rope_rotate(row, hd, inv, pos0 + r);\n        }\n    }"),
    "one_slot_per_loop": ("int si = (sq->mode == ORA_PER_LOOP && rec) ? loop_i : 0;", "int si = 0;"),
    "v_unscaled": ("acc += s[e] * (double)vs[row] * (double)vc[row * hd + i];", "acc += s[e] * (double)vc[row * hd + i];"),
    "k_group_scale_index": ("d += dg * (double)ks[row * ngk + g];", "d += dg * (double)ks[row * ngk];"),
    "rollback_keeps_rows": ("if (q->slots[i].rows > n) q->slots[i].rows = n;", ";"),
    "all_rows_read_the_last": ("matvec(m->w.head, h + (size_t)r * H, c->vocab, H, lg);",
                               "matvec(m->w.head, h + (size_t)(t - 1) * H, c->vocab, H, lg);"),
    "prompt_loops_ignored": ("        loops = m->prompt_loops;", "        ;"),
    "readout_rows_appended": ("int overwrite = sq->mode == ORA_LAST_LOOP && li >= c->n_in && loop_i > 0;",
                              "int overwrite = sq->mode == ORA_LAST_LOOP && rec && loop_i > 0;"),
    "probe_every_token": ("return q->exit_rate >= 0.35f || q->exit_tokens % 8u == 0u;", "return 1;"),
    "second_pass_from_readout": ("for (int j = 0; j < H; j++) h[j] = state[j] + input[j];",
                                 "for (int j = 0; j < H; j++) h[j] = h[j] + input[j];"),
    "rollback_unfreezes": ("if (q->slots[i].rows > n) q->slots[i].rows = n;",
                           "if (q->slots[i].rows > n) { q->slots[i].rows = n; q->slots[i].frozen = 0; }"),
}
# Not planted: `state = justnorm(h)` after a loop acts on a vector a slerp has just
# normalised, so dropping it changes results only at the 1e-7 level of eps.


def _run(name, tmp):
    a, b = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(a) == 1, name
    d = os.path.join(tmp, name)
    os.makedirs(d, exist_ok=True)
    shutil.copy(os.path.join(ROOT, "oracle", "dory_oracle.h"), d)
    with open(os.path.join(d, "dory_oracle.c"), "w") as f:
        f.write(src.replace(a, b))
    lib = os.path.join(d, "liboracle.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", lib, os.path.join(d, "dory_oracle.c"), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, DORY_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PINS],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    return name, r.returncode


@pytest.mark.slow
def test_every_planted_mistake_is_caught(tmp_path):
    with cf.ThreadPoolExecutor(4) as ex:
        results = dict(ex.map(lambda n: _run(n, str(tmp_path)), MUTANTS))
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, f"mistakes no pin catches: {survivors}"
