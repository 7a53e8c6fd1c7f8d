"""Plants plausible mistakes in copies of the oracle (CPU only) and checks
that the pins catch each one.  The oracle source itself is never changed.
Each mutant runs in a child process, so a mutant that crashes (an
out-of-bounds read, say) also counts as caught."""
import os
import subprocess
import sys

import pytest

import oracle as O
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

# (name, text in oracle.c, planted replacement)
MUTANTS = [
    ("causal_top_left", "return j <= i + Lk - Lq;", "return j <= i;"),
    ("causal_off_by_one", "return j <= i + Lk - Lq;", "return j < i + Lk - Lq;"),
    ("scale_dropped", "scratch[j] = c->scale * dot;", "scratch[j] = dot;"),
    ("lse_log2", "*lse_out = M + log(Z);", "*lse_out = M + log2(Z);"),
    ("lse_missing_max", "*lse_out = M + log(Z);", "*lse_out = log(Z);"),
    ("no_max_subtraction", "Z += exp(scratch[j] - M);", "Z += exp(scratch[j]);"),
    ("empty_row_lse_zero", "*lse_out = -INFINITY;\n        return;", "*lse_out = 0.0;\n        return;"),
    ("key_head_ignored", "+ j) * c->Hkv + kh) * c->D;", "+ j) * c->Hkv + 0) * c->D;"),
    ("value_reads_keys", "const uint16_t *vrow = key_row(c, c->v, b, j, kh);",
     "const uint16_t *vrow = key_row(c, c->k, b, j, kh);"),
    ("packed_keys_at_query_offset", "(int64_t)c->cu_k[b] + j", "(int64_t)c->cu_q[b] + j"),
    ("paged_slot_from_block", "return base + ((blk * c->BS + j % c->BS) * c->Hkv",
     "return base + ((blk * c->BS + j / c->BS % c->BS) * c->Hkv"),
    ("paged_table_row_ignored", "c->block_table[(int64_t)b * c->max_blocks + j / c->BS]", "c->block_table[j / c->BS]"),
    ("paged_head_ignored", "c->BS) * c->Hkv + kh) * c->D;", "c->BS) * c->Hkv + 0) * c->D;"),
    ("paged_one_key_short", "return c->block_table ? (int64_t)c->seqlens_k[b] :",
     "return c->block_table ? (int64_t)c->seqlens_k[b] - 1 :"),
    ("gqa_prefill_interleaved", "const int64_t kh = h / (H / Hkv);", "const int64_t kh = h % Hkv;"),
    ("weights_not_normalised", "const double w = exp(scratch[j] - M) / Z;",
     "const double w = exp(scratch[j] - M);"),
    ("gqa_interleaved", "const int32_t kh = qh / (c->Hq / c->Hkv);\n    const int64_t ctx = c->context_lens[s], D = c->D;\n    const uint16_t *qrow = c->q + ((int64_t)s * c->Hq + qh) * D;\n    double *o = ",
     "const int32_t kh = qh % c->Hkv;\n    const int64_t ctx = c->context_lens[s], D = c->D;\n    const uint16_t *qrow = c->q + ((int64_t)s * c->Hq + qh) * D;\n    double *o = "),
    ("decode_reads_whole_last_block", "for (int64_t t = 0; t < ctx; t++) {\n        const uint16_t *kr",
     "for (int64_t t = 0; t < (ctx + c->BS - 1) / c->BS * c->BS; t++) {\n        const uint16_t *kr"),
    ("decode_slot_from_block", "const int64_t slot = t % c->BS;", "const int64_t slot = t / c->BS % c->BS;"),
    ("merge_rescale_sign", "const double w_run = *run_max == -INFINITY ? 0.0 : exp(*run_max - top);",
     "const double w_run = *run_max == -INFINITY ? 0.0 : exp(top - *run_max);"),
    ("tile_state_max_not_subtracted", "const double w = exp(scores[i] - mx);", "const double w = exp(scores[i]);"),
    ("step_ignores_token_count", "if (b * c->BS + slot >= n_tok) break;", "if (b * c->BS + slot >= c->BS * c->tile_block_counts[s]) break;"),
    ("step_finalize_unguarded", "const double inv_l = state_l[u] > 0.0 ? 1.0 / state_l[u] : 0.0;",
     "const double inv_l = 1.0 / state_l[u];"),
    ("step_state_not_carried", "double carried_max = c->m[unit], carried_den = c->l[unit];",
     "double carried_max = -INFINITY, carried_den = 0.0;"),
    ("finalize_unguarded", "const double inv_l = run_den > 0.0 ? 1.0 / run_den : 0.0;",
     "const double inv_l = 1.0 / run_den;"),
    ("bwd_jacobian_without_rowdot", "const double ds = prob[j] * (dprob[j] - rowdot);",
     "const double ds = prob[j] * dprob[j];"),
    ("bwd_dk_unscaled", "dkrow[d] += c->scale * ds * bf16_value(qrow[d]);", "dkrow[d] += ds * bf16_value(qrow[d]);"),
    ("bwd_dv_from_ds", "dvrow[d] += prob[j] * bf16_value(dorow[d]);", "dvrow[d] += ds * bf16_value(dorow[d]);"),
    ("bwd_dq_from_values", "dqrow[d] += c->scale * ds * bf16_value(krow[d]);",
     "dqrow[d] += c->scale * ds * bf16_value(c->v[((k0 + j) * Hkv + kh) * D + d]);"),
    ("bwd_group_first_head_only", "for (int64_t h = kh * R; h < (kh + 1) * R; h++)",
     "for (int64_t h = kh * R; h < kh * R + 1; h++)"),
    ("bwd_unnormalised_probs", "prob[j] = prob[j] == -INFINITY ? 0.0 : exp(prob[j] - M) / Z;",
     "prob[j] = prob[j] == -INFINITY ? 0.0 : exp(prob[j] - M);"),
    ("bwd_given_out_ignored",
     "rowdot = 0.0;\n                for (int64_t d = 0; d < D; d++) rowdot += bf16_value(dorow[d]) * orow[d];",
     "(void)orow;"),
    ("tile_levels_ascending", "for (int64_t r = max_tiles - 1; r >= 0; r--) {", "for (int64_t r = 0; r < max_tiles; r++) {"),
    ("tile_count_floor", "const int64_t n = (seq_len_at(cu_q, b) + block_q - 1) / block_q;",
     "const int64_t n = seq_len_at(cu_q, b) / block_q;"),
    ("tile_sort_ascending", "+ sort_grain - 1) / sort_grain < kx) {", "+ sort_grain - 1) / sort_grain > kx) {"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name}: anchor text not found exactly once"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"liboracle_{name}.so"
    O.build(str(path), str(lib))
    return str(lib)


_RUNNER = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle as O
from oracle_pins import ALL_PINS
lib = O.load({lib!r})
failed = 0
for pin in ALL_PINS:
    try:
        pin(lib)
    except Exception as e:
        failed += 1
        print("caught by", pin.__name__, type(e).__name__)
sys.exit(3 if failed else 0)
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER.format(root=os.path.dirname(tests), tests=tests, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin caught the planted mistake '{name}':\n{r.stdout}{r.stderr}"


def test_unmutated_copy_passes(tmp_path):
    """Control: the same child-process runner passes on an unmodified copy, so
    a caught mutant is caught by a pin and not by the harness."""
    lib = _build_mutant(tmp_path, "control", "#include <math.h>", "#include <math.h>")
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER.format(root=os.path.dirname(tests), tests=tests, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
