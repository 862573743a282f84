"""Every plausible mistake planted in a copy of the oracle must be caught by at
least one pin (CPU only).

Each mutation is a textual edit of ``oracle/oracle.c`` compiled into a scratch
library; the real oracle is untouched.  This shows that the pins constrain
each part of the oracle: GQA mapping, scale, causal boundary, LSE, the
normalisation of Out, operand indexing, merge weights and order, the paged
gather.
"""
import os
import subprocess

import pytest

from tests.oracle_pins import ALL_PINS

ORACLE_C = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                        "oracle.c")

# (name, exact source text, replacement, occurrence to replace (0-based) or None for all)
MUTATIONS = [
    ("gqa_modulo_mapping", "const int hk = h / group;", "const int hk = h % Hkv;", 0),
    ("scale_dropped", "s[j - lo] = scale * dot;", "s[j - lo] = dot;", 0),
    ("scale_squared", "s[j - lo] = scale * dot;", "s[j - lo] = scale * scale * dot;", 0),
    ("causal_off_by_one", "if (causal && hi > pos + 1) hi = pos + 1;",
     "if (causal && hi > pos) hi = pos;", 0),
    ("causal_ignored", "if (causal && hi > pos + 1) hi = pos + 1;", "", 0),
    ("lse_without_max", "const double L = m + log(sum);", "const double L = log(sum);", 0),
    ("out_unnormalised", "const double w = exp(s[j - lo] - L);",
     "const double w = exp(s[j - lo] - m);", 0),
    ("k_transposed_index", "dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);",
     "dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[D - 1 - d]);", 0),
    ("v_wrong_head", "const uint16_t* vrow = v + ((b * Skv + j) * Hkv + hk) * (int64_t)D;",
     "const uint16_t* vrow = v + ((b * Skv + j) * Hkv + (hk + 1) % Hkv) * (int64_t)D;", 0),
    ("last_key_dropped", "for (int64_t j = lo; j < hi; ++j) sum += exp(s[j - lo] - m);",
     "for (int64_t j = lo; j < hi - 1; ++j) sum += exp(s[j - lo] - m);", 0),
    ("merge_weight_sign", "const double w = exp(Li - L);", "const double w = exp(L - Li);", 0),
    ("merge_lse_without_max", "const double L = M + log(sum);", "const double L = log(sum);", 0),
    ("merge_accepts_duplicates", "if (order[i].key == order[i - 1].key) { free(order); return -2; }",
     "", 0),
    ("merge_arrival_order", "qsort(order, (size_t)n_parts, sizeof(orc_order_item), orc_cmp_items);",
     "", 0),
    ("decode_wrong_slot", "const uint16_t* krow = k_pool + ((page * Hkv + hk) * P + j % P) * (int64_t)D;",
     "const uint16_t* krow = k_pool + ((page * Hkv + hk) * P + (j + 1) % P) * (int64_t)D;", 0),
    ("decode_drops_current_token", "for (int64_t j = 0; j < len; ++j) sum += exp(s[j] - m);",
     "for (int64_t j = 0; j < len - 1; ++j) sum += exp(s[j] - m);", 0),
    ("bwd_delta_dropped", "const double ds = p * (dp[j] - delta);", "const double ds = p * dp[j];", 0),
    ("bwd_delta_unweighted", "delta += s[j] * dp[j];", "delta += dp[j];", 0),
    ("bwd_dq_scale_dropped", "dqrow[d] += scale * ds * kd;", "dqrow[d] += ds * kd;", 0),
    ("bwd_dk_sign", "dk[koff + d] += scale * ds * qd;", "dk[koff + d] -= scale * ds * qd;", 0),
    ("bwd_dv_uses_ds", "dv[koff + d] += p * gd;", "dv[koff + d] += ds * gd;", 0),
    ("bwd_dp_uses_k", "g += bf16_to_double(grow[d]) * bf16_to_double(v[koff + d]);",
     "g += bf16_to_double(grow[d]) * bf16_to_double(k[koff + d]);", 0),
    ("bwd_causal_off_by_one", "if (causal && hi > pos + 1) hi = pos + 1;",
     "if (causal && hi > pos) hi = pos;", 1),
    ("bwd_wrong_group", "for (int h = hk * group; h < (hk + 1) * group; ++h) {",
     "for (int h = hk; h < Hq; h += Hkv) {", 0),
    ("lm_logz_without_max", "const double lz = m + log(sum);", "const double lz = log(sum);", 0),
    ("lm_wrong_token", "logp[t] = z[tokens[t]] - lz;", "logp[t] = z[(tokens[t] + 1) % V] - lz;", 0),
    ("lm_sign", "logp[t] = z[tokens[t]] - lz;", "logp[t] = lz - z[tokens[t]];", 0),
    ("lm_row_stride", "const float* row = w + (int64_t)v * H;", "const float* row = w + (int64_t)v;", 0),
    ("lm_last_row_dropped", "for (int v = 0; v < V; ++v) sum += exp(z[v] - m);",
     "for (int v = 0; v < V - 1; ++v) sum += exp(z[v] - m);", 0),
]


def _mutant(tmp_path, name, old, new, occ):
    src = open(ORACLE_C).read()
    assert old in src, f"mutation {name}: source text not found"
    parts = src.split(old)
    if occ is None:
        text = new.join(parts)
    else:
        text = old.join(parts[: occ + 1]) + new + old.join(parts[occ + 1:])
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", str(c), "-o", str(so),
                           "-lm"])
    return str(so)


@pytest.mark.parametrize("name,old,new,occ", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, occ):
    lib = _mutant(tmp_path, name, old, new, occ)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib_path=lib)
        except (AssertionError, ValueError) as e:
            caught.append((pin.__name__, str(e)[:80]))
            break
    assert caught, f"no pin caught the planted mistake {name}"
