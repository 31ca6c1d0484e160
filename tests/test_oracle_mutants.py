"""Plant plausible mistakes in copies of oracle.c and check that the pins
catch every one of them (the oracle's own source is never modified)."""
import os

import pytest

import oracle
import oracle_pins

# (id, original snippet, mutated snippet): every occurrence is replaced.
MUTANTS = [
    ("kv_head_modulo", "int g = h / G;", "int g = h % J->Hkv;"),
    ("slot_off_by_one", "t % J->bs, J->Hkv", "(t + 1) % J->bs, J->Hkv"),
    ("page_index_shift", "[(long long)s * J->max_blocks + t / J->bs]",
     "[(long long)s * J->max_blocks + (t + 1) / J->bs]"),
    ("pool_head_swapped", "(((block * Hkv + g) *", "(((block * Hkv + (Hkv - 1 - g)) *"),
    ("drops_last_token", "scores(J, q_row(J, s, h), s, kv_head(J, h), 0, L, z)",
     "scores(J, q_row(J, s, h), s, kv_head(J, h), 0, L - 1, z)"),
    ("exp_sign", "exp(z[t - t0] - zmax)", "exp(zmax - z[t - t0])"),
    ("no_max_subtraction", "exp(z[t - t0] - zmax)", "exp(z[t - t0])"),
    ("scale_dropped", "z[t - t0] = J->scale * dot;", "z[t - t0] = dot;"),
    ("unnormalised", "res[d] = acc[d] / sum;", "res[d] = acc[d];"),
    ("half_exponent_bias", "expo - 25", "expo - 24"),
    ("half_subnormal", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("partial_max_natural_units", "J->m[pi] = ORACLE_LOG2E * zmax;", "J->m[pi] = zmax;"),
    ("merge_weight_sign", "exp2(m[r * NP + i] - M)", "exp2(M - m[r * NP + i])"),
    ("merge_drops_l", "double w = l[r * NP + i] *", "double w = 1.0 *"),
    ("partition_tail_dropped", "int t1 = t0 + J->P < L ? t0 + J->P : L;",
     "int t1 = t0 + J->P < L ? t0 + J->P : L - 1;"),
    ("varlen_causal_off_by_one", "int lim = L - qlen + j + 1;", "int lim = L - qlen + j;"),
    ("varlen_not_causal", "int lim = L - qlen + j + 1;", "int lim = L;"),
    ("varlen_row_offset", "long long row = J->cu_q[s] + j;", "long long row = J->cu_q[s] + qlen - 1 - j;"),
    ("bf16_wrong_half", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b;"),
    ("f32_read_as_half", "if (J->dtype == 2) return (double)((const float *)base)[idx];",
     "if (J->dtype == 2) return oracle_half_to_double(((const uint16_t *)base)[idx]);"),
    ("dot_skips_last_dim", "for (int d = 0; d < J->D; ++d)\n            dot +=",
     "for (int d = 0; d < J->D - 1; ++d)\n            dot +="),
]


@pytest.mark.parametrize("mid,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, mid, orig, mut):
    src = open(oracle.SRC_PATH).read()
    assert orig in src, f"mutation site for {mid} not found in oracle.c"
    msrc = tmp_path / "oracle_mut.c"
    msrc.write_text(src.replace(orig, mut))
    lib = oracle.compile_oracle(str(msrc), str(tmp_path / f"liboracle_{mid}.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:
            caught.append(f"{pin.__name__}: {str(e)[:80]}")
    assert caught, f"mutant {mid} passed every pin"
