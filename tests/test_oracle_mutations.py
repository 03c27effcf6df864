"""Planted mistakes in a copy of the oracle must fail the pins.

Each case copies oracle/gdn_oracle.c, makes one plausible slip in the copy
(on the CPU, never in the real source), builds it, and runs the pin tests
against it in a child process; the child must fail.  This shows that the pins
would catch that slip in the real oracle.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTATIONS = {
    "decay_after_correction": (
        "            for (int c = 0; c < g->dk; ++c)\n                row[c] = alpha * row[c];\n",
        "",
        "                row[c] = row[c] + u * kh[c];\n",
        "                row[c] = alpha * (row[c] + u * kh[c]);\n"),
    "sign_of_correction": ("const double u = beta * (v[i] - p);", "const double u = beta * (v[i] + p);"),
    "decay_dropped": ("row[c] = alpha * row[c];", "row[c] = 1.0 * row[c];"),
    "output_before_correction": ("r = r + row[c] * qh[c];", "r = r + (row[c] - u * kh[c]) * qh[c];"),
    "interleaved_groups": ("const int grp = h / g->G;", "const int grp = h % g->Hk;"),
    "scale_uses_dv": ("const double scale = 1.0 / sqrt((double)g->dk);", "const double scale = 1.0 / sqrt((double)g->dv);"),
    "no_eps_in_norm": ("const double rk = 1.0 / sqrt(nk + ORACLE_EPS);", "const double rk = 1.0 / sqrt(nk);"),
    "gate_sign": ("const double alpha = exp(-softplus(a[h]));", "const double alpha = exp(-softplus(-a[h]));"),
    "reversed_taps": ("acc = acc + load_act(w, w_bf16, (size_t)c * g->W + j) * t[j];",
                      "acc = acc + load_act(w, w_bf16, (size_t)c * g->W + (g->W - 1 - j)) * t[j];"),
    "tail_not_shifted": ("            t[j] = t[j + 1];\n", "            t[j] = t[j];\n"),
    "key_state_transposed": ("p = p + row[c] * kh[c];",
                             "p = p + S[((size_t)h * g->dv + (c % g->dv)) * g->dk + (i % g->dk)] * kh[c];"),
    "depth_off_by_one": ("        depth[i] = depth[parent[i]] + 1;\n", "        depth[i] = depth[parent[i]];\n"),
}

# Slips in the per-channel-decay step (recur_token_kda), which comes after the
# scalar step in the file: these edit the LAST occurrence of their anchor and run
# against the variant's own pins.
KDA_MUTATIONS = {
    "kda_decay_after_correction": (
        "            for (int c = 0; c < g->dk; ++c)\n                row[c] = al[c] * row[c];\n",
        "",
        "                row[c] = row[c] + u * kh[c];\n",
        "                row[c] = al[c] * (row[c] + u * kh[c]);\n"),
    "kda_one_gate_per_head": ("al[c] = exp(-softplus(a[(size_t)h * g->dk + c]));",
                              "al[c] = exp(-softplus(a[(size_t)h * g->dk]));"),
    "kda_decays_value_rows": ("row[c] = al[c] * row[c];", "row[c] = al[i % g->dk] * row[c];"),
    "kda_gate_sign": ("al[c] = exp(-softplus(a[(size_t)h * g->dk + c]));",
                      "al[c] = exp(-softplus(-a[(size_t)h * g->dk + c]));"),
    "kda_channel_reversed": ("al[c] = exp(-softplus(a[(size_t)h * g->dk + c]));",
                             "al[c] = exp(-softplus(a[(size_t)h * g->dk + (g->dk - 1 - c)]));"),
    "kda_sign_of_correction": ("const double u = beta * (v[i] - p);", "const double u = beta * (v[i] + p);"),
}


def _mutant_fails_pins(name, edits, last, pin_files, tmp_path):
    src = open(SRC).read()
    for old, new in zip(edits[::2], edits[1::2]):
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = new.join(src.rsplit(old, 1)) if last else src.replace(old, new, 1)
    c = tmp_path / "mutant.c"
    c.write_text(src)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", str(so), str(c), "-lm"])
    env = dict(os.environ, GDN_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", f) for f in pin_files]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name} passed every pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    _mutant_fails_pins(name, MUTATIONS[name], False, ["test_oracle_pins.py", "test_chunk_algebra.py"], tmp_path)


@pytest.mark.parametrize("name", sorted(KDA_MUTATIONS))
def test_kda_pins_catch_planted_mistake(name, tmp_path):
    _mutant_fails_pins(name, KDA_MUTATIONS[name], True, ["test_oracle_kda.py"], tmp_path)
