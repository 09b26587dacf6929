"""Plant plausible mistakes in copies of the oracle and check that a pin trips.

Each mutant is the oracle's C source with one small textual change, built into
a temporary library and run (in a child process, so a crashing mutant cannot
take the test runner down) against the pin battery of tests/oracle_pins.py.
The test passes when at least one pin fails for every mutant, and the
unmodified source passes them all.  CPU only.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTANTS = {
    # the new write beta v k^T is dropped
    "drop_write": ("g * (s - beta * w[r] * k[c]) + beta * v[r] * k[c]",
                   "g * (s - beta * w[r] * k[c])"),
    # the erase term enters with the wrong sign
    "erase_sign": ("g * (s - beta * w[r] * k[c])", "g * (s + beta * w[r] * k[c])"),
    # the gate also decays the new write
    "decay_on_write": ("g * (s - beta * w[r] * k[c]) + beta * v[r] * k[c]",
                       "g * (s - beta * w[r] * k[c] + beta * v[r] * k[c])"),
    # the erase uses the projection of the wrong side: (I - beta k k^T) S
    "transposed_erase": ("S[(size_t)r * dk + c] = g * (s - beta * w[r] * k[c])",
                         "S[(size_t)r * dk + c] = g * (s - beta * w[c % dv] * k[r % dk])"),
    # the path is applied node-to-root instead of root-to-node
    "reversed_path": ("for (int a = 0, b = len - 1; a < b; ++a, --b) {",
                      "for (int a = 0, b = len - 1; a < 0; ++a, --b) {"),
    # the output is read before the node's own update
    "pre_update_output": (
        "        gdn_step(dv, dk, Si, kb, vb, bi, gi, w);\n"
        "        lg[((size_t)b * P->Hv + h) * N + i] = lgi;\n"
        "        state_times(dv, dk, Si, P->q + ix_qk(P, b, i, hk), o + ix_v(P, b, i, h));\n",
        "        state_times(dv, dk, Si, P->q + ix_qk(P, b, i, hk), o + ix_v(P, b, i, h));\n"
        "        gdn_step(dv, dk, Si, kb, vb, bi, gi, w);\n"
        "        lg[((size_t)b * P->Hv + h) * N + i] = lgi;\n"),
    # the ancestor mask also marks the node itself
    "mask_includes_self": ("for (int m = 0; m + 1 < len; ++m)\n                mb",
                           "for (int m = 0; m < len; ++m)\n                mb"),
    # value heads map to key heads round-robin instead of in groups
    "head_map": ("const int hk = h / (P->Hv / P->Hk);", "const int hk = h % P->Hk;"),
    # the write vector forgets the gate on the parent state
    "u_no_gate": ("bi * (vb[r] - gi * w[r])", "bi * (vb[r] - w[r])"),
    # the path log-gate misses the node's own gate
    "log_gamma_no_self": ("            lgi += log(gi);\n", "\n"),
    # memo mode starts children from S0 instead of the parent's state
    "memo_from_s0": ("const double* Sp = par[i] < 0 ? S0 : S + (size_t)par[i] * SS;",
                     "const double* Sp = S0;"),
    # a parent equal to the node itself is accepted as valid
    "check_allows_self": ("par[i] >= i) return i + 1;", "par[i] > i) return i + 1;"),
    # the acceptance walk takes the last matching child instead of the first
    "accept_last_child": ("                    found = i;\n                    break;\n",
                          "                    found = i;\n"),
    # the acceptance walk compares against the child's own prediction
    "accept_own_target": ("if (par[i] == cur && dr[i] == want) {", "if (par[i] == cur && dr[i] == tg[i]) {"),
    # the accepted length counts the prefix as a node
    "accept_len_off": ("        int cur = -1, len = 0;", "        int cur = -1, len = 1;"),
    # tree construction expands one candidate per step whatever the width
    "build_one_per_step": ("            int m = w;\n", "            int m = 1;\n"),
    # equal scores after one parent go to the higher rank
    "build_tie_rank": ("return a->c < b->c ? -1 : (a->c > b->c);", "return a->c > b->c ? -1 : (a->c < b->c);"),
    # equal scores go to the higher parent index
    "build_tie_parent": ("if (a->p != b->p) return a->p < b->p ? -1 : 1;",
                         "if (a->p != b->p) return a->p > b->p ? -1 : 1;"),
    # a node's children read the drafter row of the node before it
    "build_row_off": ("cand[nc].s = sc[i] + lp[(size_t)(i + 1) * K + c];",
                      "cand[nc].s = sc[i] + lp[(size_t)i * K + c];"),
    # every node's token is read from the prefix's row
    "build_token_row": ("out_tok[n] = tk[(size_t)(cand[t].p + 1) * K + cand[t].c];",
                        "out_tok[n] = tk[cand[t].c];"),
    # a child's score forgets its parent's score
    "build_no_accumulate": ("cand[nc].s = sc[i] + lp[(size_t)(i + 1) * K + c];",
                            "cand[nc].s = lp[(size_t)(i + 1) * K + c];"),
}

CHILD = r"""
import json, sys
sys.path[:0] = [{root!r}, {here!r}]
import oracle, oracle_pins
lib = oracle.load({so!r})
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except Exception as e:           # AssertionError, or a crash-free error
        failed.append(pin.__name__)
        break
print(json.dumps(failed))
"""


def run_battery(so):
    code = CHILD.format(root=ROOT, here=HERE, so=so)
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300)
    if p.returncode != 0:
        return ["<crashed: %d>" % p.returncode]
    return json.loads(p.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    so = oracle.build(str(c), str(tmp_path / "libmutant.so"))
    failed = run_battery(so)
    assert failed, f"no pin caught mutant {name}"


def test_pristine_passes(tmp_path):
    so = oracle.build(SRC, str(tmp_path / "libpristine.so"))
    assert run_battery(so) == []
