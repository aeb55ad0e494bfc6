"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one of them (CPU only).

Each mutation edits one expression of ``oracle/oracle.c`` in a temporary copy
(a dropped scale, a flipped mask, a wrong sign, a transposed index, a missing
term), builds it with gcc into a temporary directory and runs the small pins
from ``oracle_pins.py`` on it.  The shipped source is never modified.  A
mutation that no pin rejects would mean the pins leave that part of the
oracle unchecked.
"""
import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "logits_drop_scale": ("S[i * N + j] = scale * acc;", "S[i * N + j] = acc;"),
    "causal_mask_flipped": ("if (causal && j > i)", "if (causal && j < i)"),
    "causal_mask_off_by_one": ("if (causal && j > i)", "if (causal && j >= i)"),
    "lse_drop_max": ("double L = m + log(sum);", "double L = log(sum);"),
    "lse_log2": ("double L = m + log(sum);", "double L = m + log2(sum);"),
    "p_unnormalised": ("row[j] = exp(row[j] - L);", "row[j] = exp(row[j] - m);"),
    "o_reversed_v": ("orow[c] += p * vh[j * d + c];", "orow[c] += p * vh[j * d + (d - 1 - c)];"),
    "delta_drop_p": ("Di += P[i * N + jj] * acc;", "Di += acc;"),
    "ds_sign": ("(dS[i * N + jj] - Di)", "(dS[i * N + jj] + Di)"),
    "dq_drop_scale": ("grow[c] *= scale;", "grow[c] *= 1.0;"),
    "dq_uses_v": ("grow[c] += s * kh[jj * d + c];", "grow[c] += s * vh[jj * d + c];"),
    "dk_drop_scale": ("krow[c] *= scale;", "krow[c] *= 1.0;"),
    "dk_uses_p": ("krow[c] += s * qh[ii * d + c];", "krow[c] += p * qh[ii * d + c];"),
    "dv_transposed_p": ("double p = P[ii * N + j], s", "double p = P[j * N + ii], s"),
    "dv_uses_q": ("vrow[c] += p * gh[ii * d + c];", "vrow[c] += p * qh[ii * d + c];"),
    "decode_top_left_mask": ("const long last = causal ? off + i : Nk - 1;",
                             "const long last = causal ? i : Nk - 1;"),
    "decode_mask_off_by_one": ("const long last = causal ? off + i : Nk - 1;",
                               "const long last = causal ? off + i - 1 : Nk - 1;"),
    "decode_drop_scale": ("S[j] = scale * acc;", "S[j] = acc;"),
    "decode_lse_drop_max": ("const double L = m + log(sum);", "const double L = log(sum);"),
    "decode_p_unnormalised": ("const double p = exp(S[j] - L);", "const double p = exp(S[j] - m);"),
    "decode_v_row_shift": ("orow[c] += p * vh[j * d + c];\n      }\n      free(S);",
                           "orow[c] += p * vh[((j + 1) % Nk) * d + c];\n      }\n      free(S);"),
}


def _caught(orc) -> list:
    hits = []
    for i, pin in enumerate(pins.ALL_SMALL_PINS):
        try:
            pin(orc)
        except AssertionError:
            hits.append(i)
        except (FloatingPointError, ValueError, RuntimeError):
            hits.append(i)
    return hits


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(tmp_path, name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor %r not found in oracle.c" % old
    src = tmp_path / "oracle_mut.c"
    src.write_text(text.replace(old, new))
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / "liboracle_mut.so"))
    hits = _caught(oracle.Oracle(lib))
    assert hits, "no pin detects the planted mistake %r" % name


def test_unmutated_oracle_passes_every_pin():
    assert _caught(oracle.default()) == []


# Mistakes in the grouped-query layer of the oracle (Python): the shared
# K, V gradient averaged instead of summed, and query heads mapped to K, V
# heads round-robin (h % H_kv) instead of in consecutive groups (h // G).
def _mean_reduce(g, H_kv):
    B, H, N, d = g.shape
    if H_kv == H:
        return g
    return g.reshape(B, H_kv, H // H_kv, N, d).mean(axis=2)


def _roundrobin_expand(t, H):
    if t.shape[1] == H:
        return t
    return np.ascontiguousarray(np.tile(t, (1, H // t.shape[1], 1, 1)))


@pytest.mark.parametrize("name,attr,fn", [("gqa_grad_mean", "_reduce_kv", _mean_reduce),
                                          ("gqa_roundrobin_heads", "_expand_kv", _roundrobin_expand)])
def test_pins_catch_gqa_mutation(monkeypatch, name, attr, fn):
    monkeypatch.setattr(oracle, attr, fn)
    assert _caught(oracle.default()), "no pin detects the planted mistake %r" % name
