"""Plant plausible mistakes in the checker's decode-layer composition (CPU only) and check
that the closed-form pins of test_oracle_layer_pins.py catch every one.

Each mutant is oracle.decode_layer's own source with one textual change, compiled in the
checker's namespace and swapped in for the duration of the test; the pins call
oracle.decode_layer through the module, so they run the mutant.  The unmutated pins pass in
test_oracle_layer_pins.py.
"""
from __future__ import annotations

import inspect
import textwrap

import pytest

import oracle
from tests import test_oracle_layer_pins as pins

ROPE_Q = "q = rope(q, nq, hd, pos, shape.rope_theta)"
ROPE_K = "k = rope(k, nkv, hd, pos, shape.rope_theta)"

MUTANTS = {
    "rope dropped from k": [(ROPE_K, "k = k")],
    "rope dropped from q": [(ROPE_Q, "q = q")],
    "rope applied to v as well": [(ROPE_K, ROPE_K + "; v = rope(v, nkv, hd, pos, shape.rope_theta)")],
    "rope at pos + 1": [(ROPE_Q, ROPE_Q.replace("pos,", "pos + 1,")), (ROPE_K, ROPE_K.replace("pos,", "pos + 1,"))],
    "rope with the frequencies of the other pair order": [
        (ROPE_Q, "q = rope(q[::-1].copy(), nq, hd, pos, shape.rope_theta)[::-1].copy()"),
        (ROPE_K, "k = rope(k[::-1].copy(), nkv, hd, pos, shape.rope_theta)[::-1].copy()")],
    "new k and v written at slot pos + 1": [("kc[:, pos, :]", "kc[:, pos + 1, :]"), ("vc[:, pos, :]", "vc[:, pos + 1, :]")],
    "new k and v written at slot pos - 1": [("kc[:, pos, :]", "kc[:, pos - 1, :]"), ("vc[:, pos, :]", "vc[:, pos - 1, :]")],
    "only the new k written": [("vc[:, pos, :] = v16.reshape(nkv, hd)", "pass")],
    "k written into the v cache": [("vc[:, pos, :] = v16.reshape(nkv, hd)", "vc[:, pos, :] = k16.reshape(nkv, hd)")],
    "kv heads swapped at the write": [("kc[:, pos, :] = k16.reshape(nkv, hd)", "kc[:, pos, :] = k16.reshape(nkv, hd)[::-1]"),
                                      ("vc[:, pos, :] = v16.reshape(nkv, hd)", "vc[:, pos, :] = v16.reshape(nkv, hd)[::-1]")],
    "attention over pos keys (new slot left out)": [("pos + 1, shape.max_ctx)", "pos, shape.max_ctx)")],
    "attention over pos + 2 keys": [("pos + 1, shape.max_ctx)", "pos + 2, shape.max_ctx)")],
    "norm 2 fed h instead of h1": [("n2 = rmsnorm(h1_in,", "n2 = rmsnorm(h,")],
    "norm 2 fed the attention output residual only": [("n2 = rmsnorm(h1_in,", "n2 = rmsnorm(yo,")],
    "gains swapped": [('rmsnorm(h, w["attn_norm"]', 'rmsnorm(h, w["ffn_norm"]'),
                      ('rmsnorm(h1_in, w["ffn_norm"]', 'rmsnorm(h1_in, w["attn_norm"]')],
    "norm 1 with the ffn gain": [('rmsnorm(h, w["attn_norm"]', 'rmsnorm(h, w["ffn_norm"]')],
    "attention residual dropped": [("h1 = h + yo", "h1 = yo")],
    "ffn residual added to h instead of h1": [("h2 = h1_in + yd", "h2 = h + yd")],
    "ffn residual dropped": [("h2 = h1_in + yd", "h2 = yd")],
    "swiglu operands swapped": [("swiglu(g, u)", "swiglu(u, g)")],
    "gate and up both from the gate matrix": [('w["up"], n2)', 'w["gate"], n2)')],
}


def mutant(changes):
    src = textwrap.dedent(inspect.getsource(oracle.decode_layer))
    for old, new in changes:
        assert src.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
        src = src.replace(old, new)
    ns = dict(vars(oracle))
    exec(compile(src, "<mutant decode_layer>", "exec"), ns)
    return ns["decode_layer"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_layer_pins_catch_mutation(name, monkeypatch):
    monkeypatch.setattr(oracle, "decode_layer", mutant(MUTANTS[name]))
    caught = []
    for pin in pins.PINS:
        try:
            pin()
        except Exception as e:  # an assertion, or an index past the cache
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught the mutation '{name}'"


def test_unmutated_source_passes_every_pin(monkeypatch):
    monkeypatch.setattr(oracle, "decode_layer", mutant([]))
    for pin in pins.PINS:
        pin()
