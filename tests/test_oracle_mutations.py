"""The oracle pins must catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle's source (on
the CPU, never on a GPU), runs every pin of test_oracle_pins.py against the
mutant and requires at least one of them to fail.
"""

import importlib.util
import inspect
import os
import types

import pytest

import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "sspec_ref.py")

MUTATIONS = {
    "kv head by modulo": ("h = g // G\n        raw", "h = g % hkv\n        raw"),
    "mask one short": ("n_vis = L - kp1 + i + 1", "n_vis = L - kp1 + i"),
    "sm_scale dropped": ("row = scale * raw[i, :n_vis]", "row = raw[i, :n_vis]"),
    "lse in base 2": ("lse_i = m + math.log(", "lse_i = m + math.log2("),
    "sum instead of mean": (".reshape(G * kp1, L).mean(axis=0)", ".reshape(G * kp1, L).sum(axis=0)"),
    "last verify query dropped": ("probs[h * G:(h + 1) * G].reshape(G * kp1, L)",
                                  "probs[h * G:(h + 1) * G, :-1].reshape(G * (kp1 - 1), L)"),
    "ties to highest index": ("np.lexsort((np.arange(L), -scores))",
                              "np.lexsort((-np.arange(L), -scores))"),
    "K rounded not ceiled": ("math.ceil(float(s) * float(L))", "round(float(s) * float(L))"),
    "draft tail one short": ("np.arange(sel_len, ctx_len) if", "np.arange(sel_len + 1, ctx_len) if"),
    "draft ignores selection": ("kept = np.asarray(sel_h)[np.asarray(sel_h) < lim]",
                                "kept = np.arange(lim)"),
    "gather slot wrong": ("rows = pages[phys, :, j % page_size, :]",
                          "rows = pages[phys, :, (j + 1) % page_size, :]"),
    "probabilities not normalised": ("p = np.exp(row - lse_i)", "p = np.exp(row - m)"),
    "append one position late": ("j = int(ctx_lens[r]) - n + i", "j = int(ctx_lens[r]) - n + i + 1"),
    "append slot from the page index": ("kp[page, :, j % page_size, :] = k_new[off + i]",
                                        "kp[page, :, (j // page_size) % page_size, :] = k_new[off + i]"),
    "append rows not advanced": ("        off += n\n    return kp, vp, skipped", "    return kp, vp, skipped"),
    "rollback keeps one rejected": ("new_ctx = np.where(isv, ctx - (k - a), ctx)",
                                    "new_ctx = np.where(isv, ctx - (k - a) + 1, ctx)"),
    "rollback leaves sel_len": ("np.where(isv, np.minimum(np.asarray(sel_len, np.int64), new_ctx)",
                                "np.where(isv, np.asarray(sel_len, np.int64)"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} not unique in the oracle"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pin_calls():
    calls = []
    for nm, fn in inspect.getmembers(pins, inspect.isfunction):
        if not nm.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames, values = params[0].args
            names = [a.strip() for a in argnames.split(",")]
            for v in values:
                calls.append((fn, dict(zip(names, v if isinstance(v, tuple) else (v,)))))
        else:
            calls.append((fn, {}))
    return calls


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    mod = _mutant(name)
    monkeypatch.setattr(pins, "O", mod)
    failed = []
    for fn, kw in _pin_calls():
        try:
            fn(**kw)
        except Exception:
            failed.append(fn.__name__)
    assert failed, f"no pin caught the planted mistake {name!r}"
