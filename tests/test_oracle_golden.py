"""The oracle against hand-derived worked examples (tests/golden/hand_worked.json).

The pages print no numeric example, so each fixture case was worked out by
hand: its inputs make every softmax weight rational, and the expected O, LSE
and gradients are exact closed forms, stored as expressions over ``log`` and
``atanh`` with the derivation beside them.  Each case names the passage it
exercises.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

_PATH = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
_NAMES = {"log": math.log, "atanh": math.atanh}


def _val(expr):
    return float(eval(expr, {"__builtins__": {}}, _NAMES))  # fixture is ours


def _arr(nested):
    if isinstance(nested, str):
        return _val(nested)
    return [_arr(x) for x in nested]


def _cases():
    with open(_PATH) as f:
        return json.load(f)["cases"]


def _kwargs(args):
    kw = {"scale": _val(args["scale"])}
    if args.get("causal"):
        kw["causal"] = True
    if "window" in args:
        kw["window"] = tuple(args["window"])
    if "softcap" in args:
        kw["softcap"] = _val(args["softcap"])
    if "alibi_slopes" in args:
        kw["alibi_slopes"] = np.array(_arr(args["alibi_slopes"]))
    return kw


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_oracle_matches_hand_worked_example(case):
    q = np.array(_arr(case["q"]))[None]
    k = np.array(_arr(case["k"]))[None]
    v = np.array(_arr(case["v"]))[None]
    kw = _kwargs(case["args"])
    O, L = oracle.attention_fwd(q, k, v, **kw)
    np.testing.assert_allclose(O[0], np.array(_arr(case["O"])), rtol=0,
                               atol=1e-12)
    np.testing.assert_allclose(L[0], np.array(_arr(case["LSE"])), rtol=0,
                               atol=1e-12)
    if "dO" in case:
        do = np.array(_arr(case["dO"]))[None]
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, **kw)
        for got, key in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            np.testing.assert_allclose(got[0], np.array(_arr(case[key])),
                                       rtol=0, atol=1e-12, err_msg=key)


def test_fixture_is_well_formed():
    cases = _cases()
    assert len({c["name"] for c in cases}) == len(cases)
    for c in cases:
        assert c["cite"] and c["derivation"]
        Sq, Hq, D = np.array(_arr(c["q"])).shape
        Sk, Hkv, _ = np.array(_arr(c["k"])).shape
        assert np.array(_arr(c["v"])).shape == (Sk, Hkv, D)
        assert np.array(_arr(c["O"])).shape == (Sq, Hq, D)
        assert np.array(_arr(c["LSE"])).shape == (Hq, Sq)
