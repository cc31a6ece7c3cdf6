"""The oracle on hand-derived worked examples stored under tests/golden.

The pages print no numeric example, so the fixtures are derived by hand from
their definitions; each fixture states its sources and derivation.
"""

import ast
import json
import math
import os
from fractions import Fraction

import numpy as np

from oracle import sla

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


_FUNCS = {"exp": math.exp, "sqrt": math.sqrt, "log": math.log}


def _value(expr):
    """Evaluate a fixture expression: numbers, + - * /, parentheses, exp/sqrt/log."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.BinOp) and isinstance(node.op, (ast.Add, ast.Sub, ast.Mult, ast.Div)):
            a, b = ev(node.left), ev(node.right)
            return {ast.Add: a + b, ast.Sub: a - b, ast.Mult: a * b,
                    ast.Div: a / b if b else math.inf}[type(node.op)]
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if isinstance(node, ast.Call) and isinstance(node.func, ast.Name) and node.func.id in _FUNCS:
            return _FUNCS[node.func.id](*[ev(a) for a in node.args])
        raise ValueError(f"unsupported expression {ast.dump(node)}")
    return ev(ast.parse(str(expr), mode="eval"))


def test_hand_example_three_way_split():
    g = _load("hand_sla3_2x2.json")
    q, k, v = (np.array(g[n], dtype=np.float64)[None, None] for n in ("q", "k", "v"))
    b = g["block"]
    nkb = sla.num_blocks(g["N"], b)
    keep, marg = Fraction(g["k_crit"], nkb), Fraction(g["k_marg"], nkb)
    cls, s, qp, kp = sla.class_map(q, k, b, "sla3", keep=keep, marg=marg)
    assert cls[0, 0].tolist() == g["cls"]
    o_s, lse, o_lin, o = sla.forward(q, k, v, cls, b)
    want_s = np.vectorize(_value)(np.array(g["o_s"], dtype=object)).astype(float)
    want_l = np.vectorize(_value)(np.array(g["o_lin"], dtype=object)).astype(float)
    want_lse = np.array([_value(x) for x in g["lse"]])
    np.testing.assert_allclose(o_s[0, 0], want_s, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o_lin[0, 0], want_l, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], want_s + want_l, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], want_lse, rtol=1e-14)


def test_page_settings_counts():
    g = _load("page_settings.json")
    nkb = sla.num_blocks(g["tokens_long_layer"], g["tile_tokens"])
    assert nkb == 1920
    for sp in g["sparsity_levels"]:
        keep = Fraction(1) - Fraction(str(sp))
        kc = sla.count_from_fraction(keep, nkb)
        # the kept share of tiles is exactly the stated complement of the sparsity
        assert Fraction(kc, nkb) == keep
