"""Hand-derived closed-form cases (tests/golden/hand_worked.json) against the oracle (CPU)."""
import ast
import json
import math
import operator
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
    GOLD = json.load(f)

_NAMES = {"ln2": math.log(2.0), "ln3": math.log(3.0)}
_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul, ast.Div: operator.truediv,
        ast.USub: operator.neg}


def ev(expr):
    """Evaluate a fixture expression: numbers, ln2, ln3, + - * / and parentheses only."""
    def go(node):
        if isinstance(node, ast.Expression):
            return go(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.Name) and node.id in _NAMES:
            return _NAMES[node.id]
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](go(node.left), go(node.right))
        if isinstance(node, ast.UnaryOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](go(node.operand))
        raise ValueError("unsupported fixture expression: " + expr)
    return go(ast.parse(str(expr), mode="eval"))


@pytest.mark.parametrize("case", GOLD["cases"], ids=[c["name"] for c in GOLD["cases"]])
def test_hand_worked(orc, case):
    L = len(case["u"])
    N = case["N"]
    y, h = orc.scan(
        np.array(case["u"], float).reshape(1, 1, L),
        np.array(case["delta"], float).reshape(1, 1, L),
        np.array(case["A"], float).reshape(1, N),
        np.array(case["B"], float).reshape(1, N, L),
        np.array(case["C"], float).reshape(1, N, L),
        D=np.array([case["D"]], float),
        z=None if case["z"] is None else np.array([ev(v) for v in case["z"]]).reshape(1, 1, L),
        delta_bias=np.array([case["bias"]], float),
        zoh=case["zoh"], reverse=case["reverse"])
    np.testing.assert_allclose(y[0, 0], [ev(v) for v in case["y"]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(h[0, 0], [ev(v) for v in case["final_state"]], rtol=1e-14, atol=1e-15)


with open(os.path.join(HERE, "golden", "conv_hand_worked.json")) as f:
    CONV_GOLD = json.load(f)


@pytest.mark.parametrize("case", CONV_GOLD["cases"], ids=[c["name"] for c in CONV_GOLD["cases"]])
def test_conv_hand_worked(orc, case):
    K = case["K"]
    x = np.array([ev(v) for v in case["x"]]).reshape(1, 1, -1)
    st = None if case["state"] is None else np.array(case["state"], float).reshape(1, 1, K - 1)
    u, so = orc.conv1d(x, np.array(case["w"], float).reshape(1, K), np.array([ev(case["bias"])]), st)
    np.testing.assert_allclose(u[0, 0], [ev(v) for v in case["u"]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(so[0, 0], [ev(v) for v in case["state_out"]], rtol=1e-14, atol=1e-15)
