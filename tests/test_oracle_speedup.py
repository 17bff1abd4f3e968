"""Pins for oracle.speedup: closed forms of the identity, its derivative against a
finite difference, and the acceptance rates implied by the Vegas page's Figure 10a."""
import json
import os

import pytest

from oracle import speedup as sp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vegas_fig10.json")


def test_closed_forms():
    assert sp.speedup(0.7, 0, 0.3) == 1.0                   # no speculation
    for k in range(1, 12):
        assert sp.speedup(1.0, k, 0.0) == k + 1              # free drafts, all accepted
        assert abs(sp.speedup(0.4, k, 0.4) - 1.0) < 1e-15    # alpha == gamma: break-even


@pytest.mark.parametrize("alpha,gamma", [(0.9, 0.1), (0.5, 0.6), (0.3, 0.3), (0.87, 0.05)])
def test_derivative_sign_and_value(alpha, gamma):
    for k in (1.0, 3.0, 8.0):
        h = 1e-6
        fd = (sp.speedup(alpha, k + h, gamma) - sp.speedup(alpha, k - h, gamma)) / (2 * h)
        d = sp.dspeedup_dk(alpha, k, gamma)
        assert abs(fd - d) < 1e-8
        if alpha > gamma:
            assert d > 0
        elif alpha < gamma:
            assert d < 0
        else:
            assert d == 0


def test_alpha_from_figure_10a():
    g = json.load(open(GOLDEN))
    q = g["tokens_per_iteration"]["Qwen3-8B"]
    o = g["tokens_per_iteration"]["gpt-oss-20b"]
    a_q = sp.alpha_from_tokens_per_iter(q["values"][-1], q["gamma"])
    a_o = sp.alpha_from_tokens_per_iter(o["values"][-1], o["gamma"])
    assert abs(a_q - (6.24 - 1) / 6) < 1e-12 and abs(a_q - 0.8733) < 1e-4
    assert abs(a_o - 0.906) < 1e-12
    # numerator of the identity recovers the tokens per iteration
    assert abs(a_q * q["gamma"] + 1 - 6.24) < 1e-12
    for vals in (q["values"], o["values"]):
        assert all(1.0 <= v <= 1 + q["gamma"] for v in vals)
