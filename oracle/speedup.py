"""Speculative speedup identity (oracle; test infrastructure only).

Sparse Glimpse page, "What carries the argument" and the referee summary of
Eq. (1)-(2): with speculation length k, acceptance rate alpha and relative
drafting cost gamma, the speedup is S = (alpha*k + 1) / (k*gamma + 1), and a
longer horizon helps only while alpha > gamma.

alpha is read as expected accepted drafts / k, so alpha*k + 1 is the expected
number of tokens per iteration (the bonus token included).
"""
from __future__ import annotations


def speedup(alpha: float, k: float, gamma: float) -> float:
    return (alpha * k + 1.0) / (k * gamma + 1.0)


def dspeedup_dk(alpha: float, k: float, gamma: float) -> float:
    """Derivative of the identity in k: (alpha - gamma) / (k*gamma + 1)^2."""
    return (alpha - gamma) / (k * gamma + 1.0) ** 2


def alpha_from_tokens_per_iter(tokens_per_iter: float, k: int) -> float:
    """Acceptance rate implied by tokens decoded per iteration (bonus token included)."""
    return (tokens_per_iter - 1.0) / k
