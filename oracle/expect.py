"""Closed forms of the Module 11 lecture used as pins (oracle). Test infrastructure only.

* §6 "Expected progress per cycle": with the same conditional acceptance
  probability alpha at every reached position and gamma drafted tokens, a
  cycle emits E = 1 + alpha + ... + alpha^gamma = (1 - alpha^(gamma+1))/(1 - alpha)
  tokens on average (gamma + 1 when alpha = 1).
* §7: in general E = 1 + sum_k prod_{i<=k} a_i (a tail sum over the
  conditional rates a_i), and the first-order speed scenario is
  S = E / (1 + gamma c).
* §1: the weight-streaming ceiling Q <= BW / W.
"""
from __future__ import annotations


def expected_tokens(alpha: float, gamma: int) -> float:
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def expected_tokens_tail(rates) -> float:
    total, prod = 1.0, 1.0
    for a in rates:
        prod *= a
        total += prod
    return total


def speed(alpha: float, gamma: int, c: float) -> float:
    return expected_tokens(alpha, gamma) / (1.0 + gamma * c)


def weight_stream_ceiling(bandwidth_bytes_per_s: float, bytes_per_step: float) -> float:
    return bandwidth_bytes_per_s / bytes_per_step
