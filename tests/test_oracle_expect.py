"""Pins of the closed forms against every number the lecture prints for them."""
import pytest

from oracle import expect
from tests.conftest import golden


def test_expected_tokens_printed():
    g = golden("expected_tokens.json")
    for c in g["E"]:
        assert round(expect.expected_tokens(c["alpha"], c["gamma"]), c["decimals"]) == pytest.approx(c["value"])
    assert expect.expected_tokens(1.0, 4) == 5.0
    # the finite sum and the closed form agree
    for a in [0.1, 0.6, 0.8, 0.9, 0.99]:
        for gam in range(9):
            assert expect.expected_tokens(a, gam) == pytest.approx(sum(a ** k for k in range(gam + 1)), rel=1e-13)


def test_tail_sum_printed():
    g = golden("expected_tokens.json")
    for c in g["tail_sum"]:
        assert round(expect.expected_tokens_tail(c["rates"]), c["decimals"]) == pytest.approx(c["value"])


def test_speed_printed_and_argmax():
    g = golden("expected_tokens.json")
    for c in g["speed"]:
        assert round(expect.speed(c["alpha"], c["gamma"], c["c"]), c["decimals"]) == pytest.approx(c["value"])
    am = g["speed_argmax"]
    best = max(range(am["gammas"][0], am["gammas"][1] + 1), key=lambda gm: expect.speed(am["alpha"], gm, am["c"]))
    assert best == am["gamma_star"]
    # growth rule of section 7: S_{g+1} > S_g  <=>  alpha^(g+1) > c * S_g
    for gm in range(1, 10):
        grow = expect.speed(0.8, gm + 1, 0.1) > expect.speed(0.8, gm, 0.1)
        assert grow == (0.8 ** (gm + 1) > 0.1 * expect.speed(0.8, gm, 0.1))


def test_ceilings_and_scenarios_printed():
    g = golden("expected_tokens.json")
    for c in g["ceiling"]:
        assert round(expect.weight_stream_ceiling(c["bandwidth"], c["bytes"]), c["decimals"]) == pytest.approx(c["value"])
    bf16 = expect.weight_stream_ceiling(3.35e12, 16e9)
    fp4 = expect.weight_stream_ceiling(3.35e12, 4.5e9)
    vals = [bf16 * expect.speed(0.8, 5, 0.06),
            fp4 * expect.speed(0.875, 1, 0.05),
            fp4 * expect.speed(0.875, 1, 0.05 * 16 / 4.5)]
    for c, v in zip(g["scenario"], vals):
        assert round(v, c["decimals"]) == pytest.approx(c["value"])
