"""Planted mistakes: the oracle's pins must catch plausible errors in a scorer.

The pins of test_oracle_pins.py are functions of the scoring routine they
check.  Here they run against a plain numpy restatement of the score formula
(Strata pull request #228, part 1, first paragraph:
score(t, b) = sum_h relu(sum_i k_b[i] * q_{t,h}[i]), with S and B from the
same page's arithmetic contract), once as written and once per planted
mistake.  The restatement as written must pass every pin; each mistake must
fail at least one.  This shows that the pins would notice such a mistake in
the C oracle itself, not only that the oracle passes them.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from test_oracle_pins import (load_hand_examples, pin_coded_fixture, pin_exact_bruteforce,
                              pin_f32_queries, pin_hand_example, pin_integer_fixture,
                              pin_invariants, pin_single_head_matmul, pin_trivial_closed_forms)


def _as_f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.float32:
        return x.astype(np.float64)
    return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)


def numpy_scores(q, kblk, nb, mistake: str | None = None) -> oracle.Scores:
    """The score, S and B of every row r = g*nq + t and block b < nb, in
    float64 numpy, with an optional planted mistake."""
    Q = _as_f64(np.ascontiguousarray(q))            # [nq][G][H][D]
    K = _as_f64(np.ascontiguousarray(kblk))[:, :nb]  # [G][nb][D]
    nq, G, H, D = Q.shape
    if mistake == "transposed_head_index" and G > 1:
        # q-head read as h*G + g instead of g*H + h
        Q = Q.reshape(nq, H * G, D).reshape(nq, H, G, D).transpose(0, 2, 1, 3)
    if mistake == "off_by_one_block" and nb > 1:
        K = np.roll(K, -1, axis=1)
    if mistake == "dropped_channel":
        Q = Q.copy()
        Q[..., D - 1] = 0.0
    prod = Q[:, :, :, None, :] * K[None, :, None, :, :]   # [nq][G][H][nb][D]
    if mistake == "fp16_accumulation":
        d = np.zeros(prod.shape[:-1], dtype=np.float16)
        with np.errstate(over="ignore", invalid="ignore"):
            for i in range(D):
                d = (d + prod[..., i].astype(np.float16)).astype(np.float16)
        d = d.astype(np.float64)
    else:
        d = prod.sum(axis=-1)                              # [nq][G][H][nb]
    if mistake == "flipped_sign":
        d = -d
    if mistake == "dropped_head" and H > 1:
        d = d[:, :, :-1]
    if mistake == "relu_after_head_sum":
        sc = np.maximum(d.sum(axis=2), 0.0)
    elif mistake == "no_relu":
        sc = d.sum(axis=2)
    elif mistake == "abs_instead_of_relu":
        sc = np.abs(d).sum(axis=2)
    else:
        sc = np.maximum(d, 0.0).sum(axis=2)                # [nq][G][nb]
    if mistake == "S_of_the_sum":
        S = np.abs(d).sum(axis=2)
    else:
        S = np.abs(prod).sum(axis=(2, 4))
    sc = sc.transpose(1, 0, 2).reshape(G * nq, nb)
    S = S.transpose(1, 0, 2).reshape(G * nq, nb)
    rel = oracle.BOUND_REL * (2.0 if mistake == "loose_bound" else 1.0)
    B = rel * S + (0.0 if mistake == "bound_without_abs_term" else oracle.BOUND_ABS) * sc
    return oracle.Scores(sc, S, B, np.arange(G * nq, dtype=np.int64))


MISTAKES = ["transposed_head_index", "off_by_one_block", "dropped_channel", "fp16_accumulation",
            "flipped_sign", "dropped_head", "relu_after_head_sum", "no_relu",
            "abs_instead_of_relu", "S_of_the_sum", "loose_bound", "bound_without_abs_term"]


def run_pins(scores_fn) -> list[str]:
    """Names of the pins that fail for scores_fn."""
    pins = [(f"bruteforce_{s}", lambda f, s=s: pin_exact_bruteforce(f, s)) for s in range(12)]
    pins += [("single_head_matmul", pin_single_head_matmul), ("coded", pin_coded_fixture),
             ("integer", pin_integer_fixture), ("trivial", pin_trivial_closed_forms),
             ("invariants", pin_invariants), ("f32_queries", pin_f32_queries)]
    pins += [(f"hand_{ex['name']}", lambda f, ex=ex: pin_hand_example(f, ex))
             for ex in load_hand_examples()]
    failed = []
    for name, pin in pins:
        try:
            pin(scores_fn)
        except (AssertionError, ArithmeticError, ValueError):
            # a pin that cannot even evaluate the result (an overflow to
            # infinity, a shape that does not match) fails too
            failed.append(name)
    return failed


def test_numpy_restatement_passes_every_pin():
    assert run_pins(numpy_scores) == []


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mistake_fails_a_pin(mistake):
    failed = run_pins(lambda q, k, nb: numpy_scores(q, k, nb, mistake))
    assert failed, f"no pin catches {mistake}"
