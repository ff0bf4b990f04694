"""The Newton-CG logistic-regression oracle against its pins, and copies of it with planted
mistakes that the pins must catch (no GPU)."""
import importlib.util
import os
import sys

import pytest

import oracle.logreg as lr
from logreg_checks import CHECKS

SRC = lr.__file__


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_logreg_oracle(check):
    check(lr)


# (name, original text, replacement): each mutant changes one spot of oracle/logreg.py
MUTATIONS = [
    ("sigmoid_of_minus_t", "np.where(t >= 0, 1.0 / (1.0 + e), e / (1.0 + e))",
     "np.where(t >= 0, e / (1.0 + e), 1.0 / (1.0 + e))"),
    ("loss_drops_label_term", "np.logaddexp(0.0, t) - np.asarray(c, np.float64) * t", "np.logaddexp(0.0, t)"),
    ("objective_drops_penalty", "+ 0.5 * lam * np.dot(w, w)", ""),
    ("curvature_is_p", "return p * (1.0 - p)", "return p"),
    ("curvature_misses_factor", "return p * (1.0 - p)", "return 0.5 * p * (1.0 - p)"),
    ("gradient_sign", "X.T @ (p - np.asarray(c, np.float64))", "X.T @ (np.asarray(c, np.float64) - p)"),
    ("gradient_drops_penalty", "+ lam * np.asarray(w, np.float64)", ""),
    ("hvp_drops_penalty", "return X.T @ (D * (X @ d)) + lam * d", "return X.T @ (D * (X @ d))"),
    ("hvp_drops_weights", "return X.T @ (D * (X @ d)) + lam * d", "return X.T @ (X @ d) + lam * d"),
    ("cg_first_direction_uphill", "    d = -r\n", "    d = r\n"),
    ("cg_residual_sign", "r = r + a * q", "r = r - a * q"),
    ("cg_beta_inverted", "b = rr_new / rr", "b = rr / rr_new"),
    ("cg_no_conjugation", "d = -r + b * d", "d = -r"),
    ("forcing_constant", "eps = min(cg_forcing, np.sqrt(gnorm)) * gnorm", "eps = cg_forcing * gnorm"),
    ("change_drops_cross_term", "lam * (a * np.dot(w, s) + 0.5 * a * a * np.dot(s, s))",
     "lam * (0.5 * a * a * np.dot(s, s))"),
    ("change_penalty_not_halved", "0.5 * a * a * np.dot(s, s)", "a * a * np.dot(s, s)"),
    ("armijo_wrong_sign", "if fa <= f0 + c1 * a * gs:", "if fa <= f0 - c1 * a * gs:"),
    ("margins_ignore_step", "t = t + a * xs", "t = t + xs"),
    ("iterate_ignores_step", "w = w + a * s", "w = w + s"),
    ("stops_on_absolute_gradient", "if gnorm <= grad_tol * g0:", "if gnorm <= grad_tol:"),
]


def _load_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, (name, src.count(old))
    path = os.path.join(str(tmp_path), "logreg_%s.py" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("logreg_%s" % name, path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod  # dataclasses look the module up by name
    try:
        spec.loader.exec_module(mod)
    finally:
        del sys.modules[spec.name]
    return mod


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_logreg_mutant_is_caught(mutation, tmp_path):
    name, old, new = mutation
    mod = _load_mutant(name, old, new, tmp_path)
    caught = []
    for check in CHECKS:
        try:
            check(mod)
        except Exception as e:  # an assertion, or a crash the mistake causes
            caught.append((check.__name__, type(e).__name__))
    assert caught, "mutant %s passes every pin" % name
