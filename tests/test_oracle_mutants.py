"""Planted mistakes in the oracle (on the CPU only) must be caught by the pins.

Each mutant swaps one oracle function for a plausibly-wrong variant; at least
one pin test must then fail.  This shows the pins constrain the oracle rather
than restate it.
"""

import numpy as np
import pytest

from oracle import muon_oracle as orc
import tests.test_oracle_pins as pins

_ORIG_NS = orc.newton_schulz
_ORIG_NORM = orc.frobenius_normalise
_ORIG_MOM = orc.momentum_update
_ORIG_ORTHO = orc.orthogonalise
_ORIG_APPLY = orc.apply_update


def _ns_coeffs(a_f, b_f, c_f):
    def ns(X0, steps=5, a=orc.NS_A, b=orc.NS_B, c=orc.NS_C, record=False):
        return _ORIG_NS(X0, steps, a_f(a), b_f(b), c_f(c), record)
    return ns


def _ns_operand_swapped(X0, steps=5, a=orc.NS_A, b=orc.NS_B, c=orc.NS_C, record=False):
    X = np.asarray(X0, dtype=np.float64)
    its = [X]
    for _ in range(steps):
        A = X.T @ X                      # Gram on the wrong side
        B = b * A + c * (A @ A)
        X = a * X + B @ X                # shape error unless square; wrong if square
        its.append(X)
    return its if record else X


def _ns_wrong_order(X0, steps=5, a=orc.NS_A, b=orc.NS_B, c=orc.NS_C, record=False):
    X = np.asarray(X0, dtype=np.float64)
    its = [X]
    for _ in range(steps):
        A = X @ X.T
        X = a * X + b * A @ X + c * A @ X     # A^2 term dropped to A
        its.append(X)
    return its if record else X


def _norm_spectral(X, eps=orc.DEFAULT_EPS):
    X = np.asarray(X, dtype=np.float64)
    return X / (np.linalg.norm(X, 2) + eps)


def _mom_no_damp(M, G, mu=0.95, nesterov=True, form="ema"):
    M_new = mu * M + G if form == "ema" else mu * M + G
    U = G + mu * M_new if nesterov else M_new
    return M_new, U


def _mom_nesterov_old(M, G, mu=0.95, nesterov=True, form="ema"):
    M_new = mu * M + (1 - mu) * G
    U = (1 - mu) * G + mu * M if nesterov else M_new   # uses the old buffer
    return M_new, U


def _ortho_no_transpose_back(U, steps=5, eps=orc.DEFAULT_EPS, a=orc.NS_A, b=orc.NS_B, c=orc.NS_C):
    U = np.asarray(U, dtype=np.float64)
    if U.shape[0] > U.shape[1]:
        X = orc.newton_schulz(orc.frobenius_normalise(U.T, eps), steps, a, b, c)
        return X.reshape(U.shape)        # forgets to transpose back
    return _ORIG_ORTHO(U, steps, eps, a, b, c)


def _adam_no_bias_correction(W, G, M, V, t, lr=orc.DEFAULT_ADAM_LR, betas=orc.DEFAULT_ADAM_BETAS,
                             eps=orc.DEFAULT_ADAM_EPS, weight_decay=orc.DEFAULT_ADAM_WEIGHT_DECAY):
    b1, b2 = betas
    M1 = b1 * M + (1 - b1) * G
    V1 = b2 * V + (1 - b2) * G * G
    return W - lr * weight_decay * W - lr * M1 / (np.sqrt(V1) + eps), M1, V1


def _adam_eps_in_sqrt(W, G, M, V, t, lr=orc.DEFAULT_ADAM_LR, betas=orc.DEFAULT_ADAM_BETAS,
                      eps=orc.DEFAULT_ADAM_EPS, weight_decay=orc.DEFAULT_ADAM_WEIGHT_DECAY):
    b1, b2 = betas
    M1 = b1 * M + (1 - b1) * G
    V1 = b2 * V + (1 - b2) * G * G
    mh, vh = M1 / (1 - b1 ** t), V1 / (1 - b2 ** t)
    return W - lr * weight_decay * W - lr * mh / np.sqrt(vh + eps), M1, V1


def _adam_decay_after_update(W, G, M, V, t, lr=orc.DEFAULT_ADAM_LR, betas=orc.DEFAULT_ADAM_BETAS,
                             eps=orc.DEFAULT_ADAM_EPS, weight_decay=orc.DEFAULT_ADAM_WEIGHT_DECAY):
    b1, b2 = betas
    M1 = b1 * M + (1 - b1) * G
    V1 = b2 * V + (1 - b2) * G * G
    mh, vh = M1 / (1 - b1 ** t), V1 / (1 - b2 ** t)
    W1 = W - lr * mh / (np.sqrt(vh) + eps)
    return W1 - lr * weight_decay * W1, M1, V1


_ORIG_ADAM = orc.adamw_update


def _adam_betas_swapped(W, G, M, V, t, lr=orc.DEFAULT_ADAM_LR, betas=orc.DEFAULT_ADAM_BETAS,
                        eps=orc.DEFAULT_ADAM_EPS, weight_decay=orc.DEFAULT_ADAM_WEIGHT_DECAY):
    return _ORIG_ADAM(W, G, M, V, t, lr, (betas[1], betas[0]), eps, weight_decay)


def _muon_decay_after_update(W, O, lr, weight_decay, scale):
    W1 = _ORIG_APPLY(W, O, lr, 0.0, scale)
    return W1 - lr * weight_decay * W1


_ORIG_SCALE = orc.shape_scale


def _scale_rows_cols_exchanged(rows, cols, mode=orc.SCALE_ORIGINAL):
    return _ORIG_SCALE(cols, rows, mode) if mode == orc.SCALE_ORIGINAL else _ORIG_SCALE(rows, cols, mode)


def _scale_match_uses_min(rows, cols, mode=orc.SCALE_ORIGINAL):
    if mode == orc.SCALE_MATCH_RMS_ADAMW:
        return float(0.2 * np.sqrt(min(rows, cols)))
    return _ORIG_SCALE(rows, cols, mode)


def _scale_spectral_inverted(rows, cols, mode=orc.SCALE_ORIGINAL):
    if mode == orc.SCALE_SPECTRAL:
        return float(np.sqrt(cols / rows))
    return _ORIG_SCALE(rows, cols, mode)


MUTANTS = {
    "scale_spectral_inverted": ("shape_scale", _scale_spectral_inverted),
    "scale_rows_cols_exchanged": ("shape_scale", _scale_rows_cols_exchanged),
    "scale_match_rms_uses_min": ("shape_scale", _scale_match_uses_min),
    "muon_decay_after_update": ("apply_update", _muon_decay_after_update),
    "adam_no_bias_correction": ("adamw_update", _adam_no_bias_correction),
    "adam_eps_inside_sqrt": ("adamw_update", _adam_eps_in_sqrt),
    "adam_decay_after_update": ("adamw_update", _adam_decay_after_update),
    "adam_betas_swapped": ("adamw_update", _adam_betas_swapped),
    "b_sign_flipped": ("newton_schulz", _ns_coeffs(lambda a: a, lambda b: -b, lambda c: c)),
    "c_term_dropped": ("newton_schulz", _ns_coeffs(lambda a: a, lambda b: b, lambda c: 0.0)),
    "a_rounded": ("newton_schulz", _ns_coeffs(lambda a: 3.44, lambda b: b, lambda c: c)),
    "operand_swapped": ("newton_schulz", _ns_operand_swapped),
    "square_term_as_linear": ("newton_schulz", _ns_wrong_order),
    "spectral_normalisation": ("frobenius_normalise", _norm_spectral),
    "momentum_without_damping": ("momentum_update", _mom_no_damp),
    "nesterov_reads_old_buffer": ("momentum_update", _mom_nesterov_old),
    "tall_not_transposed_back": ("orthogonalise", _ortho_no_transpose_back),
}

PIN_TESTS = [
    lambda: [pins.test_closed_form_all_iterates(s) for s in [(4, 7), (24, 9), (33, 17)]],
    pins.test_orthogonalise_matches_closed_form_tall_and_wide,
    pins.test_worked_example,
    pins.test_quintic_band_after_five_steps,
    pins.test_polar_invariants,
    pins.test_transpose_equivariance,
    pins.test_momentum_geometric_series,
    pins.test_split_rows_blocks_are_independent,
    pins.test_update_decays_the_pre_update_weight,
    pins.test_shape_scale_rms_properties,
    pins.test_adamw_first_step_is_a_signed_step,
    pins.test_adamw_constant_gradient_keeps_the_signed_step,
    pins.test_adamw_first_moment_off_sees_every_gradient_alone,
    pins.test_adamw_decay_and_zero_lr,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = 0
    for t in PIN_TESTS:
        try:
            with np.errstate(all="ignore"):
                t()
        except (AssertionError, ValueError, np.linalg.LinAlgError):
            caught += 1
    assert caught >= 1, f"mutant {name} survived every pin"
