"""The oracle pins must catch plausible mistakes. Each mutant below is a wrong version of the
oracle's step (planted here, on the CPU, never in the product); every mutant must make at
least one pin in test_oracle_pins fail."""
import numpy as np
import pytest

import oracle.kda as ok
import tests.test_oracle_pins as pins


def _m_readout_before_update(S, q, k, v, a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    Sd = a[..., :, None] * S
    u = np.einsum("...ij,...i->...j", Sd, k)
    o = np.einsum("...ij,...i->...j", Sd, q)
    return Sd + b[..., None, None] * (k[..., :, None] * (v - u)[..., None, :]), o


def _m_decay_after_delta(S, q, k, v, a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    u = np.einsum("...ij,...i->...j", S, k)
    Sn = a[..., :, None] * (S + b[..., None, None] * (k[..., :, None] * (v - u)[..., None, :]))
    return Sn, np.einsum("...ij,...i->...j", Sn, q)


def _m_undecayed_prediction(S, q, k, v, a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    u = np.einsum("...ij,...i->...j", S, k)
    Sn = a[..., :, None] * S + b[..., None, None] * (k[..., :, None] * (v - u)[..., None, :])
    return Sn, np.einsum("...ij,...i->...j", Sn, q)


def _m_decay_on_value_axis(S, q, k, v, a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    dv = S.shape[-1]
    Sd = a[..., None, :dv] * S if a.shape[-1] >= dv else S
    u = np.einsum("...ij,...i->...j", Sd, k)
    Sn = Sd + b[..., None, None] * (k[..., :, None] * (v - u)[..., None, :])
    return Sn, np.einsum("...ij,...i->...j", Sn, q)


def _m_sign_flip(S, q, k, v, a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    Sd = a[..., :, None] * S
    u = np.einsum("...ij,...i->...j", Sd, k)
    Sn = Sd + b[..., None, None] * (k[..., :, None] * (v + u)[..., None, :])
    return Sn, np.einsum("...ij,...i->...j", Sn, q)


def _m_b_dropped_on_erase(S, q, k, v, a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    Sd = a[..., :, None] * S
    u = np.einsum("...ij,...i->...j", Sd, k)
    Sn = Sd + k[..., :, None] * (b[..., None] * v - u)[..., None, :]
    return Sn, np.einsum("...ij,...i->...j", Sn, q)


def _m_key_query_swapped(S, q, k, v, a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    Sd = a[..., :, None] * S
    u = np.einsum("...ij,...i->...j", Sd, q)
    Sn = Sd + b[..., None, None] * (k[..., :, None] * (v - u)[..., None, :])
    return Sn, np.einsum("...ij,...i->...j", Sn, q)


PINS = [pins.test_hand_derived_2x2, pins.test_scalar_geometric_series,
        pins.test_one_step_from_zero_reads_updated_state,
        pins.test_unit_key_readout_writes_value_exactly,
        pins.test_no_write_keeps_state_and_reads_it, pins.test_pure_decay_scales_key_rows,
        pins.test_transition_matrix_closed_form, pins.test_orthonormal_keys_overwrite_memory,
        pins.test_relaxed_kaczmarz_converges_to_least_squares]


@pytest.mark.parametrize("mutant", [_m_readout_before_update, _m_decay_after_delta,
                                    _m_undecayed_prediction, _m_decay_on_value_axis,
                                    _m_sign_flip, _m_b_dropped_on_erase, _m_key_query_swapped])
def test_some_pin_catches_mutant(mutant, monkeypatch):
    monkeypatch.setattr(ok, "kda_step", mutant)
    monkeypatch.setattr(pins, "kda_step", mutant)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError, np.linalg.LinAlgError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutant.__name__}"
