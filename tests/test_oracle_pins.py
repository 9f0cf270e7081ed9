"""The CPU oracle against facts fixed by the pages and by mathematics (no GPU)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_recurrent_oracle_pin(pin):
    pin(oracle.recurrent)


@pytest.mark.parametrize("pin", oracle_pins.KDA_PINS, ids=lambda p: p.__name__)
def test_recurrent_oracle_kda_pin(pin):
    pin(oracle.recurrent)


def test_kda_chunked_form_at_full_head_size():
    oracle_pins.pin_kda_chunked(oracle.recurrent, big=True)


def test_kda_forms_match_hand_example():
    oracle_pins.pin_kda_hand_example(oracle.bruteforce)
    for cs in (1, 2, 64):
        oracle_pins.pin_kda_hand_example(
            lambda *a, **kw: oracle.chunked(*a, **kw, chunk_size=cs))


def test_kda_rejects_bad_gate_shape():
    c = oracle_pins.random_case(41, [6], 1, 1, 4, 4, kda=True)
    c["g"] = c["g"][:, :, :3]
    with pytest.raises(ValueError):
        oracle.recurrent(**c)


@pytest.mark.parametrize("pin", oracle_pins.PROLOGUE_PINS, ids=lambda p: p.__name__)
def test_prologue_pin(pin):
    pin()


def test_chunked_form_at_full_head_size():
    # d = 128, chunk 64: the size at which the pages report ~1e-11 agreement
    oracle_pins.pin_chunked(oracle.recurrent, big=True)


def test_bruteforce_matches_hand_example():
    # the product form is itself checked against the hand-worked example
    oracle_pins.pin_hand_example(oracle.bruteforce)


def test_chunked_matches_hand_example():
    for cs in (1, 2, 64):
        oracle_pins.pin_hand_example(
            lambda *a, **kw: oracle.chunked(*a, **kw, chunk_size=cs))


def test_forward_substitution_inverse():
    rng = np.random.default_rng(0)
    A = np.tril(rng.standard_normal((64, 64)) * 0.3, k=-1)
    X = oracle.forward_substitution_inverse(A)
    assert np.max(np.abs(X @ (np.eye(64) + A) - np.eye(64))) < 1e-10
    assert np.allclose(np.triu(X, 1), 0.0) and np.allclose(np.diag(X), 1.0)


def test_decode_equals_one_token_prefill():
    c = oracle_pins.random_case(21, [1, 1, 1], 1, 2, 8, 8)
    o, fs = oracle.recurrent(**c)
    od, sd = oracle.decode_step(c["q"], c["k"], c["v"], c["g"], c["beta"], c["initial_state"])
    assert np.max(np.abs(od - o)) < 1e-13 and np.max(np.abs(sd - fs)) < 1e-13


def test_thread_count_does_not_change_results():
    c = oracle_pins.random_case(22, [50, 30], 2, 4, 16, 16)
    o1, s1 = oracle.recurrent(**c, nthreads=1)
    o4, s4 = oracle.recurrent(**c, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)


def test_rejects_bad_arguments():
    c = oracle_pins.random_case(23, [5], 2, 3, 4, 4)   # Hv % Hk != 0
    with pytest.raises(ValueError):
        oracle.recurrent(**c)
    c = oracle_pins.random_case(24, [5], 1, 1, 4, 4)
    c["cu_seqlens"] = np.array([0, 4])                  # does not end at T
    with pytest.raises(ValueError):
        oracle.recurrent(**c)
