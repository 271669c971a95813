"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("L", [1, 2, 3])
def test_exhaustive_tiny(L):
    pins.check_exhaustive_tiny(oracle, L=L)


def test_random_int_all_chunks():
    for seed in range(3):
        pins.check_random_int_all_chunks(oracle, seed)


def test_chunk_phases():
    pins.check_chunk_phases(oracle)


def test_brute_force_float():
    pins.check_brute_force_float(oracle)


def test_association_orders():
    pins.check_association_orders(oracle)


def test_last_row():
    pins.check_last_row(oracle)


def test_causality():
    pins.check_causality(oracle)


def test_linearity_and_normalised_cases():
    pins.check_linearity_and_normalised_cases(oracle)


def test_query_scale_invariance():
    pins.check_query_scale_invariance(oracle)


def test_recurrent_vs_prefix_page_inputs():
    pins.check_recurrent_vs_prefix_page_inputs(oracle)


def test_resume():
    pins.check_resume(oracle)


def test_elu1():
    pins.check_elu1(oracle)


def test_favor_closed_form():
    pins.check_favor_closed_form(oracle)


def test_favor_convergence():
    pins.check_favor_convergence(oracle)


def test_decay_reduces_to_plain():
    pins.check_decay_reduces_to_plain(oracle)


def test_decay_forms_exact():
    pins.check_decay_forms_exact(oracle)


def test_decay_closed_forms():
    pins.check_decay_closed_forms(oracle)


def test_decay_phases():
    pins.check_decay_phases(oracle)


def test_decay_resume():
    pins.check_decay_resume(oracle)


def test_decay_forward():
    pins.check_decay_forward(oracle)


def test_softmax_reference():
    pins.check_softmax_reference(oracle)


def test_loglinear_buckets():
    pins.check_loglinear_buckets(oracle)


def test_loglinear_forms():
    pins.check_loglinear_forms(oracle)


def test_loglinear_causality():
    pins.check_loglinear_causality(oracle)


def test_loglinear_state():
    pins.check_loglinear_state(oracle)


def test_loglinear_resume():
    pins.check_loglinear_resume(oracle)


def test_apply_phi_in_scale():
    pins.check_apply_phi_in_scale(oracle)


def test_forward_scaled_favor_is_softmax():
    pins.check_forward_scaled_favor_is_softmax(oracle)


def test_forward_noncausal():
    pins.check_forward_noncausal(oracle)


def test_forward_causal_scaled():
    pins.check_forward_causal_scaled(oracle)


def test_over_heads():
    pins.check_over_heads(oracle)


def test_delta_page_example():
    pins.check_delta_page_example(oracle)


def test_delta_readback():
    pins.check_delta_readback(oracle)


def test_delta_orthogonal_keys():
    pins.check_delta_orthogonal_keys(oracle)


def test_delta_scalar_closed_form():
    pins.check_delta_scalar_closed_form(oracle)


def test_delta_forms():
    pins.check_delta_forms(oracle)


def test_delta_transform():
    pins.check_delta_transform(oracle)


def test_delta_causality_resume():
    pins.check_delta_causality_resume(oracle)
