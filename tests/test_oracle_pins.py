"""The oracle against what the pages and the mathematics fix (CPU only)."""

import numpy as np
import pytest

from tests import pins

PINS = [
    pins.check_rms_closed_form,
    pins.check_rms_invariant,
    pins.check_bf16_vs_torch,
    pins.check_rope_hand_values,
    pins.check_rope_complex_form,
    pins.check_rope_relative,
    pins.check_mrope_degenerates,
    pins.check_mrope_sections,
    pins.check_mrope_single_component,
    pins.check_mrope_relative,
    pins.check_mrope_model_brute,
    pins.check_attention_closed_form,
    pins.check_attention_invariants,
    pins.check_gqa_equals_mha,
    pins.check_mlp_closed_form,
    pins.check_projection_orientation,
    pins.check_prefill_equals_steps,
    pins.check_input_projection,
    pins.check_bucket_copy_invariance,
    pins.check_code_predictor_recompute,
    pins.check_frame_input,
    pins.check_penalty_and_argmax,
    pins.check_sampling_inverse_cdf,
    pins.check_sampling_temperature,
    pins.check_sampling_topk,
    pins.check_sampling_top_p,
    pins.check_sampling_ties_and_penalty,
    pins.check_sampling_greedy_limit,
    pins.check_sampling_frequencies,
    pins.check_controls,
    pins.check_conv_causal,
    pins.check_transconv_phases,
    pins.check_quant_closed_form,
    pins.check_quant_error_bound,
    pins.check_quant_bytes_golden,
    pins.check_bucket_schedule_golden,
    pins.check_talker_bytes_golden,
    pins.check_run_lm_brute,
    pins.check_run_lm_asr_stress_golden,
    pins.check_run_talker_brute,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


@pytest.mark.parametrize("kv_bf16,qk_norm,bias,hq,hkv", [
    (False, True, True, 4, 2),    # Talker-like: GQA, QK norm
    (True, True, False, 4, 2),    # bf16 cache
    (True, False, True, 4, 4),    # ASR-like: MHA, q/k/v bias, no QK norm
    (False, True, False, 4, 1),   # one KV head
])
def test_cached_equals_recompute(kv_bf16, qk_norm, bias, hq, hkv):
    pins.check_cached_equals_recompute(kv_bf16, qk_norm, bias, hq, hkv)
