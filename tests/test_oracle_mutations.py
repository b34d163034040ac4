"""Plants plausible mistakes in the oracle (on the CPU) and checks that the
pins in test_oracle_pins.py catch each one."""
import numpy as np
import pytest

from oracle import moe_oracle as O
import tests.test_oracle_pins as P


def _swapped_gate_up(xrows, w13, w2, act, act_quant=None, h_fp8=None):
    I = w13.shape[0] // 2
    return O.__dict__["_orig_gated_ffn"](xrows, np.concatenate([w13[I:], w13[:I]]), w2, act, act_quant, h_fp8)


def _fails(fn, *a, **k):
    with pytest.raises(AssertionError):
        fn(*a, **k)


def test_swapped_gate_and_up_is_caught(monkeypatch):
    monkeypatch.setitem(O.__dict__, "_orig_gated_ffn", O.gated_ffn)
    monkeypatch.setattr(O, "gated_ffn", _swapped_gate_up)
    _fails(P.test_brute_force_all_experts_then_mask, 17, 32, 5, 3, 16, "silu")


def test_highest_index_tie_break_is_caught(monkeypatch):
    def bad_topk(z, k):
        z = np.asarray(z, dtype=np.float64)
        E = z.shape[-1]
        return (E - 1 - np.argsort(-z[..., ::-1], axis=-1, kind="stable"))[..., :k]
    monkeypatch.setattr(O, "select_topk", bad_topk)
    _fails(P.test_topk_brute_force_with_ties_and_signed_zero)


def test_missing_renorm_is_caught(monkeypatch):
    orig = O.route
    monkeypatch.setattr(O, "route", lambda z, k, renormalize=True, per_expert_scale=None, *rest:
                        orig(z, k, False, per_expert_scale, *rest))
    _fails(P.test_closed_form_softmax_over_selected, 8, 2)
    _fails(P.test_worked_example_from_page)


def test_scale_indexed_by_slot_is_caught(monkeypatch):
    orig = O.route

    def bad(z, k, renormalize=True, per_expert_scale=None, *rest):
        w, ids = orig(z, k, renormalize, None, *rest)
        if per_expert_scale is not None:
            w = w * np.asarray(per_expert_scale)[:k][None, :]
        return w, ids
    monkeypatch.setattr(O, "route", bad)
    _fails(P.test_scale_fold_identity)


def test_softmax_over_selected_only_is_caught_without_renorm(monkeypatch):
    def bad_softmax(z):
        z = np.asarray(z, dtype=np.float64)
        e = np.exp(z - z.max(axis=-1, keepdims=True))
        return e / e.max(axis=-1, keepdims=True)
    monkeypatch.setattr(O, "softmax_all", bad_softmax)
    _fails(P.test_no_renorm_is_full_softmax_gathered, 8, 2)


def test_dropped_cubic_term_in_gelu_is_caught(monkeypatch):
    monkeypatch.setattr(O, "gelu_tanh", lambda a: 0.5 * a * (1 + np.tanh(np.sqrt(2 / np.pi) * a)))
    monkeypatch.setitem(O.ACTIVATIONS, "gelu_tanh", O.gelu_tanh)
    _fails(P.test_activations_match_torch)


def test_group_score_by_sum_is_caught(monkeypatch):
    def bad(z, n_groups, topk_groups):
        z = np.asarray(z, dtype=np.float64)
        T, E = z.shape
        gsz = E // n_groups
        picked = np.argsort(-z.reshape(T, n_groups, gsz).sum(-1), axis=-1, kind="stable")[:, :topk_groups]
        m = np.zeros((T, n_groups), dtype=bool)
        np.put_along_axis(m, picked, True, axis=-1)
        return np.repeat(m, gsz, axis=-1)
    monkeypatch.setattr(O, "group_mask", bad)
    _fails(P.test_group_limited_worked_case)
    _fails(P.test_group_limited_topk_brute_force, 16, 4, 2, 3)


def test_higher_group_index_tie_break_is_caught(monkeypatch):
    orig = O.group_mask
    monkeypatch.setattr(O, "group_mask", lambda z, G, KG: orig(np.asarray(z)[:, ::-1], G, KG)[:, ::-1])
    _fails(P.test_group_limited_worked_case)


def test_sigmoid_sign_error_is_caught(monkeypatch):
    monkeypatch.setattr(O, "sigmoid_scores", lambda z: 1.0 / (1.0 + np.exp(np.asarray(z, dtype=np.float64))))
    _fails(P.test_sigmoid_scores_match_library_and_closed_forms)
    _fails(P.test_sigmoid_route_sorts_probabilities, True)


def test_fp8_scale_for_wrong_maximum_is_caught(monkeypatch):
    def bad(a):
        a = np.asarray(a, dtype=np.float32)
        scale = (np.abs(a).max(axis=-1) / np.float32(240.0)).astype(np.float32)
        scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
        return O.encode_e4m3fn((a / scale[:, None]).astype(np.float32)), scale
    monkeypatch.setattr(O, "quantize_rows_fp8", bad)
    _fails(P.test_dynamic_fp8_rows_properties)
    _fails(P.test_fp8_dynamic_ffn_matches_torch_composition)


def test_truncating_e4m3_encode_is_caught(monkeypatch):
    orig = O.encode_e4m3fn

    def bad(x):
        x = np.asarray(x, dtype=np.float32)
        c = orig(x)
        back = O.decode_e4m3fn(c)
        over = np.abs(back) > np.abs(x)  # rounded away from zero: step back (truncation)
        return np.where(over & ((c & 0x7F) > 0), c - 1, c).astype(np.uint8)
    monkeypatch.setattr(O, "encode_e4m3fn", bad)
    _fails(P.test_e4m3_encode_matches_torch_including_ties)


def test_h_quantised_without_bf16_rounding_is_caught(monkeypatch):
    monkeypatch.setattr(O, "round_bf16", lambda a: np.asarray(a, dtype=np.float64))
    _fails(P.test_fp8_dynamic_ffn_matches_torch_composition)


def test_block_tail_without_residual_is_caught(monkeypatch):
    orig = O.moe_layer

    def bad(x, layer, rows=None, logits=None):
        r = orig(x, dict(layer, block_tail=False), rows, logits)
        if layer.get("block_tail"):
            r["out"] = O.rmsnorm(r["out"], layer.get("gamma_post_ff"))  # residual dropped
        return r
    monkeypatch.setattr(O, "moe_layer", bad)
    _fails(P.test_gemma_branch_matches_torch_composition)


def test_swapped_mxfp4_nibbles_are_caught(monkeypatch):
    orig = O.decode_mxfp4
    monkeypatch.setattr(O, "decode_mxfp4",
                        lambda packed, scales: orig(((np.asarray(packed) & 15) << 4) | (np.asarray(packed) >> 4), scales))
    _fails(P.test_mxfp4_layer_equals_layer_on_torch_decoded_weights)


def test_e8m0_bias_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(O, "decode_e8m0", lambda c: np.where(np.asarray(c).astype(np.int64) == 255, np.nan,
                                                             np.ldexp(1.0, np.asarray(c).astype(np.int64) - 126)))
    _fails(P.test_e2m1_and_e8m0_decode_closed_forms)
    _fails(P.test_mxfp4_layer_equals_layer_on_torch_decoded_weights)


def test_mxfp4_scale_blocks_of_16_are_caught(monkeypatch):
    def bad(packed, scales):
        packed = np.asarray(packed).astype(np.int64)
        codes = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(packed.shape[:-1] + (2 * packed.shape[-1],))
        sc = O.decode_e8m0(scales)
        sc = np.repeat(sc, 16, axis=-1)                      # blocks of 16 ...
        sc = np.concatenate([sc, sc], axis=-1)[..., :codes.shape[-1]]  # ... padded to the row length
        return O.decode_e2m1(codes) * sc
    monkeypatch.setattr(O, "decode_mxfp4", bad)
    _fails(P.test_mxfp4_layer_equals_layer_on_torch_decoded_weights)


def test_unstable_permutation_is_caught(monkeypatch):
    orig = O.permutation

    def bad(ids, E):  # each expert's slots in descending flat order
        counts, offsets, order = orig(ids, E)
        order = np.concatenate([order[offsets[e]:offsets[e + 1]][::-1] for e in range(E)] or [order])
        return counts, offsets, order.astype(np.int64)
    monkeypatch.setattr(O, "permutation", bad)
    _fails(P.test_permutation_matches_stable_argsort, 33, 8, 2)


def test_gemma_router_without_the_hidden_size_factor_is_caught(monkeypatch):
    orig = O.router_input

    def bad(x, mode="plain", router_scale=None, eps=O.RMS_EPS):
        r = orig(x, mode, router_scale, eps)
        return r * np.sqrt(np.asarray(x).shape[-1]) if mode == "gemma" else r
    monkeypatch.setattr(O, "router_input", bad)
    _fails(P.test_router_input_has_unit_norm)
    _fails(P.test_gemma_branch_matches_torch_composition)


def test_scale_before_renormalisation_is_caught(monkeypatch):
    orig = O.route

    def bad(z, k, renormalize=True, per_expert_scale=None, *rest):
        w, ids = orig(z, k, False, None, *rest)
        if per_expert_scale is not None:
            w = w * np.asarray(per_expert_scale, dtype=np.float64)[ids]
        if renormalize:
            w = w / w.sum(axis=-1, keepdims=True)  # the scale is renormalised away
        return w, ids
    monkeypatch.setattr(O, "route", bad)
    _fails(P.test_scale_fold_identity)


def test_shared_experts_not_at_unit_weight_are_caught(monkeypatch):
    orig = O.moe_layer

    def bad(x, layer, rows=None, logits=None, h_fp8=None):
        sh = layer.get("shared")
        if sh is not None:  # shared experts at weight 1/2: their down projections halved
            sh = (sh[0], np.asarray(sh[1], dtype=np.float64) * 0.5)
        return orig(x, dict(layer, shared=sh), rows, logits, h_fp8)
    monkeypatch.setattr(O, "moe_layer", bad)
    _fails(P.test_two_shared_experts_equal_one_of_double_width)


def test_rmsnorm_eps_outside_the_root_is_caught(monkeypatch):
    def bad(x, gamma=None, eps=O.RMS_EPS):
        x = np.asarray(x, dtype=np.float64)
        y = x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)
        return y if gamma is None else y * np.asarray(gamma, dtype=np.float64)
    monkeypatch.setattr(O, "rmsnorm", bad)
    _fails(P.test_gemma_branch_matches_torch_composition)


def test_swapped_post_norm_weights_are_caught(monkeypatch):
    orig = O.moe_layer

    def bad(x, layer, rows=None, logits=None, h_fp8=None):
        d = layer.get("dense")
        if d is not None:
            d = dict(d, gamma_post1=d.get("gamma_post2"), gamma_post2=d.get("gamma_post1"))
        return orig(x, dict(layer, dense=d), rows, logits, h_fp8)
    monkeypatch.setattr(O, "moe_layer", bad)
    _fails(P.test_gemma_branch_matches_torch_composition)
