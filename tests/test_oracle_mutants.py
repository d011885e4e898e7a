"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake in the oracle (on the CPU, via monkeypatch) and checks that at least
one pin then fails."""
import numpy as np
import pytest

import oracle.dsa as od
import oracle.fp8 as of
import test_oracle_attn as ta
import test_oracle_cache as tc
import test_oracle_forward as tf
import test_oracle_fp8 as t8
import test_oracle_indexer as ti
import test_oracle_kl as tk
import test_oracle_topk as tt


def _fails(pins, golden_dir):
    for pin in pins:
        try:
            if "golden_dir" in pin.__code__.co_varnames[: pin.__code__.co_argcount]:
                pin(golden_dir)
            else:
                pin()
        except (AssertionError, IndexError, ValueError):
            return True
    return False


INDEXER_PINS = [ti.test_hand_example_exact, ti.test_fp8_dot_equals_integer_dot,
                ti.test_brute_force_python_loops, ti.test_scales_fold_through_relu]
TOPK_PINS = [tt.test_bruteforce_many_seeds, tt.test_hand_example, tt.test_zero_ties_lower_index_wins,
             tt.test_causal_range_and_padding]
ATTN_PINS = [ta.test_k_ge_L_equals_dense_causal, ta.test_zero_query_gives_mean_of_values,
             ta.test_single_index_gives_that_value_row, ta.test_permutation_invariance_and_duplicates]
FWD_PINS = [tf.test_chunked_prefill_equals_tail_of_full_prefill, tf.test_forward_with_k_ge_L_is_dense_causal]


def _no_relu(q_row, w_row, K, n_cand):
    out = np.full(K.shape[0], -np.inf)
    out[:n_cand] = w_row @ (q_row @ K[:n_cand].T)
    return out


def _causal_off_by_one(q_row, w_row, K, n_cand):
    return _ORIG_ROW(q_row, w_row, K, min(K.shape[0], n_cand + 1))


def _weights_after_sum(q_row, w_row, K, n_cand):
    out = np.full(K.shape[0], -np.inf)
    out[:n_cand] = w_row.sum() * np.maximum(q_row @ K[:n_cand].T, 0).mean(0)
    return out


_ORIG_ROW = od.index_scores_row
_ORIG_TOPK = od.topk_select_row
_ORIG_ATT = od.sparse_mqa_attention_row


def _ties_to_higher(row, k, n_cand):
    r = np.asarray(row, float)[:n_cand][::-1]
    sel = _ORIG_TOPK(r, k, n_cand)
    m = sel >= 0
    sel[m] = n_cand - 1 - sel[m]
    keep = np.sort(sel[m])
    out = np.full(k, -1)
    out[: keep.size] = keep
    return out


def _strict_past(row, k, n_cand):
    return _ORIG_TOPK(row, k, n_cand - 1)


def _value_from_tail(q_row, kv, idx_row, d_v, sm_scale):
    kv2 = np.concatenate([kv[:, d_v:], kv[:, :d_v]], axis=1)[:, : kv.shape[1]]
    o, _ = _ORIG_ATT(q_row, kv2, idx_row, d_v, sm_scale)
    _, lse = _ORIG_ATT(q_row, kv, idx_row, d_v, sm_scale)
    return o, lse


def _no_scale(q_row, kv, idx_row, d_v, sm_scale):
    return _ORIG_ATT(q_row, kv, idx_row, d_v, 1.0)


def _drop_duplicates(q_row, kv, idx_row, d_v, sm_scale):
    return _ORIG_ATT(q_row, kv, np.unique(np.asarray(idx_row)), d_v, sm_scale)


@pytest.mark.parametrize("mutant", [_no_relu, _causal_off_by_one, _weights_after_sum])
def test_indexer_mutants_caught(monkeypatch, golden_dir, mutant):
    monkeypatch.setattr(od, "index_scores_row", mutant)
    assert _fails(INDEXER_PINS + FWD_PINS, golden_dir)


def test_dequant_scale_mutant_caught(monkeypatch, golden_dir):
    monkeypatch.setattr(od, "dequantize", lambda c, s: of.e4m3_decode(c) * np.sqrt(np.asarray(s))[..., None])
    assert _fails(INDEXER_PINS, golden_dir)


def test_decode_bias_mutant_caught(monkeypatch, golden_dir):
    orig = of.e4m3_decode
    monkeypatch.setattr(t8, "e4m3_decode", lambda c: orig(c) * 0.5)
    assert _fails([t8.test_decode_exhaustive_matches_torch, t8.test_format_facts], golden_dir)


@pytest.mark.parametrize("mutant", [_ties_to_higher, _strict_past])
def test_topk_mutants_caught(monkeypatch, golden_dir, mutant):
    monkeypatch.setattr(od, "topk_select_row", mutant)
    assert _fails(TOPK_PINS, golden_dir)


@pytest.mark.parametrize("mutant", [_value_from_tail, _no_scale, _drop_duplicates])
def test_attention_mutants_caught(monkeypatch, golden_dir, mutant):
    monkeypatch.setattr(od, "sparse_mqa_attention_row", mutant)
    assert _fails(ATTN_PINS, golden_dir)


_ORIG_QUANT = of.quantize_rows


def _scale_447(x):
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(447.0), np.float32(1.0)).astype(np.float32)
    return of.e4m3_encode((x / scale[..., None]).astype(np.float64)), scale


def _truncating(x):
    codes, scale = _ORIG_QUANT(x)
    y = (np.asarray(x, np.float32) / scale[..., None]).astype(np.float64)
    dec = of.e4m3_decode(codes)
    # step toward zero wherever round-to-nearest went away from zero
    away = np.abs(dec) > np.abs(y)
    return np.where(away & ((codes & 0x7F) > 0), codes - 1, codes).astype(np.uint8), scale


@pytest.mark.parametrize("mutant", [_scale_447, _truncating])
def test_quantize_mutants_caught(monkeypatch, golden_dir, mutant):
    monkeypatch.setattr(tc, "quantize_rows", mutant)
    pins = [tc.test_largest_element_maps_to_448, tc.test_power_of_two_scale_invariance,
            tc.test_zero_rows, tc.test_half_step_error_bound, tc.test_matches_torch_composition]
    assert _fails(pins, golden_dir)


def test_append_position_mutant_caught(monkeypatch, golden_dir):
    orig = od.cache_append
    monkeypatch.setattr(tc.oracle, "cache_append",
                        lambda k, kv, kc, ks, kvc, pos: orig(k, kv, kc, ks, kvc, np.asarray(pos) + 1))
    assert _fails([tc.test_cache_append_bookkeeping], golden_dir)


_ORIG_KL = od._kl_terms


def _kl_grad_sign(I, p):
    loss, g = _ORIG_KL(I, p)
    return loss, -g


def _kl_reversed(I, p):
    I = np.asarray(I, float)
    p = np.asarray(p, float)
    q = np.exp(I - I.max())
    q /= q.sum()
    pos = (p > 0) & (q > 0)
    return float(np.sum(q[pos] * np.log(q[pos] / p[pos]))), q - p


def _kl_ignores_causal(I_row, p_row, n_cand):
    return od._kl_terms(I_row, p_row)


@pytest.mark.parametrize("mutant", [_kl_grad_sign, _kl_reversed])
def test_kl_term_mutants_caught(monkeypatch, golden_dir, mutant):
    monkeypatch.setattr(od, "_kl_terms", mutant)
    pins = [tk.test_matches_torch_kl_div_and_autograd, tk.test_one_hot_target_closed_form,
            tk.test_finite_differences]
    assert _fails(pins, golden_dir)


def test_kl_causal_mutant_caught(monkeypatch, golden_dir):
    monkeypatch.setattr(tk.oracle, "indexer_kl_dense_row", _kl_ignores_causal)
    assert _fails([tk.test_causal_range_and_unnormalised_target], golden_dir)


# ---- sparse attention backward
import test_oracle_attn_bwd as tb  # noqa: E402

BWD_PINS = [tb.test_central_finite_differences, tb.test_k_ge_L_equals_torch_autograd_of_dense_causal,
            tb.test_query_and_latent_gradients_identity, tb.test_one_distinct_token_closed_form]


def _bwd_variant(drop_value=False, no_centre=False, dq_unscaled=False, dkv_from_do=False,
                 dup_once=False, centre_sign=1.0):
    def row(q_row, kv, idx_row, do_row, d_v, sm_scale):
        N = kv.shape[0]
        idx_row = np.asarray(idx_row)
        sel = idx_row[(idx_row >= 0) & (idx_row < N)]
        H, d_qk = q_row.shape
        dkv = np.zeros((N, d_qk))
        if sel.size == 0:
            return np.zeros((H, d_qk)), dkv
        C = np.asarray(kv[sel], dtype=np.float64)
        z = sm_scale * (q_row @ C.T)
        P = np.exp(z - z.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dP = do_row @ C[:, :d_v].T
        D = np.sum(P * dP, axis=1, keepdims=True)
        dz = P * dP if no_centre else P * (dP - centre_sign * D)
        dq = (1.0 if dq_unscaled else sm_scale) * (dz @ C)
        src = np.concatenate([do_row, q_row[:, d_v:]], axis=1) if dkv_from_do else q_row
        dC = sm_scale * (dz.T @ src)
        if not drop_value:
            dC[:, :d_v] += P.T @ do_row
        if dup_once:
            dkv[sel] = dC
        else:
            np.add.at(dkv, sel, dC)
        return dq, dkv
    return row


@pytest.mark.parametrize("kw", [dict(drop_value=True), dict(no_centre=True), dict(dq_unscaled=True),
                                dict(dkv_from_do=True), dict(dup_once=True), dict(centre_sign=-1.0)])
def test_attention_bwd_mutants_caught(monkeypatch, golden_dir, kw):
    # the unmodified variant passes every pin
    monkeypatch.setattr(od, "sparse_mqa_attention_bwd_row", _bwd_variant())
    assert not _fails(BWD_PINS, golden_dir)
    monkeypatch.setattr(od, "sparse_mqa_attention_bwd_row", _bwd_variant(**kw))
    assert _fails(BWD_PINS, golden_dir)


# ---- sparse attention, MHA mode
import test_oracle_mha as tm  # noqa: E402

MHA_PINS = [tm.test_absorption_equals_mqa_mode, tm.test_k_ge_L_equals_dense_causal_mha,
            tm.test_single_index_gives_that_heads_value_row, tm.test_keys_values_shapes_and_shared_rope]
_ORIG_KV = od.mha_keys_values
_ORIG_MHA_ROW = od.sparse_mha_attention_row


def _kv_no_rope(kv, w_uk, w_uv, d_c):
    K, V = _ORIG_KV(kv, w_uk, w_uv, d_c)
    K = K.copy()
    K[:, :, w_uk.shape[1]:] = 0.0
    return K, V


def _kv_head0_keys(kv, w_uk, w_uv, d_c):
    return _ORIG_KV(kv, np.broadcast_to(w_uk[:1], w_uk.shape), w_uv, d_c)


def _kv_values_next_head(kv, w_uk, w_uv, d_c):
    return _ORIG_KV(kv, w_uk, np.roll(w_uv, 1, axis=0), d_c)


def _mha_no_scale(q_row, K, V, idx_row, sm_scale):
    return _ORIG_MHA_ROW(q_row, K, V, idx_row, 1.0)


def _mha_drop_duplicates(q_row, K, V, idx_row, sm_scale):
    return _ORIG_MHA_ROW(q_row, K, V, np.unique(np.asarray(idx_row)), sm_scale)


@pytest.mark.parametrize("mutant", [_kv_no_rope, _kv_head0_keys, _kv_values_next_head])
def test_mha_keys_values_mutants_caught(monkeypatch, golden_dir, mutant):
    monkeypatch.setattr(od, "mha_keys_values", mutant)
    assert _fails(MHA_PINS, golden_dir)


@pytest.mark.parametrize("mutant", [_mha_no_scale, _mha_drop_duplicates])
def test_mha_row_mutants_caught(monkeypatch, golden_dir, mutant):
    monkeypatch.setattr(od, "sparse_mha_attention_row", mutant)
    assert _fails(MHA_PINS, golden_dir)
