"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case swaps one internal step of the oracle for a plausible wrong version
(a dropped mask, a wrong index, a transposed operand, a wrong log base) and
re-runs one of the pinning checks, which must then fail.
"""
import numpy as np
import pytest

import oracle.attention_ref as att
import oracle.union_ref as uni
from tests import test_oracle_attention as ta
from tests import test_oracle_union as tu


def _no_causal(q_rows, k_sel, v_sel, keys, pos, scale):
    return att.__dict__["_orig"](q_rows, k_sel, v_sel, keys, np.full_like(pos, 1 << 40), scale)


def _swap_kv(q_rows, k_sel, v_sel, keys, pos, scale):
    return att.__dict__["_orig"](q_rows, v_sel, k_sel, keys, pos, scale)


def _wrong_scale(q_rows, k_sel, v_sel, keys, pos, scale):
    return att.__dict__["_orig"](q_rows, k_sel, v_sel, keys, pos, 1.0)


def _log2_lse(q_rows, k_sel, v_sel, keys, pos, scale):
    o, lse = att.__dict__["_orig"](q_rows, k_sel, v_sel, keys, pos, scale)
    return o, lse / np.log(2.0)


def _off_by_one_causal(q_rows, k_sel, v_sel, keys, pos, scale):
    return att.__dict__["_orig"](q_rows, k_sel, v_sel, keys, pos - 1, scale)


@pytest.mark.parametrize("mutant,check", [
    (_no_causal, lambda: ta.test_dense_case_matches_sdpa(1, 4, 1, 64, (1024,), (256,))),
    (_swap_kv, lambda: ta.test_dense_case_matches_sdpa(1, 4, 1, 64, (1024,), (256,))),
    (_wrong_scale, lambda: ta.test_dense_case_matches_sdpa(1, 4, 1, 64, (1024,), (256,))),
    (_log2_lse, ta.test_closed_form_zero_keys_gives_mean_of_values),
    (_off_by_one_causal, ta.test_single_admissible_key_returns_its_value),
])
def test_attention_mutants_are_caught(monkeypatch, mutant, check):
    monkeypatch.setitem(att.__dict__, "_orig", att._softmax_attend)
    monkeypatch.setattr(att, "_softmax_attend", mutant)
    with pytest.raises(AssertionError):
        check()


def test_union_group_mapping_mutant_is_caught(monkeypatch):
    real = uni.union_tables_ref

    def mutant(mask, H_kv, n_q_blocks, n_kv_blocks):
        # wrong head -> group mapping: h % H_kv instead of h // G
        mask = np.asarray(mask)
        perm = np.argsort(np.arange(mask.shape[1]) % H_kv, kind="stable")
        return real(mask[:, perm], H_kv, n_q_blocks, n_kv_blocks)

    monkeypatch.setattr(tu, "union_tables_ref", mutant)
    with pytest.raises(AssertionError):
        tu.test_group_mapping_consecutive_heads()
    with pytest.raises(AssertionError):
        tu.test_brute_force_seeded()


def test_union_ignores_extent_mutant_is_caught(monkeypatch):
    real = uni.union_tables_ref

    def mutant(mask, H_kv, n_q_blocks, n_kv_blocks):
        # cells outside the sequence's extent wrongly counted
        B, _, NQ_max, NKB_max = np.asarray(mask).shape
        return real(mask, H_kv, [NQ_max] * B, [NKB_max] * B)

    monkeypatch.setattr(tu, "union_tables_ref", mutant)
    with pytest.raises(AssertionError):
        tu.test_hand_worked_fixture()
