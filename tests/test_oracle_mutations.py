"""The oracle pins are strong enough: plant a plausible mistake in the oracle
(on the CPU, by monkeypatching one of its functions) and check that the
hand-derived example or the brute-force comparison fails."""
import numpy as np
import pytest

import oracle.misa_oracle as om
import test_oracle_pins as pins


def _fails(fn):
    try:
        fn()
    except Exception:    # an assertion, or a shape error the mistake causes
        return True
    return False


def _golden_both():
    pins.test_golden_handworked(False)
    pins.test_golden_handworked(True)


def _brute_some():
    for seed in (0, 2, 4):
        for B in (2, 3, 7):
            pins.test_oracle_vs_brute_force(seed, B)


def _dagger():
    pins.test_dagger_identities()


def mut_drop_tail(monkeypatch):
    monkeypatch.setattr(om, "tail_of", lambda keys, t, B: None)


def mut_strict_causal(monkeypatch):
    orig = om.score_query

    def bad(qt, wt, keys, t, heads, n_cols=None):
        out = orig(qt, wt, keys, t - 1, heads, n_cols)
        return out
    monkeypatch.setattr(om, "score_query", bad)


def mut_ties_high_id(monkeypatch):
    def bad(values, ids, count):
        order = np.argsort(-ids, kind="stable")
        v = values[order] + 0.0
        return order[np.argsort(-v, kind="stable")[:count]]
    monkeypatch.setattr(om, "top_positions", bad)


def mut_abs_weight(monkeypatch):
    orig = om.head_importance

    def bad(qt, wt, pooled, tail, t, B):
        return orig(qt, np.abs(wt), pooled, tail, t, B)
    monkeypatch.setattr(om, "head_importance", bad)


def mut_sum_pool(monkeypatch):
    def bad(keys, B):
        n_full = keys.shape[0] // B
        return np.stack([keys[m * B:(m + 1) * B].sum(axis=0) for m in range(n_full)]) if n_full \
            else np.zeros((0, keys.shape[1]))
    monkeypatch.setattr(om, "pool_full_blocks", bad)


def mut_block_offset(monkeypatch):
    # blocks aligned to the first query instead of the sequence start
    def bad(keys, B):
        sh = keys[1:]
        n_full = sh.shape[0] // B
        return np.stack([sh[m * B:(m + 1) * B].mean(axis=0) for m in range(n_full)]) if n_full \
            else np.zeros((0, keys.shape[1]))
    monkeypatch.setattr(om, "pool_full_blocks", bad)


def mut_fp8_bias(monkeypatch):
    orig = om.e4m3fn_to_f64
    monkeypatch.setattr(om, "e4m3fn_to_f64", lambda c: orig(c) * 0.5)


def mut_dagger_routed_heads(monkeypatch):
    def bad(qt, wt, keys, cand):
        out = np.full(len(cand), om.NEG_INF)
        ok = cand >= 0
        dots = qt[:2] @ keys[cand[ok]].T
        out[ok] = (wt[:2, None] * np.maximum(dots, 0.0)).sum(axis=0)
        return out
    monkeypatch.setattr(om, "score_candidates", bad)


def mut_relu_dropped(monkeypatch):
    def bad(qt, wt, keys, t, heads, n_cols=None):
        n_cols = keys.shape[0] if n_cols is None else n_cols
        out = np.full(n_cols, om.NEG_INF)
        heads = np.sort(np.asarray(heads))
        out[:t + 1] = (wt[heads][:, None] * (qt[heads] @ keys[:t + 1].T)).sum(axis=0)
        return out
    monkeypatch.setattr(om, "score_query", bad)


def mut_transposed_q(monkeypatch):
    # query t scored with the query of the previous row
    orig = om.SeqContext.score

    def bad(self, i, heads):
        return om.score_query(self.q[max(i - 1, 0)], self.w[i], self.keys, self.t(i), heads)
    monkeypatch.setattr(om.SeqContext, "score", bad)


MUTATIONS = [mut_drop_tail, mut_strict_causal, mut_ties_high_id, mut_abs_weight, mut_sum_pool,
             mut_block_offset, mut_fp8_bias, mut_dagger_routed_heads, mut_relu_dropped,
             mut_transposed_q]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_planted_oracle_mistake_is_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    caught = _fails(_golden_both) or _fails(_brute_some) or _fails(_dagger)
    assert caught, f"{mutation.__name__} passed every pin"
