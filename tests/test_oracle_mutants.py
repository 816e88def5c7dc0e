"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case edits one expression of a copy of the oracle's source (a dropped
term, a wrong sign, index or operand, a missing scale, a wrong mask), loads the
edited copy as a throw-away module and runs every pin of tests/test_oracle.py
against it. At least one pin must fail. The unedited copy must pass them all,
so a failure is due to the planted mistake and not to the harness.
"""
import os
import types

import numpy as np
import pytest

import tests.test_oracle as pins

# mistakes such as an all-masked row produce NaN in worker threads on purpose
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPLICATED = os.path.join(ROOT, "oracle", "replicated.py")
SAMPLED = os.path.join(ROOT, "oracle", "sampled.py")
GROUPS = os.path.join(ROOT, "oracle", "groups.py")
TREE = os.path.join(ROOT, "oracle", "tree.py")


def _load(path, old=None, new=None, nth=1, inject=None):
    """Module from `path` with the nth occurrence of `old` replaced by `new`.
    inject: names to place in the module instead of its package-relative
    imports (which a stand-alone copy cannot resolve)."""
    src = open(path).read()
    if inject:
        src = "\n".join(l for l in src.split("\n") if not l.startswith("from ."))
    if old is not None:
        pos = -1
        for _ in range(nth):
            pos = src.find(old, pos + 1)
            assert pos >= 0, f"mutation site not found: {old!r} (occurrence {nth})"
        src = src[:pos] + new + src[pos + len(old):]
    mod = types.ModuleType("oracle_copy_" + os.path.basename(path)[:-3])
    mod.__dict__.update(inject or {})
    exec(compile(src, path, "exec"), mod.__dict__)
    return mod


def _pin_calls():
    calls = [(pins.test_oracle_matches_library_attention_and_autograd, (c,)) for c in pins.SMALL_CASES]
    calls += [
        (pins.test_n1_is_ordinary_causal_attention, ()),
        (pins.test_lse_against_softmax_output_with_identity_v, ()),
        (pins.test_scale_zero_closed_form, ((9, [7, 0, 3, 12], 4, 2, 8),)),
        (pins.test_scale_zero_closed_form, ((0, [5, 8], 2, 1, 4),)),
        (pins.test_constant_v, ()),
        (pins.test_finite_differences_of_packed_loss, ()),
        (pins.test_locality_and_prompt_invariance, ()),
        (pins.test_response_permutation, ()),
        (pins.test_replica_zero_gradient_split_gives_same_sums, ()),
        (pins.test_sampled_oracle_matches_replicated, ((13, [9, 0, 17, 4], 4, 2, 8),)),
        (pins.test_sampled_oracle_matches_replicated, ((0, [7, 11], 2, 1, 8),)),
        (pins.test_attended_keys_definition, ()),
        (pins.test_attended_keys_against_independent_definition, ()),
        (pins.test_group_oracle_matches_dense_masked_attention, (0,)),
        (pins.test_group_oracle_matches_dense_masked_attention, (1,)),
        (pins.test_group_oracle_one_group_is_the_single_group_oracle, ()),
        (pins.test_groups_are_isolated, ()),
        (pins.test_group_attended_keys_against_independent_definition, ()),
        (pins.test_tree_oracle_matches_dense_masked_attention, (0,)),
        (pins.test_tree_oracle_matches_dense_masked_attention, (1,)),
        (pins.test_one_level_tree_is_the_single_group_oracle, ()),
        (pins.test_tree_attended_keys_against_independent_definition, ()),
    ]
    return calls


def _failing_pins(monkeypatch, rep, smp, grp, tre):
    monkeypatch.setattr(pins, "oracle_fwd_bwd", rep.oracle_fwd_bwd)
    monkeypatch.setattr(pins, "rows_fwd_bwd", smp.rows_fwd_bwd)
    monkeypatch.setattr(pins, "keys_dkdv", smp.keys_dkdv)
    monkeypatch.setattr(pins, "attended_keys", smp.attended_keys)
    monkeypatch.setattr(pins, "oracle_groups_fwd_bwd", grp.oracle_groups_fwd_bwd)
    monkeypatch.setattr(pins, "attended_keys_groups", grp.attended_keys_groups)
    monkeypatch.setattr(pins, "group_starts", grp.group_starts)
    monkeypatch.setattr(pins, "oracle_tree_fwd_bwd", tre.oracle_tree_fwd_bwd)
    monkeypatch.setattr(pins, "attended_keys_tree", tre.attended_keys_tree)
    monkeypatch.setattr(pins, "segment_starts", tre.segment_starts)
    failed = []
    with np.errstate(all="ignore"):
        for fn, args in _pin_calls():
            try:
                fn(*args)
            except Exception:  # an assertion, or a crash the mistake causes
                failed.append(fn.__name__)
    return failed


# (file, old, new, occurrence): each a plausible slip in the oracle.
MUTANTS = {
    # replicated oracle
    "fwd_mask_drops_diagonal": (REPLICATED, "np.where(j <= i, S, -np.inf)", "np.where(j < i, S, -np.inf)", 1),
    "bwd_mask_drops_diagonal": (REPLICATED, "np.where(j <= i, S, -np.inf)", "np.where(j < i, S, -np.inf)", 2),
    "fwd_mask_reversed": (REPLICATED, "np.where(j <= i, S, -np.inf)", "np.where(j >= i, S, -np.inf)", 1),
    "lse_drops_max": (REPLICATED, "lse[r0:r1] = (m + np.log(l))[:, 0]", "lse[r0:r1] = np.log(l)[:, 0]", 1),
    "o_unnormalised": (REPLICATED, "Pm = E / l", "Pm = E", 1),
    "bwd_dS_sign": (REPLICATED, "dS = Pm * (dPm - (Pm * dPm)", "dS = Pm * (dPm + (Pm * dPm)", 1),
    "bwd_dS_drops_rowsum": (REPLICATED, "dS = Pm * (dPm - (Pm * dPm).sum(axis=1, keepdims=True))", "dS = Pm * dPm", 1),
    "bwd_dq_no_scale": (REPLICATED, "dq[r0:r1] = scale * (dS @ k[:r1])", "dq[r0:r1] = dS @ k[:r1]", 1),
    "bwd_dk_no_scale": (REPLICATED, "dk[:r1] += scale * (dS.T @ q[r0:r1])", "dk[:r1] += dS.T @ q[r0:r1]", 1),
    "bwd_dk_wrong_operand": (REPLICATED, "dk[:r1] += scale * (dS.T @ q[r0:r1])", "dk[:r1] += scale * (dS.T @ k[r0:r1])", 1),
    "bwd_dv_unnormalised": (REPLICATED, "dv[:r1] += Pm.T @ g", "dv[:r1] += E.T @ g", 1),
    "bwd_dP_wrong_operand": (REPLICATED, "dPm = g @ v[:r1].T", "dPm = g @ k[:r1].T", 1),
    "prompt_dO_not_split": (REPLICATED, "doh[:P] / N", "doh[:P]", 1),
    "prompt_dK_overwritten": (REPLICATED, "dK[:P, g] += dkn[:P]", "dK[:P, g] = dkn[:P]", 1),
    "prompt_dV_overwritten": (REPLICATED, "dV[:P, g] += dvn[:P]", "dV[:P, g] = dvn[:P]", 1),
    "prompt_dQ_overwritten": (REPLICATED, "dQ[:P, h] += dqn[:P]", "dQ[:P, h] = dqn[:P]", 1),
    "gqa_interleaved_groups": (REPLICATED, "for h in range(g * G, (g + 1) * G):", "for h in range(g, Hq, Hkv):", 1),
    "response_prompt_keys_reversed": (REPLICATED, "kn = np.concatenate([kg[:P], kg[seg]])", "kn = np.concatenate([kg[:P][::-1], kg[seg]])", 1),
    # packed-definition oracle
    "A_prompt_drops_diagonal": (SAMPLED, "return np.arange(0, t + 1)", "return np.arange(0, t)", 1),
    "A_response_sees_other_responses": (SAMPLED, "np.arange(o[n], t + 1)", "np.arange(P, t + 1)", 1),
    "A_response_misses_prompt_key": (SAMPLED, "np.concatenate([np.arange(0, P), np.arange(o[n], t + 1)])", "np.concatenate([np.arange(1, P), np.arange(o[n], t + 1)])", 1),
    "rows_dQ_no_scale": (SAMPLED, "dQ[i, hs] = scale * (dS @ KA)", "dQ[i, hs] = dS @ KA", 1),
    "rows_lse_drops_max": (SAMPLED, "LSE[hs, i] = (m + np.log(l))[:, 0]", "LSE[hs, i] = np.log(l)[:, 0]", 1),
    "keys_mask_drops_diagonal": (SAMPLED, "allowed = kidx[None, :] <= t", "allowed = kidx[None, :] < t", 1),
    "keys_dk_no_scale": (SAMPLED, "dk[hit] = scale * (dS[:, cols].T @ Qb)", "dk[hit] = dS[:, cols].T @ Qb", 1),
    "keys_skip_first_prompt_rows": (SAMPLED, "for r in range(lo, P, row_block)", "for r in range(lo + 1, P, row_block)", 1),
    "keys_gqa_one_head": (SAMPLED, "for h in range(kv_head * G, (kv_head + 1) * G)", "for h in range(kv_head * G, kv_head * G + 1)", 1),
    # several prompt groups
    "groups_start_not_advanced": (GROUPS, "s.append(s[-1] + int(P) + sum(int(x) for x in L))", "s.append(int(P) + sum(int(x) for x in L))", 1),
    "groups_keys_not_shifted": (GROUPS, "return s[b] + attended_keys(t - s[b]", "return attended_keys(t - s[b]", 1),
    "groups_dK_from_dV": (GROUPS, 'out["dK"][a:e] = r["dK"]', 'out["dK"][a:e] = r["dV"]', 1),
    "groups_lse_shifted": (GROUPS, 'out["LSE"][:, a:e] = r["LSE"]', 'out["LSE"][:, a:e] = np.roll(r["LSE"], 1, axis=1)', 1),
    # multi-level prefix trees
    "tree_dO_not_split": (TREE, "1.0 / n_paths[x]", "1.0", 1),
    "tree_paths_without_root": (TREE, "paths.append(path[::-1])", "paths.append(path[::-1][1:] or path)", 1),
    "tree_keys_without_ancestors": (TREE, "parts = [np.arange(s[a], s[a + 1]) for a in anc[::-1]] + [np.arange(s[v], t + 1)]", "parts = [np.arange(s[v], t + 1)]", 1),
    "tree_dK_not_accumulated": (TREE, "np.add.at(dK[:, g], idx, dkn)", "dK[idx, g] = dkn", 1),
}


def _load_all(path=None, old=None, new=None, nth=1):
    rep = _load(REPLICATED, old, new, nth) if path == REPLICATED else _load(REPLICATED)
    smp = _load(SAMPLED, old, new, nth) if path == SAMPLED else _load(SAMPLED)
    inj = {"oracle_fwd_bwd": rep.oracle_fwd_bwd, "attended_keys": smp.attended_keys}
    grp = (_load(GROUPS, old, new, nth, inject=inj) if path == GROUPS
           else _load(GROUPS, inject=inj))
    tinj = {"causal_attention_fwd": rep.causal_attention_fwd, "causal_attention_bwd": rep.causal_attention_bwd}
    tre = (_load(TREE, old, new, nth, inject=tinj) if path == TREE else _load(TREE, inject=tinj))
    return rep, smp, grp, tre


def test_unedited_copy_passes_every_pin(monkeypatch):
    assert _failing_pins(monkeypatch, *_load_all()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(monkeypatch, name):
    path, old, new, nth = MUTANTS[name]
    failed = _failing_pins(monkeypatch, *_load_all(path, old, new, nth))
    assert failed, f"no pin catches the planted mistake {name}"
