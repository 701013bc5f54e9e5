"""Planted mistakes in copies of the oracle: every one must fail a pin.

Each mutant below is a plausible slip in the oracle: a dropped term, a wrong
index, operand order or head mapping, a boundary off by one, a reversed tie
rule, a non-strict threshold.  The test writes a copy of the oracle package
with one mutation into a temporary directory (its C part is compiled there
with gcc), points the pin test modules at that copy and runs their pins until
one fails.  A mutant that passed every pin would mean the pins leave that part
of the oracle free.  An unmutated copy must pass them all.  CPU only: the
mistakes are planted in the oracle, never in the product library.
"""
import importlib.util
import os
import re

import pytest

import oracle
import test_oracle_attention as TA
import test_oracle_overlap as TO
import test_oracle_topk_policy as TP

ORACLE_DIR = os.path.dirname(os.path.abspath(oracle.__file__))

# (old, new) replacements in hylra_oracle.c; each `old` occurs exactly once.
C_MUTANTS = {
    "logit scale dropped": [
        ("      s[t] = scale * acc;", "      s[t] = acc;")],
    "query head mapped to the wrong KV head": [
        ("h = row % Hq, g = h / G;", "h = row % Hq, g = h % Hkv;")],
    "K tile read dimension-major": [
        ("  return ((page * Hkv + g) * ORACLE_BLOCK + tok) * d + c;",
         "  return ((page * Hkv + g) * d + c) * ORACLE_BLOCK + tok;")],
    "V sub-tile and lane swapped": [
        ("  const int64_t sub = tok / ORACLE_SUBTILE;",
         "  const int64_t sub = tok % (ORACLE_BLOCK / ORACLE_SUBTILE);"),
        ("         tok % ORACLE_SUBTILE;",
         "         tok / (ORACLE_BLOCK / ORACLE_SUBTILE);")],
    "last context token dropped": [
        ("    const int T = clamp_ctx(ctx[b], max_blocks);\n    double *s",
         "    const int T = clamp_ctx(ctx[b] - 1, max_blocks);\n    double *s")],
    "probabilities not normalised": [
        ("        const double p = exp(s[t] - m) / l;",
         "        const double p = exp(s[t] - m);")],
    "log-sum-exp without the max": [
        ("      lse[row] = m + log(l);", "      lse[row] = log(l);")],
    "sparse set of the wrong KV head": [
        ("if (sel[((int64_t)b * Hkv + g) * k + r] == n)",
         "if (sel[((int64_t)b * Hkv + (Hkv - 1 - g)) * k + r] == n)")],
    "block score over strided heads": [
        ("        for (int h = g * G; h < (g + 1) * G; ++h)",
         "        for (int h = g; h < Hq; h += Hkv)")],
    "block starts one token late": [
        ("for (int t = n * ORACLE_BLOCK; t < (n + 1) * ORACLE_BLOCK && t < T; ++t)",
         "for (int t = n * ORACLE_BLOCK + 1; t < (n + 1) * ORACLE_BLOCK && t < T; ++t)")],
    "ties go to the higher block id": [
        ("  if (g_sort_score[a] < g_sort_score[b]) return 1;\n  return (a > b) - (a < b);",
         "  if (g_sort_score[a] < g_sort_score[b]) return 1;\n  return (a < b) - (a > b);")],
    "selection emitted in score order": [
        ("      qsort(order, keff, sizeof(int), ascending_int);\n", "")],
    "smallest scores selected": [
        ("  if (g_sort_score[a] > g_sort_score[b]) return -1;\n"
         "  if (g_sort_score[a] < g_sort_score[b]) return 1;",
         "  if (g_sort_score[a] < g_sort_score[b]) return -1;\n"
         "  if (g_sort_score[a] > g_sort_score[b]) return 1;")],
    "selection padded with 0": [
        ("dst[r] = r < keff ? order[r] : -1;", "dst[r] = r < keff ? order[r] : 0;")],
}

# (old, new) replacements in the oracle's __init__.py.
PY_MUTANTS = {
    "softmax scale 1/d": [
        ("        scale = 1.0 / math.sqrt(d)", "        scale = 1.0 / d")],
    "threshold not strict": [
        ("        return (not force[j]) and M[j][i] > theta",
         "        return (not force[j]) and M[j][i] >= theta")],
    "forced layers may reuse": [
        ("        return (not force[j]) and M[j][i] > theta",
         "        return M[j][i] > theta")],
    "similarity matrix transposed": [
        ("        return (not force[j]) and M[j][i] > theta",
         "        return (not force[j]) and M[i][j] > theta")],
    "similarity ranked before resets": [
        ("    if a[0] != b[0]:\n        return a[0] < b[0]\n    return a[1] > b[1]",
         "    if a[1] != b[1]:\n        return a[1] > b[1]\n    return a[0] < b[0]")],
    "optimal reuse not taken on reconstruction": [
        ("acc_s + M[j + 1][i] + u[1] >= s_opt - SIM_TIE:",
         "acc_s + M[j + 1][i] + u[1] > s_opt + SIM_TIE:")],
    "reuse keeps the first reset's set": [
        ("            carried, margin = topk(score, layer[\"ctx\"], k)\n",
         "            fresh, margin = topk(score, layer[\"ctx\"], k)\n"
         "            carried = fresh if carried is None else carried\n")],
    "policy check accepts any earlier source": [
        ("    return all(s == j or s == src[j - 1] for j, s in enumerate(src) if j > 0)",
         "    return all(0 <= s <= j for j, s in enumerate(src) if j > 0)")],
    "overlap over the source set": [
        ("total += len(sets[p][i][s] & tgt) / len(tgt)",
         "total += len(sets[p][i][s] & tgt) / max(1, len(sets[p][i][s]))")],
    "empty target slices counted": [
        ("                    if not tgt:\n                        continue",
         "                    if not tgt:\n                        used += 1\n"
         "                        continue")],
}


def _pins():
    """The pins of the oracle, cheapest first (a mutant stops at its first
    failing pin)."""
    return [
        ("attention worked examples", TA.test_golden_worked_examples),
        ("attention closed forms", TA.test_closed_forms),
        ("top-k worked examples", TP.test_topk_golden),
        ("top-k special cases", TP.test_topk_special_cases),
        ("top-k vs lexsort", TP.test_topk_matches_lexsort),
        ("full attention vs sdpa", lambda: TA.test_full_matches_sdpa("f32")),
        ("sparse attention vs masked sdpa", TA.test_sparse_matches_masked_sdpa),
        ("sparse over all blocks equals full", TA.test_sparse_with_all_blocks_equals_full),
        ("block scores", TA.test_block_scores_sum_to_group_size_and_match_bruteforce),
        ("policy run: all reset equals full", TP.test_run_policy_all_reset_equals_full),
        ("policy run: k covering all blocks", TP.test_run_policy_k_covering_all_blocks_equals_full),
        ("policy run: reuse uses the source's set", TP.test_run_policy_reuse_uses_source_indices),
        ("policy run: malformed policies", TP.test_run_policy_rejects_malformed),
        ("policy worked examples", TP.test_policy_golden),
        ("policy closed forms", TP.test_policy_closed_forms),
        ("policy ties vs brute force", TP.test_policy_dp_ties_match_bruteforce),
        ("policy vs brute force", lambda: TP.test_policy_dp_matches_bruteforce(6.0)),
        ("overlap worked example", TO.test_overlap_golden),
        ("overlap sliding windows", TO.test_overlap_sliding_windows_closed_form),
        ("overlap padding and empty slices", TO.test_overlap_padding_and_empty_slices),
        ("overlap over the target set", TO.test_overlap_ratio_is_over_the_target_set),
        ("overlap identical and disjoint layers", TO.test_overlap_identical_and_disjoint_layers),
        ("overlap averages steps", TO.test_overlap_averages_steps),
    ]


def _copy(tmp_path, tag, c_edits=(), py_edits=()):
    """A copy of the oracle package with the given replacements, imported
    under its own name; its C library is compiled on first use."""
    d = tmp_path / ("oracle_copy_" + re.sub(r"\W+", "_", tag))
    d.mkdir()
    for fname, edits in (("hylra_oracle.c", c_edits), ("__init__.py", py_edits)):
        with open(os.path.join(ORACLE_DIR, fname)) as f:
            text = f.read()
        for old, new in edits:
            assert text.count(old) == 1, (tag, fname, old)
            text = text.replace(old, new)
        (d / fname).write_text(text)
    spec = importlib.util.spec_from_file_location(d.name, str(d / "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _failing_pin(copy, monkeypatch):
    for m in (TA, TP, TO):
        monkeypatch.setattr(m, "oracle", copy)
    for name, fn in _pins():
        try:
            fn()
        except (Exception, pytest.fail.Exception):
            return name
    return None


def test_unmutated_copy_passes_every_pin(tmp_path, monkeypatch):
    assert _failing_pin(_copy(tmp_path, "unmutated"), monkeypatch) is None


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_fails_a_pin(name, tmp_path, monkeypatch):
    pin = _failing_pin(_copy(tmp_path, name, c_edits=C_MUTANTS[name]), monkeypatch)
    assert pin is not None, "mutant %r passes every pin" % name


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_mutant_fails_a_pin(name, tmp_path, monkeypatch):
    pin = _failing_pin(_copy(tmp_path, name, py_edits=PY_MUTANTS[name]), monkeypatch)
    assert pin is not None, "mutant %r passes every pin" % name
