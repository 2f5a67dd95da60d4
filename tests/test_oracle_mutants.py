"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
at least one pin catches each of them.  The copies live in a temporary
directory; the real oracle is untouched."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
from oracle import build as oracle_build

SRC = os.path.join(os.path.dirname(oracle.__file__), "vpa_ref.c")

# (name, exact text in vpa_ref.c, replacement)
MUTANTS = [
    ("tie_goes_to_highest_id",
     "    if (a == b)\n        return ia < ib;", "    if (a == b)\n        return ia > ib;"),
    ("nan_loses",
     "    if (a_nan)\n        return 1;", "    if (a_nan)\n        return 0;"),
    ("nan_tie_highest_id",
     "    if (a_nan && b_nan)\n        return ia < ib;", "    if (a_nan && b_nan)\n        return ia > ib;"),
    ("signed_zeros_differ",
     "    if (a == b)\n        return ia < ib;",
     "    if (a == b && signbit(a) != signbit(b))\n        return signbit(b) != 0;\n"
     "    if (a == b)\n        return ia < ib;"),
    ("subnormals_flushed",
     "    return (double)f;", "    return fpclassify(f) == FP_SUBNORMAL ? 0.0 : (double)f;"),
    ("bf16_not_widened",
     "        return (uint32_t)h << 16;", "        return (uint32_t)h << 15;"),
    ("padding_not_masked_in_argmax",
     "        for (int64_t c = 1; c < vocab; ++c) {", "        for (int64_t c = 1; c < ld; ++c) {"),
    ("padding_not_masked_in_stats",
     "                if (hi > vocab)\n                    hi = vocab;", ""),
    ("shard_local_blocks",
     "                int64_t b = shard_lo / block + j;\n                int64_t lo = b * block, hi = lo + block;",
     "                int64_t lo = shard_lo + (int64_t)j * block, hi = lo + block;"),
    ("slot_count_short",
     "        if (last - first + 1 > m)\n            m = last - first + 1;",
     "        if (last - first > m)\n            m = last - first;"),
    ("combine_by_value_only",
     "            if (ref_better(ref_value(st.val_bits), st.id, ref_value(best.val_bits), best.id))\n                best = st;\n        }\n    return best;",
     "            if (ref_value(st.val_bits) > ref_value(best.val_bits))\n                best = st;\n        }\n    return best;"),
    ("accept_counts_all_matches",
     "        while (n < k && draft[n] == target[n])\n            ++n;",
     "        for (int32_t q = 0; q < k; ++q)\n            n += draft[q] == target[q];"),
    ("correction_is_draft",
     "        out[j] = j < n ? draft[j] : (j == n ? target[j] : -1);",
     "        out[j] = j < n ? draft[j] : (j == n ? (j < k ? draft[j] : target[j]) : -1);"),
    ("rejected_off_by_one",
     "    *n_rejected = k - n;", "    *n_rejected = k - n + 1;"),
    ("ragged_rows_without_request_offset",
     "        int64_t base = (int64_t)cu[r] + r;\n        int32_t tgt[k + 1];\n        uint32_t vb;",
     "        int64_t base = (int64_t)cu[r];\n        int32_t tgt[k + 1];\n        uint32_t vb;"),
    ("ragged_stats_bonus_from_draft_rows",
     "        tgt[k] = ref_combine_row(bonus_stats, n_shards, n_req, r, m_bonus).id;\n        if (prefilling",
     "        tgt[k] = k ? tgt[k - 1] : 0;\n        if (prefilling"),
    ("prefilling_flag_ignored",
     "            vpa_ref_argmax(row, dtype, ld, 1, vocab, &tgt[j], &vb);\n        }\n        if (prefilling && prefilling[r])",
     "            vpa_ref_argmax(row, dtype, ld, 1, vocab, &tgt[j], &vb);\n        }\n        if (0)"),
    ("prefilling_samples_its_bonus",
     "        out[j] = -1;\n    *n_sampled = 0;", "        out[j] = j == k ? 0 : -1;\n    *n_sampled = 1;"),
    ("prefilling_rejects_its_drafts",
     "    *n_sampled = 0;\n    *n_rejected = 0;", "    *n_sampled = 0;\n    *n_rejected = k;"),
    ("prefilling_flag_of_next_request",
     "        if (prefilling && prefilling[r])\n            ref_prefilling(k, out_tokens + base, num_sampled + r, num_rejected + r);\n        else\n            ref_accept(draft_ids + cu[r], tgt, k, ref_synth(accept, r), out_tokens + base,\n                       num_sampled + r, num_rejected + r);\n        if (target_ids)\n            for (int32_t j = 0; j <= k; ++j)\n                target_ids[base + j] = tgt[j];\n    }\n}\n\n/* Ragged greedy verification from gathered",
     "        if (prefilling && prefilling[r + 1 < n_req ? r + 1 : r])\n            ref_prefilling(k, out_tokens + base, num_sampled + r, num_rejected + r);\n        else\n            ref_accept(draft_ids + cu[r], tgt, k, ref_synth(accept, r), out_tokens + base,\n                       num_sampled + r, num_rejected + r);\n        if (target_ids)\n            for (int32_t j = 0; j <= k; ++j)\n                target_ids[base + j] = tgt[j];\n    }\n}\n\n/* Ragged greedy verification from gathered"),
    ("map_without_draft_id",
     "? (int64_t)ids[i] + d2t[ids[i]] : -1;", "? d2t[ids[i]] : -1;"),
    ("nan_scaled_too",
     "    if (isnan(v))\n        return bits;\n    float prod", "    float prod"),
    ("scale_rounded_twice",
     "    float prod = (float)(v * (double)scale);",
     "    float prod = (float)((float)v * 1.0000001f * scale);"),
    ("bonus_from_last_draft_row",
     "r * k + j, m_draft).id;\n        tgt[k] = ref_combine_row(bonus_stats, n_shards, n_req, r, m_bonus).id;",
     "r * k + j, m_draft).id;\n        tgt[k] = tgt[k - 1];"),
    ("synthetic_counts_ignored",
     "    return accept ? accept[r] : -1;", "    (void)accept;\n    (void)r;\n    return -1;"),
    ("synthetic_count_of_previous_request",
     "    return accept ? accept[r] : -1;", "    return accept ? accept[r > 0 ? r - 1 : 0] : -1;"),
    ("synthetic_capped_below_k",
     "        n = synth < k ? synth : k;", "        n = synth < k ? synth : k - 1;"),
    ("synthetic_off_by_one",
     "        n = synth < k ? synth : k;", "        n = synth + 1 < k ? synth + 1 : k;"),
    ("synthetic_stops_at_first_mismatch",
     "        n = synth < k ? synth : k;",
     "        while (n < synth && n < k && draft[n] == target[n])\n            ++n;"),
    ("negative_count_is_synthetic",
     "    if (synth >= 0)\n", "    if (synth >= -1)\n"),
    ("prefilling_yields_to_synthetic",
     "            vpa_ref_argmax(row, dtype, ld, 1, vocab, &tgt[j], &vb);\n        }\n        if (prefilling && prefilling[r])",
     "            vpa_ref_argmax(row, dtype, ld, 1, vocab, &tgt[j], &vb);\n        }\n        if (prefilling && prefilling[r] && !accept)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_src = tmp_path / "vpa_ref_mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle_build.build(src=str(mutant_src), lib=str(tmp_path / "libmutant.so"),
                               strict=False)
    runner = os.path.join(os.path.dirname(os.path.abspath(__file__)), "pin_runner.py")
    res = subprocess.run([sys.executable, runner, lib], capture_output=True, text=True, timeout=600)
    caught = [ln.split()[1] for ln in res.stdout.splitlines() if ln.startswith("caught")]
    crashed = res.returncode != 0
    assert caught or crashed, f"no pin catches the mutant {name}:\n{res.stdout}{res.stderr[-2000:]}"
    shutil.rmtree(tmp_path, ignore_errors=True)
