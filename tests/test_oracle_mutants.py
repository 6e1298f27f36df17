"""The pins have teeth: plant plausible mistakes in a copy of the oracle and
check that at least one pin fails for each (no GPU).

Each mutant is a textual edit of ``oracle/a2av_ref.c`` (a swapped index, a
dropped term, an inclusive instead of exclusive scan, an unstable order, an
off-by-one bound, a transposed operand). Some planted mistakes move a
chunk past the end of its buffer, so every mutant runs in a child process: the
child reports the first pin that fails, and a child killed by the memory error
before any pin fails counts as caught by that crash (reported as such).
"""
import os
import subprocess
import sys

import pytest

import oracle.ref as R
import oracle_pins

SRC = open(R.SRC).read()

MUTANTS = {
    "exchange_not_transposed": [
        ("O[d * W + s] = S[s * W + d];", "O[d * W + s] = S[d * W + s];", 0)],
    "send_scan_inclusive": [
        ("send_off[s * (W + 1) + d] = run;\n            run += S[s * W + d];",
         "run += S[s * W + d];\n            send_off[s * (W + 1) + d] = run;", 0)],
    "recv_scan_reads_S_not_O": [("run += O[d * W + s];", "run += S[d * W + s];", 0)],
    "copy_src_offset_transposed": [
        ("(size_t)send_off[s * (W + 1) + d] * R;", "(size_t)send_off[d * (W + 1) + s] * R;", 0)],
    "copy_dst_offset_transposed": [
        ("(size_t)recv_off[d * (W + 1) + s] * R;", "(size_t)recv_off[s * (W + 1) + d] * R;", 0)],
    "copy_count_transposed": [
        ("int64_t rows = S[s * W + d];\n            if (rows == 0) continue;",
         "int64_t rows = S[d * W + s];\n            if (rows == 0) continue;", 0)],
    "overrun_off_by_one": [
        ("if (send_off[s * (W + 1) + W] > in_rows[s]) st |= REF_SEND_OVERRUN;",
         "if (send_off[s * (W + 1) + W] >= in_rows[s]) st |= REF_SEND_OVERRUN;", 1)],
    "overflow_check_slack": [
        ("if (recv_off[d * (W + 1) + W] > out_cap_rows[d]) st |= REF_RECV_OVERFLOW;",
         "if (recv_off[d * (W + 1) + W] > out_cap_rows[d] + 1) st |= REF_RECV_OVERFLOW;", 1)],
    "copy_ignores_bad_offsets": [
        ("if (step != (uint64_t)S[s * W + d]) st |= REF_BAD_OFFSETS;", "(void)step;", 0)],
    "split_range_not_checked": [
        ("return v >= 0 && v <= REF_MAX_SPLIT;", "return v >= 0;", 0)],
    "pack_unstable": [
        ("for (int64_t q = 0; q < Q; q++) perm[q] = next[ids[q]]++;",
         "for (int64_t q = Q - 1; q >= 0; q--) perm[q] = next[ids[q]]++;", 0)],
    "pack_owner_modulo": [("splits[e / per_rank] += count[e];", "splits[e % W] += count[e];", 0)],
    "pack_wrong_token": [("(size_t)(q / k) * R, R);", "(size_t)(q % T) * R, R);", 0)],
    "unpack_scatter_not_gather": [
        ("memcpy((unsigned char *)out + (size_t)q * R,\n"
         "               (const unsigned char *)back + (size_t)perm[q] * R, R);",
         "memcpy((unsigned char *)out + (size_t)perm[q] * R,\n"
         "               (const unsigned char *)back + (size_t)q * R, R);", 0)],
    "source_of_drops_send_start": [
        ("*src_row = send_start + (j - recv_start);", "*src_row = (j - recv_start); (void)send_start;", 0)],
    "bad_expert_upper_bound": [("if (ids[q] < 0 || ids[q] >= E) return REF_BAD_EXPERT;",
                                "if (ids[q] < 0 || ids[q] > E) return REF_BAD_EXPERT;", 0)],
    "regroup_drops_earlier_sources": [
        ("for (int s2 = 0; s2 < s; s2++) expert_major += counts[s2 * E + d * P + j];",
         "(void)0;", 0)],
    "regroup_directions_swapped": [
        ("const int64_t from = direction == 0 ? src_major : expert_major;",
         "const int64_t from = direction == 1 ? src_major : expert_major;", 0),
        ("const int64_t to = direction == 0 ? expert_major : src_major;",
         "const int64_t to = direction == 1 ? expert_major : src_major;", 0)],
    "combine_unfused_multiply_add": [
        ("acc = fmaf(w[t * k + j], bf16_to_float(back[row * H + h]), acc);",
         "acc = w[t * k + j] * bf16_to_float(back[row * H + h]) + acc;", 0)],
    "combine_reverse_order": [
        ("for (int j = 0; j < k; j++) {\n                const int64_t row = perm[t * k + j];",
         "for (int j = k - 1; j >= 0; j--) {\n                const int64_t row = perm[t * k + j];", 0)],
    "combine_keeps_nan_payload": [
        ("if (isnan(f)) return 0x7FC0u;", "if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);", 0)],
    "combine_truncates_to_bf16": [
        ("return (uint16_t)((u + 0x7FFFu + lsb) >> 16);", "(void)lsb; return (uint16_t)(u >> 16);", 0)],
    "bucketize_reads_keys_at_output_position": [
        ("memcpy(keys_out + kpos, keys + tstart[t], (size_t)tk[t] * 8);",
         "memcpy(keys_out + kpos, keys + kpos, (size_t)tk[t] * 8);", 0)],
    "grouped_drops_earlier_sources": [
        ("            for (int s2 = 0; s2 < s; s2++) exp_pos += counts[s2 * E + e];",
         "            (void)0;", 0)],
    "grouped_pack_pos_not_advanced": [
        ("            pack_pos += n;\n        }\n    }\n    return 0;\n}",
         "            (void)n;\n        }\n    }\n    return 0;\n}", 0)],
    "combine_grouped_ignores_block_offset": [
        ("const int64_t row = X[s * E + e] + (perm[s][q] - Y[s * E + e]);",
         "const int64_t row = X[s * E + e];", 0)],
    "combine_grouped_skips_block_check": [
        ("if (p < Y[s * E + e] || p >= Y[s * E + e] + counts[s * E + e]) st |= REF_BAD_PERM;",
         "(void)p;", 0)],
    "pack_dispatch_layout1_source_major": [
        ("x->key[0] = layout == 0 ? s : e;\n                x->key[1] = layout == 0 ? e : s;",
         "x->key[0] = s;\n                x->key[1] = e;", 0)],
    "pack_dispatch_source_offsets_transposed": [
        ("if (layout == 0) run += S[g * W + d];", "if (layout == 0) run += S[d * W + g];", 0)],
    "pack_dispatch_wrong_token": [("x->tok = q / k;", "x->tok = q % T;", 0)],
    "unpack_return_ignores_layout": [("        if (layout == 0) {\n", "        if (layout == 2) {\n", 0)],
    "unpack_return_ignores_block_offset": [
        ("const int64_t row = Z[s * E + e] + (perm[s][q] - Y[s * E + e]);",
         "const int64_t row = Z[s * E + e];", 0)],
    "unpack_return_overrun_off_by_one": [
        ("if (run > recv_rows[d]) st |= REF_SEND_OVERRUN;",
         "if (run >= recv_rows[d]) st |= REF_SEND_OVERRUN;", 0)],
    "combine_return_ignores_layout": [("recv_rows, home, layout);", "recv_rows, home, 0);", 0)],
    "combine_return_uses_pack_perm": [
        ("(const uint16_t *)home[s], ident, w[s], out[s]);",
         "(const uint16_t *)home[s], perm[s], w[s], out[s]);", 0)],
    "keys_exchange_offsets_inclusive": [
        ("            recv_off_keys[d * (W + 1) + s] = run;\n            run += Sk[s * W + d];",
         "            run += Sk[s * W + d];\n            recv_off_keys[d * (W + 1) + s] = run;", 0)],
    "keys_exchange_lengths_use_key_splits": [
        ("(void *const *)lengths_out,\n                               lengths_cap, Sl, O, so, ro);",
         "(void *const *)lengths_out,\n                               lengths_cap, Sk, O, so, ro);", 0)],
    "bucketize_length_split_counts_keys": [
        ("split_lengths[d] += batch;", "split_lengths[d] += tk[t];", 0)],
    # totals, counts and offsets beside the payload
    "send_total_drops_last": [
        ("        send_off[s * (W + 1) + W] = run;",
         "        send_off[s * (W + 1) + W] = run - S[s * W + W - 1];", 0)],
    "recv_total_from_send_row": [
        ("        recv_off[d * (W + 1) + W] = run;",
         "        recv_off[d * (W + 1) + W] = send_off[d * (W + 1) + W];", 0)],
    "expert_counts_shifted": [
        ("for (int e = 0; e < E; e++) expert_counts[e] = count[e];",
         "for (int e = 0; e < E; e++) expert_counts[e] = count[(e + 1) % E];", 0)],
    "regroup_offsets_total_wrong": [
        ("    expert_offsets[P] = run;", "    expert_offsets[P] = expert_offsets[P - 1];", 0)],
    "regroup_offsets_inclusive": [
        ("        expert_offsets[j] = run;\n        for (int s = 0; s < W; s++) run += counts[s * E + d * P + j];",
         "        for (int s = 0; s < W; s++) run += counts[s * E + d * P + j];\n        expert_offsets[j] = run;", 0)],
    "keys_recv_total_short": [
        ("        recv_off_keys[d * (W + 1) + W] = run;",
         "        recv_off_keys[d * (W + 1) + W] = run - Sk[(W - 1) * W + d];", 0)],
    "keys_split_lengths_transposed": [
        ("            split_lengths[s * W + d] = Sl[s * W + d];",
         "            split_lengths[s * W + d] = Sl[d * W + s];", 0)],
    # bounds one off
    "bucketize_overrun_slack": [
        ("    if (run > n_keys) { free(tk); free(tstart); return REF_SEND_OVERRUN; }",
         "    if (run > n_keys + 1) { free(tk); free(tstart); return REF_SEND_OVERRUN; }", 0)],
    "keys_capacity_slack": [
        ("        if (rk > keys_cap[d] || rl > lengths_cap[d])",
         "        if (rk > keys_cap[d] + 1 || rl > lengths_cap[d])", 0)],
    "regroup_overflow_slack": [
        ("    if (total > out_cap) st |= REF_RECV_OVERFLOW;",
         "    if (total > out_cap + 1) st |= REF_RECV_OVERFLOW;", 0)],
    "pack_expert_bound_slack": [
        ("        if (ids[q] < 0 || ids[q] >= E) return REF_BAD_EXPERT;",
         "        if (ids[q] < 0 || ids[q] > E) return REF_BAD_EXPERT;", 0)],
}

# cheap pins first; the brute-force enumeration last
PIN_ORDER = sorted(oracle_pins.ALL_PINS,
                   key=lambda f: (f.__name__ in ("pin_brute_force_tiny", "pin_emb_two_call_consistency"),
                                  f.__name__))


def _apply(src, edits):
    for old, new, nth in edits:
        parts = src.split(old)
        assert len(parts) > nth + 1, f"pattern not found ({nth}): {old!r}"
        src = old.join(parts[:nth + 1]) + new + old.join(parts[nth + 1:])
    return src


def _run_pins_in_child(so_path):
    """Run the pins on a library in a child process; returns (how, detail)."""
    code = ("import sys, os; sys.path[:0] = [%r, %r]\n"
            "import oracle.ref as R, test_oracle_mutants as M\n"
            "o = R.Oracle(R.load(%r))\n"
            "for pin in M.PIN_ORDER:\n"
            "    try:\n"
            "        pin(o)\n"
            "    except AssertionError:\n"
            "        print('CAUGHT', pin.__name__, flush=True); os._exit(0)\n"
            "print('MISSED', flush=True); os._exit(0)\n") % (
                os.path.dirname(R.HERE), os.path.dirname(os.path.abspath(__file__)), str(so_path))
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    out = p.stdout.strip().splitlines()
    if out and out[-1].startswith("CAUGHT"):
        return "pin", out[-1].split()[1]
    if out and out[-1] == "MISSED":
        return "missed", ""
    return "crash", f"rc={p.returncode} {p.stderr[-300:]}"


def _build(tmp_path, src, name):
    c = tmp_path / "a2av_ref.c"
    c.write_text(src)
    (tmp_path / "a2av_ref.h").write_text(open(os.path.join(R.HERE, "a2av_ref.h")).read())
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(c)],
                   check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = _apply(SRC, MUTANTS[name])
    assert src != SRC
    how, detail = _run_pins_in_child(_build(tmp_path, src, f"mut_{name}"))
    print(f"{name}: {how} {detail}")
    assert how != "missed", f"no pin caught the planted mistake {name!r}"


def test_unmutated_copy_passes(tmp_path):
    """The same build route without an edit passes every pin (so a caught
    mutant is caught for its mistake, not for the build)."""
    how, detail = _run_pins_in_child(_build(tmp_path, SRC, "plain"))
    assert how == "missed", (how, detail)
