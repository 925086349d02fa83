"""Every plausible mistake planted in the oracle must fail at least one pin.

Each mutant is oracle.c with one snippet replaced, compiled on the CPU into a
temporary directory; the pins of tests/oracle_pins.py then run against it.
A mutant that passes every pin would mean the pins cannot see that mistake.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "fold_reverse_rank_order": (
        "load_val(dtype, in, ld_in, member(b, i, c, s), j)",
        "load_val(dtype, in, ld_in, member(b, c - 1 - i, c, s), j)"),
    "fold_drops_last_rank": (
        "        for (int i = 0; i < c; ++i) {\n          float v",
        "        for (int i = 0; i < (c > 1 ? c - 1 : 1); ++i) {\n          float v"),
    "prediv_not_rounded_to_dtype": (
        "return round_dtype(dtype, x / (float)c);",
        "return x / (float)c;"),
    "prediv_by_world_not_comm": (
        "float v = contribution(dtype, load_val(dtype, in, ld_in, member(b, i, c, s), j), pre_div, c);",
        "float v = contribution(dtype, load_val(dtype, in, ld_in, member(b, i, c, s), j), pre_div, W);"),
    "owner_row_off_by_one": (
        "store_val(dtype, out, ld_out, root, j, acc);",
        "store_val(dtype, out, ld_out, (root + 1) % W, j, acc);"),
    "rne_ties_away_from_zero": (
        "(lo == 0x8000u && (hi & 1u))",
        "(lo == 0x8000u)"),
    "rne_truncates": (
        "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;",
        ";"),
    "partition_size_floor": (
        "int64_t S = (T + p - 1) / p;",
        "int64_t S = T / p > 0 ? T / p : 1;"),
    "straddler_gets_owner": (
        "owner[i] = (eligible[g] && n == 1) ? pids[pid_offsets[i]] : -1;",
        "owner[i] = (eligible[g] && n >= 1) ? pids[pid_offsets[i]] : -1;"),
    "eligibility_ignored": (
        "int ok = comm_size[g] == W;",
        "int ok = 1;"),
    "ring_sends_left": (
        "int dst = (src + 1) % N;",
        "int dst = (src + N - 1) % N;"),
    "rs_interleaved_shards": (
        "load_val(dtype, in, ld_in, r, s * L + k)",
        "load_val(dtype, in, ld_in, r, k * W + s)"),
    "accumulate_init_copies": (
        "acc[r * ld_acc + j] = a + x[r * ld_x + j];",
        "acc[r * ld_acc + j] = init ? x[r * ld_x + j] : a + x[r * ld_x + j];"),
    "deferred_writes_row0_only": (
        "for (int i = 0; i < out_rows; ++i) out[i * ld_out + j] = s;",
        "out[j] = s;"),
    "probe_kept_counts_written": (
        "if (hd[r]) kept[r] += n;",
        "if (wr[r]) kept[r] += n;"),
    "zero2_partition_off_by_one": (
        "store_val(dtype, out, ld_out, (a + (j - start)) / S, j, acc);",
        "store_val(dtype, out, ld_out, (a + (j - start) + 1) / S % W, j, acc);"),
    "zero2_straddler_allreduce": (
        "int64_t S = t_comm[t] == 0 ? part_size[t_param[t]] : 0;",
        "int64_t S = 0;"),
    "relayout_segment_by_task_order": (
        "dest[t_off[t] + e] = count[q]++;",
        "dest[t_off[t] + e] = seg_start[q] + (seg_start[q + 1] - 1 - (count[q]++ - seg_start[q]));"),
    "relayout_segment_off_by_one": (
        "for (int q = 0; q < W; ++q) seg_start[q + 1] = seg_start[q] + count[q];",
        "for (int q = 0; q < W; ++q) seg_start[q + 1] = seg_start[q] + count[q] + (q == 0);"),
    "rsv_wrong_destination_row": (
        "      store_val(dtype, out, ld_out, q, k, acc);",
        "      store_val(dtype, out, ld_out, (q + 1) % W, k, acc);"),
    "buffers_first_holder_only": (
        "if (o >= 0) store_val(dtype, out, 0, 0, o + e, sum);",
        "if (o >= 0) { store_val(dtype, out, 0, 0, o + e, sum); break; }"),
    "buffers_neighbour_gradient": (
        "load_val(dtype, in, 0, 0, in_off[(int64_t)t * W + r] + e)",
        "load_val(dtype, in, 0, 0, in_off[(int64_t)t * W + (r + 1) % W] + e)"),
    "buffers_element_shift": (
        "store_val(dtype, out, 0, 0, o + e, sum);",
        "store_val(dtype, out, 0, 0, o + (e + 1) % t_numel[t], sum);"),
    "ring_rs_wrong_holder": (
        "int holder = (c - 1 + W) % W;",
        "int holder = (c - 2 + 2 * W) % W;"),
    "ring_rs_sends_left": (
        "int src = (i - 1 + W) % W;",
        "int src = (i + 1) % W;"),
    "bidir_floor_step_count": (
        "int32_t steps = algo == 0 ? N - 1 : algo == 1 ? N / 2 : 0;",
        "int32_t steps = algo == 0 ? N - 1 : algo == 1 ? (N - 1) / 2 : 0;"),
    "bidir_chunk_taken_twice": (
        "if (algo == 1 && !held[(int64_t)i * N + nr[i]]) {",
        "if (algo == 1) {"),
    "bidir_tie_taken_from_right": (
        "        if (!held[(int64_t)i * N + nl[i]]) {",
        "        if (!held[(int64_t)i * N + nl[i]] && !(algo == 1 && nl[i] == nr[i])) {"),
    "ag_step_forwards_own_chunk": (
        "        from_left[i] = nl[i];\n",
        "        from_left[i] = from_left[i];\n"),
    "ag_step0_wrong_position": (
        "memcpy((char*)out + ((int64_t)i * ld_out + (int64_t)i * L) * eb,",
        "memcpy((char*)out + ((int64_t)i * ld_out + (int64_t)((i + 1) % W) * L) * eb,"),
    "deferred_reverse_rank_order": (
        "s = (r == 0) ? acc[r * ld_acc + j] : s + acc[r * ld_acc + j];",
        "s = (r == 0) ? acc[(W - 1 - r) * ld_acc + j] : s + acc[(W - 1 - r) * ld_acc + j];"),
    "owner_honoured_on_sub_comm": (
        "int root = (t_comm[t] == 0 && owner != NULL) ? owner[t_param[t]] : -1;",
        "int root = (owner != NULL) ? owner[t_param[t]] : -1;"),
    "deferred_starts_from_zero": (
        "s = (r == 0) ? acc[r * ld_acc + j] : s + acc[r * ld_acc + j];",
        "s = s + acc[r * ld_acc + j];"),
    "relayout_ignores_bucket_column": (
        "(const char*)in + ((int64_t)r * ld_in + bucket_col + c) * eb",
        "(const char*)in + ((int64_t)r * ld_in + c) * eb"),
    "probe_strided_holders_as_contiguous": (
        "for (int b = 0; b < W / c; ++b) hd[member(b, pids[k], c, s)] = 1;",
        "for (int b = 0; b < W / c; ++b) hd[b * c + pids[k]] = 1;"),
    "rd_partner_plus": (
        "int q = i ^ d;",
        "int q = (i + d) % N;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    # the same mistake everywhere the snippet occurs (the fold appears in
    # both flush variants)
    path = tmp_path / "oracle_mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-w", "-o", str(so), str(path)], check=True)
    saved = oracle._lib
    oracle._lib = oracle.load_library(str(so))
    failed = []
    try:
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError, RuntimeError, IndexError):
                failed.append(pin.__name__)
                break
    finally:
        oracle._lib = saved
    assert failed, f"mutant {name} passes every pin"
