"""Plant plausible mistakes in copies of the oracle; the pins must catch each.

Each mutant is a one-spot textual edit of ``oracle/oracle.c`` (a dropped term,
a wrong index, a transposed operand, a wrong rounding or compare), compiled
into a temporary directory on the CPU.  The real oracle is never modified.
"""

import pytest

import oracle
import oracle_pins as pins

MUTANTS = {
    "fold_drops_rank1": ("for (int r = 1; r < nranks; r++)\n            acc = combine_f",
                         "for (int r = 2; r < nranks; r++)\n            acc = combine_f"),
    "fold_drops_last_rank_int": ("for (int r = 1; r < nranks; r++)\n            acc = combine_i",
                                 "for (int r = 1; r < nranks - 1; r++)\n            acc = combine_i"),
    "bf16_truncates": ("u += 0x7FFFu + lower_half_keep_bit;", "u += 0u * lower_half_keep_bit;"),
    "bf16_ties_away": ("u += 0x7FFFu + lower_half_keep_bit;", "u += 0x8000u + 0u * lower_half_keep_bit;"),
    "bf16_nan_unquieted": ("return (uint16_t)((u >> 16) | 0x0040u);", "return (uint16_t)(u >> 16);"),
    "max_tie_keeps_later": ("return (v > a) ? v : a;\n    return (v < a) ? v : a;\n}\n\nstatic int32_t",
                            "return (v >= a) ? v : a;\n    return (v < a) ? v : a;\n}\n\nstatic int32_t"),
    "nan_not_propagated": ("if (is_nan_f(v))\n        return v;", "if (0)\n        return v;"),
    "int_max_is_min": ("if (op == OR_MAX)\n        return (v > a) ? v : a;\n    return (v < a) ? v : a;\n}\n\n/* Element",
                       "if (op == OR_MAX)\n        return (v < a) ? v : a;\n    return (v < a) ? v : a;\n}\n\n/* Element"),
    "rs_wrong_chunk": ("fold_one(x, (size_t)r * m, nranks, i, dtype, op, y[r], i);",
                       "fold_one(x, (size_t)((r + 1) % nranks) * m, nranks, i, dtype, op, y[r], i);"),
    "ag_reverse_order": ("memcpy((char*)y[q] + at * esize, x[r], counts[r] * esize);",
                         "memcpy((char*)y[q] + at * esize, x[nranks - 1 - r], counts[r] * esize);"),
    "a2a_transposed_len": ("splits[(size_t)i * nranks + j] * esize);",
                           "splits[(size_t)j * nranks + i] * esize);"),
    "a2a_send_offset": ("send_off += splits[(size_t)i * nranks + jj];",
                        "send_off += splits[(size_t)jj * nranks + i];"),
    "bucket_skips": ("for (size_t start = 0; start < total; start += per_bucket) {\n        size_t len = total - start < per_bucket ? total - start : per_bucket;\n        for (size_t e = 0; e < len; e++) {\n            fold_one((const void* const*)flat",
                     "for (size_t start = 0; start < total; start += per_bucket + 1) {\n        size_t len = total - start < per_bucket ? total - start : per_bucket;\n        for (size_t e = 0; e < len; e++) {\n            fold_one((const void* const*)flat"),
    "hsdp_wrong_group": ("group[i] = work[i * shard + j];", "group[i] = work[(i * shard + j + shard) % nranks];"),
    "hsdp_wrong_member": ("members[jj] = grads[(size_t)(i * shard + jj) * ntensors + t];",
                          "members[jj] = grads[(size_t)(jj * replicate + i) * ntensors + t];"),
    "barrier_notifies_self": ("if (p != r)\n                    window", "if (1)\n                    window"),
    "barrier_fixed_threshold": ("window[(size_t)r * nranks + s] < g)", "window[(size_t)r * nranks + s] < 1)"),
    "exchange_wrong_peer": ("x[(r + 1) % nranks]", "x[(r + nranks - 1) % nranks]"),
    "avg_divides_by_p_minus_1": ("acc = acc / (float)nranks;", "acc = acc / (float)(nranks > 1 ? nranks - 1 : 1);"),
    "avg_int_rounds_down": ("acc = acc / nranks;", "acc = (int32_t)((acc - (acc < 0 ? nranks - 1 : 0)) / nranks);"),
    "r2s_wrong_slice": ("(const char*)x[r] + (size_t)r * m * esize", "(const char*)x[r] + (size_t)((r + 1) % nranks) * m * esize"),
    "agvec_transposed": ("memcpy(y[(size_t)q * nranks + r], x[r], counts[r] * esize);",
                         "memcpy(y[(size_t)r * nranks + q], x[r], counts[r] * esize);"),
    "dims_wrong_owner": ("from = (const char*)x[b / cp] + (a * cp + b % cp) * esize;",
                         "from = (const char*)x[b % nranks] + (a * cp + b / nranks) * esize;"),
    "broadcast_skips_last": ("for (int q = 0; q < nranks; q++)\n        memcpy(y[q], x_root, nbytes);",
                             "for (int q = 0; q + 1 < nranks; q++)\n        memcpy(y[q], x_root, nbytes);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / f"lib_{name}.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
