"""Planted mistakes for the oracle's pin tests (test infrastructure only).

Each mutant is a textual patch of a copy of oracle/oracle.c: one plausible bug
that a real implementation could make.  The shipped oracle carries none of
them; the tests build every mutant into its own library and show that at
least one pin fails against it.  A patch whose anchor text is no longer in
oracle.c fails loudly, so the list cannot silently go stale.
"""

MUTANTS = {
    "no_rope_term": ("the logits drop the 64 rope dims",
                     [("for (int i = 0; i < ORC_DQK; i++) dot += q[i] * k[i];",
                       "for (int i = 0; i < ORC_DV; i++) dot += q[i] * k[i];")]),
    "scale_sqrt_512": ("softmax scale 1/sqrt(512) instead of 1/sqrt(576)",
                       [("const double inv_sqrt = 1.0 / sqrt((double)ORC_DQK);",
                         "const double inv_sqrt = 1.0 / sqrt(512.0);")]),
    "next_physical_row": ("the gather reads the row after the right one",
                          [("  if (pg < 0 || row < 0 || row >= P->kv_rows) return -1;\n  return row;",
                            "  if (row + 1 < P->kv_rows) row += 1;\n"
                            "  if (pg < 0 || row < 0 || row >= P->kv_rows) return -1;\n  return row;")]),
    "v_from_dims_64": ("V taken from dims 64..575 instead of 0..511",
                       [("os[(size_t)sp * ORC_DV + i] += p * k[i];",
                         "os[(size_t)sp * ORC_DV + i] += p * k[64 + i];")]),
    "neighbour_head": ("each head uses its neighbour's query row",
                       [("int64_t qrow = (int64_t)b * rows + h;", "int64_t qrow = (int64_t)b * rows + (h ^ 1);")]),
    "negated_logits": ("the logits change sign",
                       [("s[t] = dot * inv_sqrt;", "s[t] = -dot * inv_sqrt;")]),
    "swapped_nibbles": ("the two e2m1 nibbles of a byte are swapped",
                        [("uint8_t nib = (i & 1) ? (byte >> 4) : (byte & 15);",
                          "uint8_t nib = (i & 1) ? (byte & 15) : (byte >> 4);")]),
    "v_without_scale": ("the fp8 per-tensor scale is left off V",
                        [("deq_row(v_dtype, v_src, phys_row(P, b, t), v_scale, v_e8m0, k);",
                          "deq_row(v_dtype, v_src, phys_row(P, b, t), v_dtype == ORC_FP8 ? 1.0 : v_scale, v_e8m0, k);")]),
    "v_from_key_cache": ("V read from the key cache although a value cache is given",
                         [("const int sep_v = P->v != NULL;", "const int sep_v = 0;")]),
}


def mutant_source(text: str, name: str) -> str:
    """oracle.c text with mutant `name` applied (each anchor must occur once)."""
    for old, new in MUTANTS[name][1]:
        n = text.count(old)
        if n != 1:
            raise AssertionError(f"mutant {name}: anchor found {n} times in oracle.c: {old!r}")
        text = text.replace(old, new)
    return text
