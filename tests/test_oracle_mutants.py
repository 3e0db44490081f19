"""Planted mistakes in the oracle must fail its pins.

Each case below is a plausible slip in ``oracle/oracle.c`` (a wrong index or
stride, an off-by-one, a dropped or reordered term, a different rounding).
The case is planted in a private copy of the source, built with the oracle's
own flags, and ``tests/test_oracle_pins.py`` is run against that build (the
oracle loads it through ``EP_ORACLE_LIB``).  The pins must fail for every case.
A case that survives marks a part of the oracle that nothing pins.

Runs on the CPU only.  The planted copies live in a temporary directory, and
every one stays inside its buffers.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, [(text in oracle.c, replacement), ...]); every text occurs exactly once
MUTANTS = [
    ("rank_round_robin",
     [("if (e >= 0) is_token_in_rank[u * P + e / El] = 1;", "if (e >= 0) is_token_in_rank[u * P + e % P] = 1;")]),
    ("alignment_overpads",
     [("      int64_t padded = ((n + A - 1) / A) * A;\n      off += padded;",
       "      int64_t padded = (n / A + 1) * A;\n      off += padded;")]),
    ("rank_prefix_exclusive",
     [("      acc += num_tokens_per_rank[s * P + d];\n      rank_prefix_matrix[s * P + d] = acc;",
       "      rank_prefix_matrix[s * P + d] = acc;\n      acc += num_tokens_per_rank[s * P + d];")]),
    ("expert_counts_by_destination",
     [("if (e >= 0) num_tokens_per_expert[(int64_t)s * E + e] += 1;",
       "if (e >= 0) num_tokens_per_expert[(int64_t)(e / El) * E + e] += 1;")]),
    ("expert_offset_stride",
     [("dst_slot[u * K + j] = (int32_t)(expert_offset[(int64_t)d * (El + 1) + l] + seen_e[e]);",
       "dst_slot[u * K + j] = (int32_t)(expert_offset[(int64_t)d * El + l] + seen_e[e]);")]),
    ("send_head_off_by_one",
     [("      send_head[u * P + d] = seen_d[d];", "      send_head[u * P + d] = seen_d[d] + 1;")]),
    ("recv_src_idx_global_token",
     [("recv_src_idx[recv_src_base[d] + seen_d[d]] = (int32_t)(u % S);",
       "recv_src_idx[recv_src_base[d] + seen_d[d]] = (int32_t)u;")]),
    ("symmetric_windows_ignored",
     [("window_row_base[d + 1] = symmetric ? (int64_t)(d + 1) * max_expanded",
       "window_row_base[d + 1] = 0 ? (int64_t)(d + 1) * max_expanded")]),
    ("scale_divides_by_447",
     [("f32_from_bits(0x7FC00000u) : amax / 448.0f;", "f32_from_bits(0x7FC00000u) : amax / 447.0f;")]),
    ("codes_by_reciprocal",
     [("float q = xf / scale;", "float q = xf * (1.0f / scale);")]),
    ("amax_skips_nan",
     [("    for (int h = 128 * b; h < 128 * b + 128; h++) {\n      float v = fabsf(oracle_bf16_to_float(x[h]));\n"
       "      if (isnan(v))",
       "    for (int h = 128 * b; h < 128 * b + 128; h++) {\n      float v = fabsf(oracle_bf16_to_float(x[h]));\n"
       "      if (0)")]),
    ("ue8m0_amax_skips_nan",
     [("    for (int h = 32 * b; h < 32 * b + 32; h++) {\n      float v = fabsf(oracle_bf16_to_float(x[h]));\n"
       "      if (isnan(v))",
       "    for (int h = 32 * b; h < 32 * b + 32; h++) {\n      float v = fabsf(oracle_bf16_to_float(x[h]));\n"
       "      if (0)")]),
    ("nan_codes_keep_sign",
     [("codes[h] = isnan(q) ? 0x7F : oracle_e4m3_encode(q);", "codes[h] = oracle_e4m3_encode(q);")]),
    ("amax_flushes_subnormal_inputs",
     [("    for (int h = 128 * b; h < 128 * b + 128; h++) {\n      float v = fabsf(oracle_bf16_to_float(x[h]));",
       "    for (int h = 128 * b; h < 128 * b + 128; h++) {\n      float v = fabsf(oracle_bf16_to_float(x[h]));\n"
       "      if (v < 1.17549435e-38f) v = 0.0f;")]),
    ("ue8m0_exponent_rounds_down",
     [("while (k < 127 && ldexp(448.0, k) < (double)amax) k++;",
       "while (k < 127 && ldexp(448.0, k + 1) <= (double)amax) k++;")]),
    ("ue8m0_exponent_not_minimal",
     [("while (k < 127 && ldexp(448.0, k) < (double)amax) k++;",
       "while (k < 127 && ldexp(448.0, k) <= (double)amax) k++;")]),
    ("ue8m0_amax_skips_last_channel",
     [("    for (int h = 32 * b; h < 32 * b + 32; h++) {\n      float v = fabsf",
       "    for (int h = 32 * b; h < 32 * b + 31; h++) {\n      float v = fabsf")]),
    ("ue8m0_codes_multiply_by_scale",
     [("codes[h] = oracle_e4m3_encode(oracle_bf16_to_float(x[h]) / scale);",
       "codes[h] = oracle_e4m3_encode(oracle_bf16_to_float(x[h]) * scale);")]),
    ("ue8m0_nan_exponent_zero",
     [("      exps[b] = 0xFF;", "      exps[b] = 0x00;")]),
    ("ue8m0_padding_exponents_left",
     [("            memset((uint8_t *)recv_scales + rr * nb32, 0, (size_t)nb32);\n          else\n"
       "            put_scales(recv_scales, scales_col_major, n_out, rr, nb, NULL);\n        } else {\n"
       "          for (int h = 0; h < H; h++) ((uint16_t *)recv_x)[rr * H + h] = 0;\n        }\n      }\n    }",
       "            (void)0;\n          else\n"
       "            put_scales(recv_scales, scales_col_major, n_out, rr, nb, NULL);\n        } else {\n"
       "          for (int h = 0; h < H; h++) ((uint16_t *)recv_x)[rr * H + h] = 0;\n        }\n      }\n    }")]),
    ("combine_flushes_subnormal_products",
     [("        float prod = w * oracle_bf16_to_float(y[r * H + h]);\n        acc = acc + prod;",
       "        float prod = w * oracle_bf16_to_float(y[r * H + h]);\n"
       "        if (fabsf(prod) < 1.17549435e-38f) prod = copysignf(0.0f, prod);\n        acc = acc + prod;")]),
    ("amax_skips_last_channel",
     [("    for (int h = 128 * b; h < 128 * b + 128; h++) {\n      float v = fabsf",
       "    for (int h = 128 * b; h < 128 * b + 127; h++) {\n      float v = fabsf")]),
    ("e4m3_ties_away",
     [("double r = nearbyint(m * 8.0); /* 3 mantissa bits, ties to even */",
       "double r = floor(m * 8.0 + 0.5); /* 3 mantissa bits, ties to even */")]),
    ("e4m3_subnormal_threshold",
     [("if (a < ldexp(1.0, -6)) {", "if (a < ldexp(1.0, -7)) {")]),
    ("bf16_ties_away",
     [("return (uint16_t)((b + 0x7FFFu + lsb) >> 16);", "return (uint16_t)((b + 0x8000u) >> 16);")]),
    ("dispatch_ignores_window_base",
     [("      int64_t r = (capacity > 0 ? (e / El) * capacity : window_row_base[e / El]) + local;\n"
       "      if (r < row_begin",
       "      int64_t r = (capacity > 0 ? (e / El) * capacity : window_row_base[0]) + local;\n"
       "      if (r < row_begin")]),
    ("meta_slot_off_by_one",
     [("        recv_src_meta[2 * rr + 1] = j;", "        recv_src_meta[2 * rr + 1] = j + 1;")]),
    ("weight_of_first_slot",
     [("if (recv_weights) recv_weights[rr] = topk_weights[u * K + j];",
       "if (recv_weights) recv_weights[rr] = topk_weights[u * K];")]),
    ("zero_padding_always",
     [("if (zero_padding && recv_x) {", "if (recv_x) {")]),
    ("fixed_tail_keeps_payload",
     [("        if (recv_x) {\n          if (fp8) {", "        if (0) {\n          if (fp8) {")]),
    ("truncation_off_by_one",
     [("if (capacity > 0 && local >= capacity) continue; /* truncated */",
       "if (capacity > 0 && local > capacity) continue; /* truncated */")]),
    ("dropped_count_off_by_one",
     [("if (used > capacity) drop += used - capacity;", "if (used > capacity) drop += used - capacity + 1;")]),
    ("col_major_scales_ignored",
     [("      recv_scales[(int64_t)b * n + rr] = v;", "      recv_scales[rr * nb + b] = v;")]),
    ("prequant_scales_of_previous_token",
     [("memcpy(scales, x_scales + u * nb, sizeof(float) * (size_t)nb);",
       "memcpy(scales, x_scales + (u > 0 ? u - 1 : u) * nb, sizeof(float) * (size_t)nb);")]),
    ("combine_slots_descending",
     [("      for (int j = 0; j < K; j++) {\n        int64_t e = topk_idx[u * K + j];\n        if (e < 0) continue;\n"
       "        int64_t local = dst_slot[u * K + j];",
       "      for (int j = K - 1; j >= 0; j--) {\n        int64_t e = topk_idx[u * K + j];\n        if (e < 0) continue;\n"
       "        int64_t local = dst_slot[u * K + j];")]),
    ("combine_fused_multiply_add",
     [("        float prod = w * oracle_bf16_to_float(y[r * H + h]);\n        acc = acc + prod;",
       "        acc = fmaf(w, oracle_bf16_to_float(y[r * H + h]), acc);")]),
    ("combine_weights_reversed",
     [("        float w = topk_weights ? topk_weights[u * K + j] : 1.0f;\n"
       "        float prod = w * oracle_bf16_to_float(y[r * H + h]);",
       "        float w = topk_weights ? topk_weights[u * K + (K - 1 - j)] : 1.0f;\n"
       "        float prod = w * oracle_bf16_to_float(y[r * H + h]);")]),
    ("combine_bias_first",
     [("      float acc = 0.0f;\n      for (int j = 0; j < K; j++) {\n        int64_t e = topk_idx[u * K + j];",
       "      float acc = bias ? oracle_bf16_to_float(bias[u * H + h]) : 0.0f;\n"
       "      for (int j = 0; j < K; j++) {\n        int64_t e = topk_idx[u * K + j];"),
      ("      if (bias) acc = acc + oracle_bf16_to_float(bias[u * H + h]);\n"
       "      out[(u - tok_begin) * H + h] = oracle_bf16_round(acc);\n    }\n  }\n  return ORACLE_OK;\n}\n\nint oracle_combine(",
       "      out[(u - tok_begin) * H + h] = oracle_bf16_round(acc);\n    }\n  }\n  return ORACLE_OK;\n}\n\nint oracle_combine(")]),
]


def _plant(name, edits, workdir):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, (name, old)
        src = src.replace(old, new)
    c = os.path.join(workdir, f"{name}.c")
    so = os.path.join(workdir, f"lib{name}.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", *oracle.CFLAGS, "-I", os.path.join(ROOT, "oracle"), "-o", so, c, "-lm"],
                   check=True, capture_output=True)
    return so


def _run_pins(so):
    env = dict(os.environ, EP_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    # the unmodified source passes (so a failure below is the planted mistake's)
    base = _plant("unmodified", [], str(tmp_path))
    rc, out = _run_pins(base)
    assert rc == 0, out
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        futs = {name: pool.submit(lambda n=name, e=edits: _run_pins(_plant(n, e, str(tmp_path))))
                for name, edits in MUTANTS}
        results = {name: f.result() for name, f in futs.items()}
    survivors = [name for name, (rc, _) in results.items() if rc != 1]
    assert not survivors, {n: results[n][1] for n in survivors}
