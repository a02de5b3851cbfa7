"""Plant a plausible mistake in a copy of the oracle's C source, build it, and
check that the pins in test_oracle.py, test_oracle_rope.py and
test_oracle_fp8.py catch it.  CPU only; the oracle in the tree is never
modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pa_oracle.c")

MUTANTS = {
    "gqa_head_map": ("const int32_t kvh = h / group;", "const int32_t kvh = h % num_kv_heads;"),
    "dropped_scale": ("s[t] = scale * dot;", "s[t] = dot;"),
    "slot_offset": ("int64_t block_offset = pos % block_size;",
                    "int64_t block_offset = (pos + 1) % block_size;"),
    "causal_off_by_one": ("const int64_t n = causal ? pos_q + 1 : L;",
                          "const int64_t n = causal ? pos_q : L;"),
    "keys_read_from_values": ("widen(key_cache, kbase + d, kv_dtype)", "widen(value_cache, kbase + d, kv_dtype)"),
    "gather_offset": ("int64_t off = t % block_size;", "int64_t off = (t + 1) % block_size;"),
    "scatter_reversed_offset": ("int64_t dst = (block * block_size + offset) * row_elems;",
                                "int64_t dst = (block * block_size + (block_size - 1 - offset)) * row_elems;"),
    "exp_sign": ("s[t] = exp(s[t] - m);", "s[t] = exp(m - s[t]);"),
    "missing_normalisation": ("double w = s[t] / l;", "double w = s[t];"),
    "transposed_query_index": ("const int64_t qbase = row * q_stride + (int64_t)h * head_dim;",
                               "const int64_t qbase = (int64_t)h * q_stride + row * head_dim;"),
    "rope_sign": ("out[a] = x[a] * c - x[b] * s;", "out[a] = x[a] * c + x[b] * s;"),
    "rope_partner": ("int32_t b = neox_style ? i + half : 2 * i + 1;",
                     "int32_t b = neox_style ? half - 1 - i + half : 2 * i + 1;"),
    "rope_frequency": ("pow(base, -2.0 * i / rotary_dim)", "pow(base, -1.0 * i / rotary_dim)"),
    "rope_cos_sin_swapped": ("table[p * rotary_dim + i] = cos(angle);", "table[p * rotary_dim + i] = sin(angle);"),
    "rope_k_from_q_columns": ("x[d] = widen(qkv, base + k_col + (int64_t)h * head_dim + d, dtype);",
                              "x[d] = widen(qkv, base + (int64_t)h * head_dim + d, dtype);"),
    "rope_table_row": ("cos_sin + positions[t] * rotary_dim", "cos_sin + positions[t] * (rotary_dim / 2)"),
    "e4m3_bias": ("v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    "e4m3_subnormal_step": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    "e4m3_ties_to_odd": ("(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)"),
    "e4m3_saturation_point": ("if (a >= 448.0)", "if (a >= 240.0)"),
    "fp8_k_scale_dropped": ("(widen(key_cache, kbase + d, kv_dtype) * k_scale)",
                            "widen(key_cache, kbase + d, kv_dtype)"),
    "fp8_scatter_multiplies": ("encode_fp8(x / k_scale, fmt)", "encode_fp8(x * k_scale, fmt)"),
    "e5m2_bias": ("v = ldexp(1.0 + m / 4.0, e - 15);", "v = ldexp(1.0 + m / 4.0, e - 16);"),
    "e5m2_subnormal_step": ("v = ldexp((double)m, -16);", "v = ldexp((double)m, -17);"),
    "e5m2_ties_to_odd": ("if (d < best_d || (d == best_d && (c & 1) == 0)) {\n            best = c;\n            best_d = d;\n        }\n    }\n    return sign | (uint8_t)best;\n}\n\nstatic",
                         "if (d < best_d || (d == best_d && (c & 1) == 1)) {\n            best = c;\n            best_d = d;\n        }\n    }\n    return sign | (uint8_t)best;\n}\n\nstatic"),
    "e5m2_saturates_to_infinity": ("        return sign | 0x7B;", "        return sign | 0x7C;"),
    "e5m2_format_ignored": ("return fmt == 1 ? oracle_e5m2_encode(y) : oracle_e4m3_encode(y);",
                            "return oracle_e4m3_encode(y);"),
    "copy_direction": ("memmove(k + dst * block_bytes, k + src * block_bytes, (size_t)block_bytes);",
                       "memmove(k + src * block_bytes, k + dst * block_bytes, (size_t)block_bytes);"),
    "copy_first_layer_only": ("for (int32_t l = 0; l < num_layers; l++) {\n            char *k",
                              "for (int32_t l = 0; l < 1; l++) {\n            char *k"),
}
PIN_FILES = [os.path.join(ROOT, "tests", name)
             for name in ("test_oracle.py", "test_oracle_rope.py", "test_oracle_fp8.py")]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new, 1))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c99", str(mutant_c), "-o", str(so), "-lm"],
                   check=True)
    env = dict(os.environ, PA_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
