"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
at least one pin catches each: the pins are only worth something if a dropped
term, a wrong sign, a wrong index or a transposed operand makes them fail."""
import os
import shutil
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "saga_oracle.c")

MUTATIONS = {
    "drop_inv_sqrt_d": ("a[t] = s * inv;", "a[t] = s;"),
    "gt_instead_of_ge": ("mask[t] = (uint8_t)(a[t] >= tau);", "mask[t] = (uint8_t)(a[t] > tau);"),
    "nth_off_by_one": ("double v = c[N - 1];", "double v = c[N < n ? N : N - 1];"),
    "key_head_modulo": ("return (int)(((int64_t)j * h_k) / h_q); }",
                        "return (int)(j % h_k); }"),
    "value_head_ceil": ("return (int)(((int64_t)j * h_v) / h_q); }",
                        "return (int)((((int64_t)j * h_v + h_q - 1) / h_q) % h_v); }"),
    "no_normalisation": ("double p = exp(a[t] - m) / den;", "double p = exp(a[t] - m);"),
    "softmax_sign": ("double p = exp(a[t] - m) / den;", "double p = exp(m - a[t]) / den;"),
    "refresh_phase": ("int refresh = (t % R) == 0;", "int refresh = (t % R) == 1 || t == 0;"),
    "transposed_key_index": ("bf16_to_double(k[c]);", "bf16_to_double(k[(c + 1) % d]);"),
    "ascending_sort": ("return (a < b) - (a > b);\n}\n\nstatic int cmp_desc_float",
                       "return (a > b) - (a < b);\n}\n\nstatic int cmp_desc_float"),
    "value_row_shift": ("const uint16_t *v = Vhead + t * (int64_t)d;",
                        "const uint16_t *v = Vhead + ((t + 1) % l_kv) * (int64_t)d;"),
    "stale_tau_every_step": ("if (refresh) tau_cur[r] = sao_nth_largest(a, l_kv, N);",
                             "if (t == 0) tau_cur[r] = sao_nth_largest(a, l_kv, N);"),
    # the growing-cache trajectory
    "growing_excludes_new_key": ("const int64_t len = l0 + t + 1;",
                                 "const int64_t len = l0 + t + (t > 0 ? 0 : 1);"),
    "growing_key_head_stride": ("sao_scores_row(q, K + ((int64_t)b * h_k + g) * cap * d, d, len, a);",
                                "sao_scores_row(q, K + ((int64_t)b * h_k + g) * len * d, d, len, a);"),
    "growing_value_head_stride": ("count[idx] = sao_attend_row(a, mk, V + ((int64_t)b * h_v + v) * cap * d, d, len,",
                                  "count[idx] = sao_attend_row(a, mk, V + ((int64_t)b * h_v + v) * len * d, d, len,"),
    "growing_refresh_phase": ("const int refresh_step = t % R == 0;",
                              "const int refresh_step = t % R == R - 1 || t == 0;"),
    "growing_never_refreshes": ("if (refresh_step) tau_cur[r] = sao_nth_largest(a, len, N);",
                                "if (t == 0) tau_cur[r] = sao_nth_largest(a, len, N);"),
    "growing_refresh_over_old_rows": ("if (refresh_step) tau_cur[r] = sao_nth_largest(a, len, N);",
                                      "if (refresh_step) tau_cur[r] = sao_nth_largest(a, l0 + 1, N);"),
}


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mut")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, workdir):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = workdir / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = workdir / f"lib_{name}.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", str(path), "-o",
                    str(so), "-lm"], check=True)
    lib = oracle.load(str(so))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutation {name}"
