"""The oracle's pins must fail on plausible slips planted in the oracle.

Each case copies oracle/oracle.cpp, applies one textual mutation (a dropped
bias, the group index taken along the output axis, gate and up swapped, a
transposed down projection, a reversed tie-break, weights not renormalised,
combine weights dropped, an unstable scatter, a negated router bias), builds
it with g++ into a temporary directory and runs the pin suite against it in a
subprocess. The suite must fail for every mutation. CPU only.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")

MUTATIONS = {
    "bias_dropped": ("bf16_value(scale[n * groups + g]) +\n         bf16_value(bias[n * groups + g]);",
                     "bf16_value(scale[n * groups + g]) +\n         0 * bf16_value(bias[n * groups + g]);"),
    "group_along_rows": ("const int64_t g = c / kGroup;", "const int64_t g = n % groups;"),
    "gate_up_swapped": ("h[n] = silu(g) * u;", "h[n] = silu(u) * g;"),
    "tie_to_higher_index": ("return l[a] > l[b];", "return l[a] >= l[b];"),
    "not_renormalised": ("zsel += p[idx[j]];", "zsel += 1.0 / k;"),
    "down_transposed": ("dequant_one(qd, sd, bd, I, r, n)", "dequant_one(qd, sd, bd, H, n % H, r % I)"),
    "combine_unweighted": ("acc[r] += static_cast<double>(w[j]) * d[r];", "acc[r] += d[r] / k;"),
    "scatter_unstable": ("const int64_t pos = offsets[e] + fill[e]++;",
                         "const int64_t pos = offsets[e] + hist[e] - 1 - fill[e]++;"),
    "router_bias_negated": ("if (rbias) acc += static_cast<double>(rbias[e]);",
                            "if (rbias) acc -= static_cast<double>(rbias[e]);"),
    "shared_expert_dropped": ("const double m = (e == E) ? 1.0 : mask[e];",
                              "const double m = (e == E) ? 0.0 : mask[e];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = tmp_path / "oracle_mut.cpp"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["g++", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c++17",
                    str(mutated), "-o", str(lib)], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
