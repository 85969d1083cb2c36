"""The prefill's fp64 exp for non-positive arguments (query_adaptive_sparse_amd/csrc/sd_exp.h),
built for the host from the same source and compared with numpy's exp: within 1.5 ulp over the whole
range down to the smallest subnormal result, exactly 1 at 0, and 0 below the underflow threshold
(clamped arguments, NaN included)."""
import os
import shutil
import subprocess
from pathlib import Path

import numpy as np
import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "query_adaptive_sparse_amd" / "csrc"

PROGRAM = r"""
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "sd_exp.h"

int main(int argc, char** argv) {
  const long n = std::atol(argv[3]);
  std::vector<double> x(n), y(n);
  FILE* f = std::fopen(argv[1], "rb");
  if (!f || std::fread(x.data(), sizeof(double), n, f) != size_t(n)) return 2;
  std::fclose(f);
  static const double tab[64] = {SD_EXP2_64_TABLE};
  const sd::ExpC c = sd::exp_consts();
  for (long i = 0; i < n; ++i) y[i] = sd::exp_nonpos(x[i], tab, c);
  f = std::fopen(argv[2], "wb");
  if (!f || std::fwrite(y.data(), sizeof(double), n, f) != size_t(n)) return 3;
  std::fclose(f);
  return 0;
}
"""


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_exp_nonpos_within_2ulp(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    src, exe = tmp_path / "exp_check.hip", tmp_path / "exp_check"
    src.write_text(PROGRAM)
    # host code only: nothing touches a GPU
    subprocess.run([hipcc, "-x", "hip", "--cuda-host-only", "-O2", "-ffp-contract=off", "-I", str(CSRC), str(src),
                    "-o", str(exe)], check=True, timeout=300, capture_output=True)
    rng = np.random.default_rng(0)
    special = np.array([0.0, -0.0, -1e-300, -1e-17, -2.0 ** -30, -0.5, -1.0, -np.log(2.0), -700.0, -708.39,
                        -709.0, -740.0, -744.4, -745.1])
    x = np.concatenate([-rng.exponential(3.0, 400_000), -rng.uniform(0.0, 745.0, 400_000),
                        -np.arange(0, 4096) * np.log(2.0) / 64, special])
    under = np.array([-745.2, -800.0, -1100.0, -1e300, -np.inf, np.nan])
    xin = np.concatenate([x, under])
    xin.astype("<f8").tofile(tmp_path / "x.bin")
    subprocess.run([str(exe), str(tmp_path / "x.bin"), str(tmp_path / "y.bin"), str(len(xin))], check=True,
                   timeout=120)
    y = np.fromfile(tmp_path / "y.bin", dtype="<f8")
    got, tail = y[:len(x)], y[len(x):]
    ref = np.exp(x)
    ulp = np.spacing(ref)  # the subnormal spacing for subnormal results
    err = np.abs(got - ref) / ulp
    normal = ref >= np.finfo(np.float64).tiny
    print(f"max error {err[normal].max():.2f} ulp (normal results), {err[~normal].max():.2f} subnormal ulp "
          f"(subnormal results), mean {err.mean():.3f} ulp over {len(x)} arguments")
    assert err.max() <= 1.5, x[np.argmax(err)]
    i0 = len(x) - len(special)
    assert got[i0] == 1.0 and got[i0 + 1] == 1.0  # exp(0), exp(-0)
    assert np.all(tail == 0.0), tail


def test_exp_table_is_the_generators():
    """The 2^(j/64) table in sd_exp.h is the one gen_exp_table.py computes (each value correctly
    rounded from a 60-digit decimal), and each entry is within half an ulp of 2^(j/64) in long
    double arithmetic."""
    import re
    import importlib.util
    spec = importlib.util.spec_from_file_location("gen_exp_table", ROOT / "query_adaptive_sparse_amd" / "gen_exp_table.py")
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    text = (CSRC / "sd_exp.h").read_text()
    body = text[text.index("#define SD_EXP2_64_TABLE"):text.index("namespace sd")]
    vals = [float.fromhex(h) for h in re.findall(r"0x[0-9a-f.]+p[+-]\d+", body)]
    assert vals == gen.table()
    for j, v in enumerate(vals):
        exact = np.power(np.longdouble(2), np.longdouble(j) / 64)
        assert abs(np.longdouble(v) - exact) <= np.longdouble(np.spacing(v)) / 2, j
