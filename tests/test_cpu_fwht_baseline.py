"""The fast CPU baseline (bench_cpu_fwht.c, an O(n log n) FWHT + int4
quantizer written apart from the oracle) computes what the oracle computes:
codes and fp16 scales match under the same rules as the GPU parity checks."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import hr_inputs
import oracle
from parity import check_quant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("n,group", [(2048, 128), (2048, 32), (512, 64)])
def test_cpu_fwht_baseline_matches_oracle(tmp_path, n, group):
    import bench
    exe = bench.build_cpu_fwht(str(tmp_path))
    inp = hr_inputs.rht_inputs(rows=48, n=n, seed=700 + group)
    xf, sf, of = tmp_path / "x.bf16", tmp_path / "s.i8", tmp_path / "out.bin"
    inp.x.view(__import__("torch").int16).numpy().tofile(xf)
    inp.signs.astype(np.int8).tofile(sf)
    r = subprocess.run([exe, str(xf), str(sf), "48", str(n), str(group), "2", str(of)],
                       capture_output=True, text=True, check=True)
    assert '"rows": 48' in r.stdout
    raw = np.fromfile(of, dtype=np.uint8)
    codes = raw[:48 * n // 2].reshape(48, n // 2)
    scales = raw[48 * n // 2:].view(np.float16).reshape(48, n // group)
    y64 = oracle.hadamard.rht(inp.x.float().numpy(), inp.signs)
    check_quant(codes, scales, y64, group, "f16")
