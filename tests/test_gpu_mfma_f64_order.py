"""The summation order of the fp64 matrix instruction, on the device.

The cross-layer projection and prediction compute each output as one fixed
sequence of fp64 additions (the reading of the Coral-KV pages' block-DPLR
predictor taken by the oracle: products of bf16 values, added in input
order).  They run on v_mfma_f64_16x16x4_f64, which is the same sequence only
if the instruction adds its four products to the accumulator one after
another in k order with an fp64 rounding each.  The self-check program built
with the library tests exactly that, bit for bit, on 2048 x 256 outputs whose
operands span wide exponent ranges (and counts the outputs where the
reverse order would differ, to show that the test can tell orders apart).
"""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(os.path.dirname(HERE), "kv_cache_quantization_head_amd", "selfcheck_mfma_f64")


@pytest.mark.gpu
def test_mfma_f64_adds_products_in_k_order():
    assert os.path.exists(EXE), f"{EXE} is missing: build the library first"
    print("selfcheck_mfma_f64", flush=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    m = re.search(r"outputs (\d+) differ_from_sequential (\d+) differ_from_reverse (\d+)", res.stdout)
    assert m, res.stdout + res.stderr
    outputs, seq, rev = (int(g) for g in m.groups())
    assert outputs == 2048 * 256
    assert rev > 1000, "the inputs do not separate summation orders"
    assert seq == 0 and res.returncode == 0
