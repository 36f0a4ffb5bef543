"""Exhaustive GPU check of the fp8 quantizer's fast steps (hardware E4M3
conversion, reciprocal bracket with a division fallback, fp32 outward rounding
of the summaries, packed wave maxima) and of the attention kernels' decoding of
codes to bf16 and split of probabilities into bf16 parts against their plain
forms, over every input they can get (tests/hip_programs/quantizer_check.hip). The codes,
scales and summaries these steps write are compared with the oracle's
quantizer in test_gpu_fp8.py."""
import subprocess

import pytest
import torch

import hip_programs as programs

pytestmark = pytest.mark.gpu


def test_quantizer_steps_exhaustive():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    programs.build()
    res = subprocess.run([programs.path("quantizer_check")], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True, timeout=120)
    print(res.stdout, flush=True)
    lines = [l for l in res.stdout.splitlines() if "mismatches" in l]
    assert len(lines) == 11, res.stdout
    assert res.returncode == 0 and all(l.endswith(": 0 mismatches") for l in lines), res.stdout
