"""The NVFP4 quantizers encode E2M1 codes with the hardware FP32 -> FP4
conversion; their bytes equal the oracle's only if that conversion rounds
like the library's encoder (nearest, ties to the even code, saturating at 6,
sign kept).  The check program built beside the library compares the two on
every fp32 value within 64 ulps of each E2M1 midpoint and grid point (both
signs), on +-0, tiny, huge and denormal values and on a million seeded random
values.  The same program checks the quantizers' per-block quotients (one
correctly rounded reciprocal per block, two FMA residual corrections per
element) against IEEE division, bit for bit wherever the quotient reaches
1/8, for divisors from every E4M3 scale times global scales over 2^-120 ..
2^120 and dividends within 4 ulps of every E2M1 midpoint and grid point."""
import json
import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "mixed_precision_flashattention_amd", "mpfa_fp4_check")


def test_hardware_fp4_conversion_rounds_like_the_encoder():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "mpfa_fp4_check is not built (run __graft_entry__.build())"
    say("case: hardware FP32->E2M1 conversion against the library's encoder")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["mismatches"] == 0 and res["values"] > 1_000_000
    assert res["quotient_mismatches"] == 0 and res["quotients"] > 1_000_000
