"""Measured ceilings of the MI355X the attention kernels run on.

Runs the `ceilings` executable (built from csrc/ceilings.hip by build.py) as a child process and
returns its measurements: full-chip bf16 and E4M3 MFMA rates, HBM streaming read and copy
bandwidth, per-CU LDS read bandwidth, vector instruction costs and the MFMA/VALU co-execution
test. Usage: python -m roofline_attention_amd.ceilings
"""
from __future__ import annotations

import json
import os
import subprocess

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ceilings")


def measure(timeout: float = 300.0) -> dict:
    if not os.path.exists(EXE):
        raise FileNotFoundError(f"{EXE} is not built: run `python -m roofline_attention_amd.build`")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=timeout, check=True)
    return json.loads(r.stdout.strip().splitlines()[-1])


if __name__ == "__main__":
    print(json.dumps(measure(), indent=1))
