"""LDS poisoning: a build of the library whose kernels fill LDS with NaN
bytes at entry and ahead of every HBM -> LDS copy (``-DATTN_DEBUG_POISON=1``,
``libattn_mi355x_poison.so``) runs the calls of tests/poison_cases.py in a
child process; the outputs must equal this process's normal build bit for
bit.  A kernel that read LDS no write of its launch (or of the current copy
into a reused ring slot) had reached would see NaN there instead of the data
or zeros the normal build happens to hold, and the outputs would differ."""

import os
import subprocess
import sys

import pytest
import torch

import poison_cases
from gpu_util import ensure_built
from online_softmax_exact_amd import build as B

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _bits(t):
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t


def test_poisoned_lds_build_matches_bitwise(tmp_path):
    ensure_built()
    if not os.path.exists(B.POISON_LIB):
        pytest.fail(f"{B.POISON_LIB} is missing: build() links it")
    path = str(tmp_path / "poisoned.pt")
    env = dict(os.environ, ATTN_MI355X_LIBRARY=B.POISON_LIB,
               PYTHONPATH=os.pathsep.join([ROOT, HERE, os.environ.get("PYTHONPATH", "")]))
    print("child: poison_cases with", B.POISON_LIB, flush=True)
    res = subprocess.run([sys.executable, os.path.join(HERE, "poison_cases.py"), path], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    poisoned = torch.load(path, weights_only=True)
    normal = poison_cases.compute()
    assert poisoned.keys() == normal.keys()
    for name, ref in normal.items():
        got = poisoned[name]
        assert got.dtype == ref.dtype and got.shape == ref.shape, name
        assert torch.equal(_bits(got), _bits(ref)), f"{name}: the poisoning build differs"
        if ref.is_floating_point():
            assert not torch.isnan(ref.float()).any(), f"{name}: NaN in the normal build"
