"""Serialized-launch check: the chunk forward (every gate), its backward, the
training path, the preconditioner scan and the decode step give the same bits when
the HIP runtime serializes every kernel launch (AMD_SERIALIZE_KERNEL=3: wait before
and after each kernel) as in the normal asynchronous run.  A difference would mean a
result that depends on how kernels of one call overlap in time.  The serialized
run is a child process (the variable is read when the runtime starts)."""

import os
import subprocess
import sys

import numpy as np
import pytest

from tests.gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(300)
def test_serialized_launches_give_the_same_bits(tmp_path):
    need_gpu()
    from tests.serial_run import run_all
    say("serialized launches: normal run")
    ref = run_all()
    path = tmp_path / "serial.npz"
    env = dict(os.environ, AMD_SERIALIZE_KERNEL="3")
    say("serialized launches: child run with AMD_SERIALIZE_KERNEL=3")
    r = subprocess.run([sys.executable, os.path.join(HERE, "serial_run.py"), str(path)], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    got = np.load(path)
    assert sorted(got.files) == sorted(ref), (sorted(got.files), sorted(ref))
    for n in ref:
        assert np.array_equal(got[n], ref[n]), n
    say(f"serialized launches: {len(ref)} results equal bit for bit")
