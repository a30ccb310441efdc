"""The C ABI used from plain C++ (tests/c_abi_driver.cpp): device memory from
hipMalloc, no torch in the process.  Its gdn_fwd output must match the fp64
oracle at the bf16 bar and equal, bit for bit, what the Python binding
returns for the same inputs; its gdn_chunk_step rollout must equal the pass."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from hybrid_linear_attention_gdn_amd import gdn
from hybrid_linear_attention_gdn_amd.inputs import Workload, make_inputs
from oracle.recurrence import gdn_recurrence
from tests.helpers import TOL_BF16, rel_max_err, state_err, to_device

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_driver")


def test_c_abi_from_plain_cpp(tmp_path):
    if not os.path.exists(EXE):
        pytest.skip("tests/c_abi_driver is not built (__graft_entry__.build() builds it)")
    w = Workload("c_abi", 1, 4, 4, 120, "bf16", 17, state_std=0.02)  # T = 480: six calls of 80 tokens
    inp = make_inputs(w)
    B, T, H, D = inp.q_bits.shape
    Tc = 80
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as fh:
        np.array([B, T, H, D, Tc], np.int32).tofile(fh)
        for a in (inp.q_bits, inp.k_bits, inp.v_bits):
            np.ascontiguousarray(a).view(np.uint16).tofile(fh)
        for a in (inp.g, inp.beta, inp.state0):
            np.ascontiguousarray(a, np.float32).tofile(fh)
    print(f"case c_abi_driver B={B} T={T} H={H} D={D}", flush=True)
    sys.stdout.flush()
    r = subprocess.run([EXE, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(fout, np.float32)
    nx, ns = B * T * H * D, B * H * D * D
    assert raw.size == 2 * (nx + ns)
    o_c, st_c = raw[:nx].reshape(B, T, H, D), raw[nx:nx + ns].reshape(B, H, D, D)
    o_roll, st_roll = raw[nx + ns:2 * nx + ns].reshape(B, T, H, D), raw[2 * nx + ns:].reshape(B, H, D, D)
    o_ref, s_ref = gdn_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.state0)
    assert rel_max_err(o_c, o_ref) <= TOL_BF16 and state_err(st_c, s_ref) <= TOL_BF16
    np.testing.assert_array_equal(o_roll, o_c)
    np.testing.assert_array_equal(st_roll, st_c)
    # the Python binding on the same inputs gives the same bits
    q, k, v, g, beta, s0 = to_device(inp)
    o_py, st_py = gdn.gdn_fwd(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o_py.cpu().numpy(), o_c)
    np.testing.assert_array_equal(st_py.cpu().numpy(), st_c)
