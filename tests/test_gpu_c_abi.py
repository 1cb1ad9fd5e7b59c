"""GPU parity through the C ABI from a C program (tests/c/abi_gpu.c): no
Python or torch in the data path. This test writes seeded inputs and the hook
order to a file, the C program allocates the replicas' gradients with
hipMalloc, binds them, fires the hooks, finalizes and writes the gradients
back out; the result must equal the oracle's bit for bit, and so must the
launch log. The same program also binds with ddpb_bind_static."""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, say, assert_bits_equal
from oracle import reducer as OR
from workloads import gen as WG

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    require_gpu()
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    out = tmp_path_factory.mktemp("cabi") / "abi_gpu"
    libdir = os.path.dirname(D.HIP_LIB)
    # the HIP runtime headers need the platform named when compiled as C
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_gpu.c"), D.HIP_LIB,
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", str(out)],
                   check=True)
    return str(out)


CASES = [
    # numels, R, cap bytes, mode
    ([5, 300, 4100, 3, 8193, 64], 3, 4 * 5000, D.MODE_FUSED),
    ([5, 300, 4100, 3, 8193, 64], 8, 4 * 5000, D.MODE_STAGED),
    ([1000, 0, 20000, 7], 20, 0, D.MODE_FUSED),
    # + 2: bound with ddpb_bind_static (no allocation, reductions on the compute stream)
    ([5, 300, 4100, 3, 8193, 64], 3, 4 * 5000, D.MODE_FUSED + 2),
    ([5, 300, 4100, 3, 8193, 64], 8, 4 * 5000, D.MODE_STAGED + 2),
    ([1000, 0, 20000, 7], 20, 0, D.MODE_FUSED + 2),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_c_program_sync_matches_oracle(exe, tmp_path, case):
    numels, R, cap, mode = CASES[case]
    P = len(numels)
    say(f"C ABI case {case}: P={P} R={R} cap={cap} mode={mode}")
    host = [[WG.normal(WG.seed_of(8, r, v, case), n).numpy() for v, n in enumerate(numels)] for r in range(R)]
    order = WG.permutation(80 + case, P)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<iiiiq", 0x44445042, P, R, mode, cap))
        f.write(struct.pack(f"<{P}q", *numels))
        f.write(struct.pack(f"<i{P}i", P, *order))
        for r in range(R):
            for v in range(P):
                f.write(np.ascontiguousarray(host[r][v], dtype="<f4").tobytes())
    res = subprocess.run([exe, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    orc = OR.Reducer(numels, R, cap)
    want = [[h.copy() for h in row] for row in host]
    orc.bind(want)
    orc.sync(order)
    data = outp.read_bytes()
    total = sum(numels)
    got = np.frombuffer(data[:4 * total * R], dtype="<f4")
    at = 0
    for r in range(R):
        for v, n in enumerate(numels):
            assert_bits_equal(got[at:at + n], want[r][v], f"case {case} r={r} v={v}")
            at += n
    m = struct.unpack_from("<i", data, 4 * total * R)[0]
    log = [tuple(struct.unpack_from("<ii", data, 4 * total * R + 4 + 8 * i)) for i in range(m)]
    assert log == [tuple(x) for x in orc.launch_log]
