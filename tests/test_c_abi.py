"""The C ABI used from C: tests/c/abi_host.c is compiled with gcc against
include/libcq.h, linked to libcq.so and run (host-only entry points, no
GPU); its printed results are checked against the oracle and hand values."""

import os
import shutil
import subprocess

import pytest

from oracle import cq_oracle as O
import rotated_codebook_bit_amd as cq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def output(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib_dir = os.path.dirname(cq.LIB_PATH)
    if not os.path.exists(cq.LIB_PATH):
        pytest.fail(f"{cq.LIB_PATH} is missing: build the library first")
    exe = str(tmp_path_factory.mktemp("cabi") / "abi_host")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), f"-L{lib_dir}", "-lcq",
                    f"-Wl,-rpath,{lib_dir}", "-o", exe], check=True, capture_output=True, text=True)
    res = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=60)
    return {line.split()[0]: line.split()[1:] for line in res.stdout.splitlines()}


def test_c_host_calls(output):
    assert output["version"][0].startswith("libcq")
    assert output["layout"] == ["0", "2400", str(2400 * 32)]
    shapes = [(4096, 4096), (300, 1000), (2, 130)]
    assert output["model_bytes"] == ["0", str(O.model_bytes(shapes, 2))]
    assert output["model_bytes_trits"] == ["0", str(O.model_bytes(shapes, O.TERNARY_TRITS))]
    po, no, total = O.blob_offsets(shapes, 2)
    assert output["blob"] == ["0"] + [str(v) for v in po + no + [total]]
    assert output["ternary"][:2] == ["0", "3"]
    assert [float(v) for v in output["ternary"][2:]] == pytest.approx([-1.2240064, 0.0, 1.2240064], abs=1e-7)
    assert output["builtin2"][:2] == ["0", "4"]
    assert [float(v) for v in output["builtin2"][2:]] == pytest.approx(list(cq.codebook(2)), abs=1e-7)
    want = O.lloyd_max(__import__("numpy").array([-2.0, -1.0, 1.0, 3.0]), 2, 10)
    assert output["lloyd1"][:2] == ["0", "2"]
    assert [float(v) for v in output["lloyd1"][2:]] == pytest.approx(list(want), abs=1e-6)
    assert output["bad_bits"][0] == "-2"
    assert output["bad_k"] == ["-4"]
