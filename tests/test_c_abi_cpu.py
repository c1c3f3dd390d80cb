"""The ABI is plain C: a C11 program compiled by gcc against include/paged_attn.h and
linked to the built library calls its host-only entry points (no GPU needed), and
what it prints agrees with the Python binding and the oracle's integer plan."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import segmented_attention_paged_amd._lib as _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(
    shutil.which("gcc") is None or not os.path.exists(_lib.LIB_PATH)
    or not os.path.isdir(ROCM_INCLUDE), reason="needs gcc, the ROCm headers and the built library")


@pytest.fixture(scope="module")
def run_c(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("c_abi") / "abi_host_check")
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-o", exe,
           "-L", lib_dir, "-lsapaged", f"-Wl,-rpath,{lib_dir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=120)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=120).stdout
    return {ln.split()[0]: ln.split()[1:] for ln in out.splitlines() if ln.strip()}


def test_version_and_plan(run_c):
    lib = _lib.load()
    assert " ".join(run_c["version"]) == lib.pa_version().decode()
    rc, *plan = [int(x) for x in run_c["plan"]]
    assert rc == _lib.PA_OK
    buf = (_lib.ctypes.c_int32 * 6)()
    assert lib.paged_attn_plan(64, 1, 32, 8, 128, 16, 512, 0, 0, buf) == _lib.PA_OK
    assert plan == list(buf)
    assert int(run_c["workspace"][0]) == lib.paged_attn_workspace_size(64, 1, 32, 8, 128, 16, 512, 0, 0)
    assert [int(x) for x in run_c["width"]] == [oracle.window_table_width(4096, 16, 16, 2048),
                                                oracle.window_table_width(0, 4, 16, 99)]


def test_describe_host_matches_oracle(run_c):
    f = run_c["describe"]
    assert int(f[0]) == _lib.PA_OK
    i = f.index("lens")
    lens = [int(x) for x in f[i + 1:i + 3]]
    j = f.index("table")
    table = np.array([int(x) for x in f[j + 1:j + 7]]).reshape(2, 3)
    k = f.index("ranges")
    ranges = np.array([int(x) for x in f[k + 1:k + 17]]).reshape(2, 2, 4)
    tab = np.array([[5, 9, 2, 11, 7, 3, 0], [8, 1, 4, 6, 10, 12, 13]], np.int32)
    ref_lens, ref_table = oracle.restrict_to_window([100, 37], tab, 20, 4, 16)
    assert lens == [int(x) for x in ref_lens]
    np.testing.assert_array_equal(table, ref_table[:, :3])
    for b in range(2):
        pages = -(-lens[b] // 16)
        for s, (first, count) in enumerate(oracle.split_page_ranges(pages, 2)):
            assert ranges[b, s, 0] == first and ranges[b, s, 1] == count
            t0, t1 = first * 16, min((first + count) * 16, lens[b])
            assert ranges[b, s, 2] == t0 and ranges[b, s, 3] == max(t1 - t0, 0)


def test_errors_are_status_codes(run_c):
    assert int(run_c["bad_dtype"][0]) == _lib.PA_ENOTSUP
    assert "query dtype" in " ".join(run_c["bad_dtype"][1:])
    assert int(run_c["empty"][0]) == _lib.PA_OK
