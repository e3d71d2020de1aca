"""The C ABI used from C: tests/c_abi_check.c includes include/spot.h as
strict C11 (-Wall -Wextra -Werror -pedantic), links against the built
library and calls the host-only entry points (no GPU needed).  The
descriptor layout is checked by the C compiler itself (static assertions),
the results against the same calls made through the Python binding."""
import os
import shutil
import subprocess

import pytest

from block_sparse_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_check.c")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(ROOT, "block_sparse_attention_amd", "libspot.so")


@pytest.fixture(scope="module")
def c_results(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    assert os.path.exists(LIB), "build the library first (__graft_entry__.build())"
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_check")
    libdir = os.path.dirname(LIB)
    subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{INCLUDE}", SRC, "-o", exe,
                    f"-L{libdir}", "-l:libspot.so", f"-Wl,-rpath,{libdir}"], check=True, capture_output=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=120).stdout
    res = {}
    for line in out.splitlines():
        key, _, val = line.partition(" ")
        res[key] = val
    return res


def test_c_program_sees_the_library_version(c_results):
    assert int(c_results["version"]) == B.ABI_VERSION == B.spot_version()
    assert c_results["status_invalid"] == B.load_library().spot_status_string(B.SPOT_ERR_INVALID).decode()


def test_c_program_validation_statuses(c_results):
    assert int(c_results["null_desc_status"]) == B.SPOT_ERR_INVALID
    assert int(c_results["null_desc_error_set"]) == 1
    assert int(c_results["select_null_status"]) == B.SPOT_ERR_INVALID
    assert int(c_results["bad_version_status"]) == B.SPOT_ERR_INVALID
    assert int(c_results["bad_head_dim_status"]) == B.SPOT_ERR_UNSUPPORTED


def test_c_program_workspace_sizes_match_the_binding(c_results):
    d = B.make_desc(dtype=B.SPOT_BF16, batch=16, hq=32, hkv=8, d=128, q_len=1, kv_len=131072, block=16,
                    top_p=0.9, score_kind=B.SPOT_SCORE_RELU_INDEXER, h_idx=4, d_idx=64)
    assert int(c_results["decode_workspace_status"]) == B.SPOT_OK
    assert int(c_results["decode_workspace_bytes"]) == B.spot_workspace_size(d, B.SPOT_OP_DECODE) > 0
    assert int(c_results["select_workspace_bytes"]) == B.spot_workspace_size(d, B.SPOT_OP_SELECT_TOPP)
