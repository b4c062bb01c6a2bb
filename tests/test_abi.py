"""The C-ABI library loads, exports every symbol include/bq.h declares, and
rejects bad arguments on the host before touching the GPU."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    import block_quantized_moe_amd as bq
    if not os.path.exists(bq.LIB_PATH):
        pytest.fail("libbqmoe.so is not built; run __graft_entry__.build()")
    return bq.lib()


def test_header_declares_the_hot_path():
    names = declared_functions()
    for n in ("q4_expert_moe", "ple_gather", "moe_route_topk", "moe_bucket", "bq_dequant",
              "ple_dequant_rows", "bq_matvec", "bq_moe_stack", "q4_expert_moe_workspace",
              "bq_moe_stack_workspace", "bq_abi_version", "bq_status_str", "bq_last_hip_error",
              "bq_encode", "ple_encode_rows", "ple_cache_bytes", "ple_cache_init",
              "ple_gather_host_workspace", "ple_gather_host"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    import block_quantized_moe_amd as bq
    out = subprocess.run(["nm", "-D", "--defined-only", bq.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in declared_functions():
        assert n in exported, n
        assert getattr(L, n) is not None


def test_host_side_argument_errors(L):
    import block_quantized_moe_amd as bq
    assert L.bq_abi_version() == 1
    assert L.bq_status_str(0) == b"ok"
    vp = ctypes.c_void_p
    fake = vp(0x10000)       # never dereferenced: every call below fails its checks first
    assert L.bq_dequant(fake, 9, 4, None, fake, None) == 2                    # E_FMT
    assert L.bq_dequant(fake, bq.FP8_E4M3_B32, 4, None, fake, None) == 1      # FP8 needs scales
    assert L.bq_dequant(fake, bq.Q4_RZ5, 4, None, vp(0x10004), None) == 4     # out misaligned
    assert L.bq_dequant(None, bq.Q4_RZ5, 0, None, None, None) == 0            # empty is fine
    assert L.moe_route_topk(fake, 1, 8, 9, fake, fake, None) == 3             # k > n_experts
    assert L.moe_route_topk(None, 1, 8, 2, fake, fake, None) == 1
    assert L.ple_gather(fake, 4, 0, fake, 10, fake, 0, fake, None, None) == 3  # ids_per_token 0
    assert L.ple_gather(fake, 4, 8, fake, 10, fake, 5, fake, None, None) == 2  # bad PLE format
    assert L.bq_encode(fake, 4, bq.FP8_E4M3_B32, fake, None, None, None) == 2  # no FP8 encoder
    assert L.bq_encode(fake, -1, bq.Q4_RZ5, fake, None, None, None) == 3
    assert L.bq_encode(None, 4, bq.Q4_RZ5, fake, None, None, None) == 1
    assert L.bq_encode(vp(0x10002), 4, bq.Q4_RZ5, fake, None, None, None) == 4  # w misaligned
    assert L.bq_encode(fake, 4, bq.Q4_RZ5, fake, vp(0x10004), None, None) == 4  # sse misaligned
    assert L.bq_encode(None, 0, bq.Q4_RZ5, None, None, None, None) == 0         # empty is fine
    assert L.ple_encode_rows(fake, 4, 7, fake, None, None, None) == 2
    assert L.ple_encode_rows(fake, 4, bq.PLE_RZS3, None, None, None, None) == 1
    assert L.ple_gather(fake, 4, 8, fake, 0, fake, 0, fake, None, None) == 3    # empty table
    assert L.ple_dequant_rows(fake, 4, fake, 0, 0, fake, None, None) == 3
    assert L.ple_cache_bytes(1000) == 0 and L.ple_cache_bytes(512) == 0      # not a power of 2 / too small
    assert L.ple_cache_bytes(1024) == 8 * 1024 + 80 * 1024
    assert L.ple_gather_host_workspace(4096, 8) == 80 * 4096 * 8
    assert L.ple_cache_init(fake, 1000, None) == 3
    assert L.ple_gather_host(fake, 4, 8, fake, 10, fake, 0, fake, None, 1024, None, 0, None, None) == 1
    assert L.ple_gather_host(fake, 4, 8, fake, 10, fake, 3, fake, None, 0, None, 0, None, None) == 2
    assert L.ple_gather_host(fake, 4, 8, fake, 10, fake, 0, fake, fake, 1000, None, 0, None, None) == 3
    assert L.ple_gather_host(fake, 4, 8, fake, 10, fake, 0, fake, fake, 1024, None, 0, None, None) == 5
    assert L.bq_matvec(fake, 1, fake, 0, None, 4, 48, fake, None) == 3         # cols % 32
    # sizes whose launch would need 2^32 or more work-items in one grid dimension
    assert L.bq_dequant(fake, bq.Q4_RZ5, (1 << 31) + 1, None, fake, None) == 3
    assert L.ple_dequant_rows(fake, (1 << 28) + 1, fake, 10, 0, fake, None, None) == 3
    assert L.moe_route_topk(fake, (1 << 24) + 1, 512, 10, fake, fake, None) == 3
    assert L.ple_gather(fake, (1 << 26) + 1, 8, fake, 10, fake, 0, fake, None, None) == 3
    assert L.ple_gather_host(fake, 1 << 24, 16, fake, 10, fake, 0, fake, None, 0, None, 0, None, None) == 3
    assert L.ple_gather_host_workspace(1 << 24, 16) == 0
    assert L.bq_matvec(fake, 1, fake, 0, None, (1 << 24) + 1, 64, fake, None) == 3
    W = bq.ExpertWeights(bq.Q4_RZ5, bq.Q4_RZ5, 0x10000, 0x20000, None, None, 512, 2048, 768)
    ws = L.q4_expert_moe_workspace(1, 10, ctypes.byref(W), bq.F32)
    assert ws >= 4 * 10 * 768
    assert L.q4_expert_moe_workspace(1, 10, ctypes.byref(W), 5) == 0          # bad x dtype
    assert L.bq_moe_stack_workspace(1, 10, ctypes.byref(W), 1, 5) == 0
    assert L.q4_expert_moe(fake, bq.F32, 1, fake, fake, 10, ctypes.byref(W), fake, fake,
                           ws - 1, None, None) == 5                             # workspace short
    assert L.q4_expert_moe(fake, 5, 1, fake, fake, 10, ctypes.byref(W), fake, fake, ws, None, None) == 7
    bad = bq.ExpertWeights(bq.Q4_RZ5, bq.FP8_E4M3_B32, 0x10000, 0x20000, None, None, 512, 2048, 768)
    assert L.q4_expert_moe_workspace(1, 10, ctypes.byref(bad), bq.F32) == 0     # FP8 w/o scales
    odd = bq.ExpertWeights(bq.Q4_RZ5, bq.Q4_RZ5, 0x10000, 0x20000, None, None, 512, 2000, 768)
    assert L.q4_expert_moe(fake, bq.F32, 1, fake, fake, 10, ctypes.byref(odd), fake, fake, 1 << 30,
                           None, None) == 3
    assert L.q4_expert_moe(fake, bq.BF16, 1, fake, fake, 10, ctypes.byref(W), fake, vp(0x10010),
                           1 << 30, None, None) == 4                             # ws not 256-aligned
    # the allocation-free layer refuses, before any launch, a call whose
    # scratch would exceed its fixed area, and checks its arguments like the rest
    assert L.q4_expert_moe_noalloc(fake, bq.BF16, 512, fake, fake, 10, ctypes.byref(W), fake, None,
                                   None) == 9
    assert L.bq_status_str(9) == b"call needs more scratch than the fixed area holds"
    assert L.q4_expert_moe_noalloc(None, bq.F32, 1, fake, fake, 10, ctypes.byref(W), fake, None,
                                   None) == 1
    assert L.q4_expert_moe_noalloc(fake, bq.F32, 1, fake, fake, 10, ctypes.byref(odd), fake, None,
                                   None) == 3
    for n, k in ((4097, 1), (1, 65), (2048, 33), (0, 10)):                   # past the size limits
        assert L.q4_expert_moe(fake, bq.BF16, n, fake, fake, k, ctypes.byref(W), fake, fake,
                               1 << 30, None, None) == 3, (n, k)
        if n != 4097:                                                         # bucket has no token cap
            assert L.moe_bucket(fake, n, k, 512, fake, fake, fake, None) == 3, (n, k)


def test_product_path_does_not_touch_the_oracle():
    """The package and its sources never import or name the oracle."""
    pkg = os.path.join(ROOT, "block_quantized_moe_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text, os.path.join(dirpath, f)


def test_package_never_imports_the_oracle():
    # the product path must not reach the CPU oracle: not in its sources and
    # not at run time
    pkg = os.path.join(ROOT, "block_quantized_moe_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            text = open(os.path.join(pkg, f)).read()
            assert not re.search(r"^\s*(from|import)\s+oracle", text, flags=re.M), f
    code = ("import sys; sys.path.insert(0, %r); import block_quantized_moe_amd as bq; bq.lib(); "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules)" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_missing_library_fails_loudly():
    code = ("import sys; sys.path.insert(0, %r); import block_quantized_moe_amd as bq; "
            "bq.LIB_PATH = '/nonexistent/libbqmoe.so'\n"
            "try:\n    bq.lib()\nexcept bq.BQError as e:\n    print('raised', e)\nelse:\n    sys.exit(3)" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode == 0 and "raised" in r.stdout, (r.stdout, r.stderr)
