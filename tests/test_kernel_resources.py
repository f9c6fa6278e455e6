"""Resource checks of the built gfx950 kernels (no GPU needed).

The code objects inside libsla.so are read back (offload bundles in the
.hip_fatbin section, then the AMDGPU metadata note of each code object) and
every kernel must run without scratch memory: no per-lane stack
(private segment) and no spilled registers.  A dynamically indexed register
array or a spill puts scratch traffic on HBM in the hot loops, which the
compiler reports only as these two numbers."""
import os
import re
import shutil
import struct
import subprocess

import pytest

from helpers import ensure_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_linear_attention_mean_amd", "libsla.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _tool(name):
    path = os.path.join(LLVM, name)
    if os.path.exists(path):
        return path
    found = shutil.which(name)
    if not found:
        pytest.skip(f"{name} not available")
    return found


def _code_objects(fatbin: bytes):
    """gfx950 code objects of every uncompressed offload bundle in the section."""
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), fatbin)]
    assert starts, "no offload bundle in .hip_fatbin"
    out = []
    for s in starts:
        p = s + len(MAGIC)
        (n,) = struct.unpack_from("<Q", fatbin, p)
        p += 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, p)
            p += 24
            triple = fatbin[p:p + tlen].decode()
            p += tlen
            if "gfx950" in triple and size:
                out.append(fatbin[s + off:s + off + size])
    return out


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    ensure_library()
    tmp = tmp_path_factory.mktemp("co")
    fat = tmp / "sla.fatbin"
    subprocess.run([_tool("llvm-objcopy"), "--dump-section", f".hip_fatbin={fat}", LIB,
                    str(tmp / "copy.so")], check=True, capture_output=True)
    info = {}
    for idx, co in enumerate(_code_objects(fat.read_bytes())):
        path = tmp / f"co{idx}.o"
        path.write_bytes(co)
        notes = subprocess.run([_tool("llvm-readelf"), "--notes", str(path)], check=True,
                               capture_output=True, text=True).stdout
        # one metadata map per kernel: its fields, then .name / .symbol
        for blk in re.split(r"\n\s+- \.", notes):
            name = re.search(r"\.name:\s+(\S+)", blk)
            priv = re.search(r"private_segment_fixed_size:\s+(\d+)", blk)
            spill = re.search(r"vgpr_spill_count:\s+(\d+)", blk)
            if name and priv and spill:
                info[name.group(1)] = (int(priv.group(1)), int(spill.group(1)))
    assert info, "no kernel metadata found"
    return info


def test_every_hot_kernel_is_present(kernels):
    names = " ".join(kernels)
    for k in ("attn_fwd_kernel", "aggregate_kernel", "kv_state_kernel", "classify_kernel",
              "bwd_prep_kernel", "bwd_kv_kernel", "bwd_q_kernel"):
        assert k in names, k


def test_no_kernel_uses_scratch(kernels):
    bad = {k: v for k, v in kernels.items() if v != (0, 0)}
    assert not bad, f"kernels with (private segment bytes, spilled VGPRs): {bad}"
