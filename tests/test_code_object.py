"""Checks of the built gfx950 code objects that need no GPU: every kernel in
the library keeps its state in registers and LDS. A kernel that spills
vector registers or puts an array in scratch memory still computes the
right values, so parity tests cannot see it, but it runs several times
slower (per-lane scratch traffic through the caches). The device code is
read from the library's offload bundles with the ROCm LLVM tools."""
import os
import re
import subprocess

import pytest

import long_context_sparse_12_amd as lcs

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

pytestmark = pytest.mark.skipif(
    not all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "clang-offload-bundler",
                                                             "llvm-readelf")),
    reason="ROCm LLVM tools not installed")


def _kernels(tmp_path):
    """[(name, {field: int})] from the AMDGPU metadata notes of every bundle."""
    fat = tmp_path / "fatbin.bin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", ".hip_fatbin=%s" % fat,
                    lcs.LIB_PATH, str(tmp_path / "lib.copy")], check=True, capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in the library"
    out = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        part = tmp_path / ("bundle%d.bin" % n)
        part.write_bytes(data[a:b])
        co = tmp_path / ("bundle%d.co" % n)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--targets=" + TARGET, "--input=%s" % part, "--output=%s" % co],
                       check=True, capture_output=True)
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(co)], check=True,
                               capture_output=True, text=True).stdout
        # one metadata map per kernel: its fields, then ".name:"
        for block in re.split(r"\n\s*- \.", notes)[1:]:
            name = re.search(r"\.name:\s+(\S+)", "." + block)
            if not name:
                continue
            fields = {k: int(v) for k, v in re.findall(
                r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count):\s+(\d+)",
                "." + block)}
            out.append((name.group(1), fields))
    return out


def test_no_kernel_uses_scratch(tmp_path):
    ks = _kernels(tmp_path)
    names = " ".join(n for n, _ in ks)
    for expected in ("idx_decode_kernel", "idx_prefill_kernel", "topk_final_kernel",
                     "sparse_mla_b_kernel", "sparse_mla_kernel", "combine_kernel",
                     "quant_rows_kernel", "topk_merge_kernel", "candidates_kernel",
                     "localize_kernel"):
        assert expected in names, expected
    # (SGPR spills go to VGPR lanes, not to memory, and are allowed)
    bad = [(n, f) for n, f in ks
           if f.get("private_segment_fixed_size", 0) or f.get("vgpr_spill_count", 0)]
    assert not bad, bad
