"""Resource use of every kernel in the built library (CPU only: reads the
gfx950 code objects that the in-tree build embedded in libattn_mi355x.so).

No kernel may use a private (scratch) segment: register arrays demoted to
scratch memory made the head-dim-256 prefill fifty times slower before its
step loop was fully unrolled.  Every kernel's LDS must fit the 160 KB of a
CU.  The ROCm LLVM tools that read the code objects are part of this image;
the test skips when the library has not been built.
"""
import pathlib
import re
import shutil
import subprocess
import tempfile
import textwrap

import pytest
import yaml

ROOT = pathlib.Path(__file__).resolve().parents[1]
LIB = ROOT / "attention_attn_fwd_06_amd" / "libattn_mi355x.so"
LLVM = pathlib.Path("/opt/rocm/llvm/bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
LDS_BYTES = 160 * 1024


def _kernels():
    if not LIB.exists():
        pytest.skip("library not built")
    tools = [LLVM / t for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    if not all(t.exists() for t in tools):
        pytest.skip("ROCm LLVM tools not found")
    objcopy, bundler, readelf = map(str, tools)
    out = {}
    with tempfile.TemporaryDirectory() as td:
        fat = pathlib.Path(td) / "fat.bin"
        subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", str(LIB), str(pathlib.Path(td) / "x.so")],
                       check=True, capture_output=True)
        data = fat.read_bytes()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
        assert starts, "no offload bundle in the library"
        for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            part = pathlib.Path(td) / f"b{n}.bin"
            part.write_bytes(data[a:b])
            co = pathlib.Path(td) / f"co{n}.elf"
            subprocess.run([bundler, "--unbundle", "--type=o", f"--input={part}",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                           check=True, capture_output=True)
            notes = subprocess.run([readelf, "--notes", str(co)], check=True, capture_output=True, text=True).stdout
            doc = notes[notes.index("---"):]
            doc = doc[:doc.index("\n...")] if "\n..." in doc else doc
            meta = yaml.safe_load(textwrap.dedent(doc.split("---", 1)[1]))
            for k in meta["amdhsa.kernels"]:
                # (VGPR spills into AGPRs need no private segment and are allowed)
                out[k[".name"]] = {f: k.get("." + f, 0) for f in
                                   ("private_segment_fixed_size", "group_segment_fixed_size", "vgpr_spill_count")}
    shutil.rmtree(td, ignore_errors=True)
    return out


def test_no_kernel_uses_scratch_and_lds_fits():
    kernels = _kernels()
    # the families the library launches, including the head-dim-256 instances
    for fam in ("prefill_fwd_kernelILi256", "prefill_fwd_kernelILi128", "decode_gqa_mfma_kernelILi256",
                "decode_gqa_mfma_kernelILi128", "decode_chunk_kernel", "lse_merge_kernel"):
        assert any(fam in n for n in kernels), fam
    for name, f in kernels.items():
        assert f.get("private_segment_fixed_size", 0) == 0, (name, f)
        assert f.get("group_segment_fixed_size", 0) <= LDS_BYTES, (name, f)
