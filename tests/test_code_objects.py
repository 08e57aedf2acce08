"""Resource usage of every kernel in this build, read from the gfx950 code
objects the build produced (no GPU needed): no kernel spills registers to
scratch memory, the eight-wave kernels fit two waves per SIMD, and the main
kernels use the register and LDS figures the design notes quote.

The device code object of each compiled source is the gfx950 entry of the
offload bundle in the object file's .hip_fatbin section; its AMDGPU metadata
note lists, per kernel, the VGPR and AGPR counts, the spill counts, the
private (scratch) segment size and the LDS (group segment) size."""
import glob
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ = os.path.join(ROOT, "exact_attention_127_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"

# kernel (demangled-name fragment) -> (VGPRs, LDS bytes) as quoted in the design notes
QUOTED = {
    "attn_mfma_bf16_kernelILi128ELi8E": (254, 131072),
    "attn_mfma_bf16_seq_kernelILi64E": (154, 32768),
    "attn_mfma_bf16_seq_kernelILi128E": (256, 65536),
    "attn_fp8_kernelILi128ELb0E": (152, 32768),
    "bwd_dkdv_kernelILi128ELi8E": (256, 132096),
    "bwd_dq_kernelILi128ELi8E": (254, 98304),
}


def _kernels():
    objs = sorted(p for p in glob.glob(os.path.join(OBJ, "*.hip.o")) if "attn_api" not in p)
    if not objs or not os.path.exists(os.path.join(LLVM, "clang-offload-bundler")):
        pytest.skip("library objects or ROCm LLVM tools not present")
    out = []
    for o in objs:
        with tempfile.TemporaryDirectory() as td:
            fb, co = os.path.join(td, "fatbin"), os.path.join(td, "gfx950.co")
            subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fb}", o,
                            os.path.join(td, "host.o")], check=True, capture_output=True)
            subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={fb}",
                            f"--output={co}", "--unbundle"], check=True, capture_output=True)
            notes = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", co], check=True,
                                   capture_output=True, text=True).stdout
        for blk in notes.split("  - .agpr_count:")[1:]:
            def field(k):
                return re.search(rf"\.{k}:\s+(\S+)", blk).group(1)
            out.append({"object": os.path.basename(o), "name": field("name"),
                        "agpr": int(blk.split()[0]), "vgpr": int(field("vgpr_count")),
                        "vgpr_spill": int(field("vgpr_spill_count")),
                        "sgpr_spill": int(field("sgpr_spill_count")),
                        "private": int(field("private_segment_fixed_size")),
                        "lds": int(field("group_segment_fixed_size"))})
    return out


def test_no_kernel_spills_or_uses_scratch():
    ks = _kernels()
    assert len(ks) >= 20
    for k in ks:
        assert k["private"] == 0 and k["vgpr_spill"] == 0 and k["sgpr_spill"] == 0, k


def test_eight_wave_kernels_fit_two_waves_per_simd():
    # 512 registers per SIMD lane, shared by the waves on it; AGPRs follow the
    # VGPRs at a 4-register granule
    for k in _kernels():
        if re.search(r"ELi8E", k["name"]):
            total = -(-k["vgpr"] // 4) * 4 + k["agpr"]
            assert total <= 256, k
            assert k["lds"] <= 160 * 1024, k


@pytest.mark.parametrize("frag", ["attn_mfma_bf16_seq_kernelILi64E", "attn_fp8_kernelI"])
def test_four_wave_forwards_fit_three_workgroups_per_cu(frag):
    # the one-tile-at-a-time d=64 kernel and the fp8 forward rely on three
    # four-wave workgroups per CU: at most 168 VGPRs (8-register granule) and
    # a third of the LDS
    hit = [k for k in _kernels() if frag in k["name"]]
    assert hit
    for k in hit:
        assert -(-k["vgpr"] // 8) * 8 + k["agpr"] <= 168, k
        assert 3 * k["lds"] <= 160 * 1024, k


def test_quoted_register_and_lds_figures():
    ks = _kernels()
    for frag, (vgpr, lds) in QUOTED.items():
        hit = [k for k in ks if frag in k["name"]]
        assert hit, frag
        for k in hit:
            assert (k["vgpr"], k["lds"]) == (vgpr, lds), k
