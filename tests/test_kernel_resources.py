"""Register, LDS and scratch budget of every gfx950 kernel (host-only check).

Compiles the kernel sources to gfx950 assembly and reads each kernel's
descriptor: the LDS it reserves, its unified VGPR + AGPR count and its
private (scratch) segment.  The tile configurations are chosen for a target
number of resident workgroups per CU, set by LDS (160 KiB per CU); the
registers must never be the tighter limit (512 per SIMD lane, allocated in
granules of 8, shared by the waves a workgroup places on each of the 4
SIMDs), and no kernel may spill to scratch.  A few extra registers in a
kernel near a boundary halve its occupancy without any other symptom.
"""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KDIR = os.path.join(ROOT, "structured_sparse_gemm_w24_amd", "csrc", "kernels")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ("gemm.hip", "splitk.hip", "tw_gemm.hip", "tw_gemm_i8.hip", "transpose.hip")

LDS_PER_CU = 160 * 1024
VGPRS_PER_SIMD_LANE = 512
VGPR_GRANULE = 8
SIMDS_PER_CU = 4


def _kernels(asm):
    """name -> {lds, vgpr, scratch, wg} from one assembly file."""
    out = {}
    for m in re.finditer(r"^\s*\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", asm, re.M | re.S):
        body = m.group(2)
        val = lambda k: int(re.search(r"\.amdhsa_" + k + r"\s+(\d+)", body).group(1))
        out[m.group(1)] = dict(lds=val("group_segment_fixed_size"), vgpr=val("next_free_vgpr"),
                               scratch=val("private_segment_fixed_size"))
    for m in re.finditer(r"\.max_flat_workgroup_size:\s*(\d+)\s*\n(?:.*\n){0,40}?\s*\.name:\s*(\S+)", asm):
        if m.group(2) in out:
            out[m.group(2)]["wg"] = int(m.group(1))
    return out


@pytest.fixture(scope="module")
def assembly():
    """source -> gfx950 assembly, compiled with the library's own flags."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from structured_sparse_gemm_w24_amd.build import HIP_FLAGS
    flags = [f for f in HIP_FLAGS if f not in ("-fPIC", "-fvisibility=hidden")]
    asm = {}
    with tempfile.TemporaryDirectory() as d:
        for src in SOURCES:
            out = os.path.join(d, src + ".s")
            cmd = [HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(KDIR, src), "-o", out]
            p = subprocess.run(cmd, capture_output=True, text=True)
            assert p.returncode == 0, p.stderr
            asm[src] = open(out).read()
    return asm


@pytest.fixture(scope="module")
def kernels(assembly):
    found = {}
    for text in assembly.values():
        found.update(_kernels(text))
    return found


def test_no_fused_multiply_add(assembly):
    """The epilogues round the product and the sum separately (float(acc) *
    scale, then + bias): no fp32 fused multiply-add may appear, except the
    compiler's own 64-bit integer division sequence (the 2^32 scalings)."""
    fma = re.compile(r"^\s*(v_(pk_)?fma(c|mk|ak)?_f32\S*|v_ma[cd]_f32\S*|v_fma_mix\S*)\s+(.*)$", re.M)
    bad = {}
    for src, text in assembly.items():
        hits = [m.group(0).strip() for m in fma.finditer(text)
                if "0x4f800000" not in m.group(4) and "0xcf800000" not in m.group(4)]
        if hits:
            bad[src] = hits[:3]
    assert bad == {}


def test_every_kernel_was_found(kernels):
    assert sum("gemm_kernel" in k for k in kernels) >= 20
    assert any("tw_gemm_kernel" in k for k in kernels)
    assert any("tw_gemm_i8_kernel" in k for k in kernels)
    assert any("splitk_reduce_kernel" in k for k in kernels)
    assert all("wg" in v for v in kernels.values()), [k for k, v in kernels.items() if "wg" not in v]


def test_no_kernel_spills_to_scratch(kernels):
    assert {k: v["scratch"] for k, v in kernels.items() if v["scratch"]} == {}


# gemm_kernel<KIND, EPI, Cfg<WM, WN, TM, TN, STAGES, GM, NTS, ROT, MP, PROD, NLD, DK>>:
# PROD (a group of loader waves beside the compute waves) is the tenth argument
_CFG = re.compile(r"CfgI(?:Li-?\d+E){6}(?:Lb[01]E){2}(?:Li-?\d+E)?(?:Lb([01])E)?(?:Li-?\d+E){0,2}E")


def _loader_waves(name):
    m = _CFG.search(name)
    return bool(m and m.group(1) == "1")


def test_registers_never_limit_occupancy_below_lds(kernels):
    """Tiles with loader waves are meant to run one workgroup per CU (their
    tile counts are chosen for that); they need registers for one."""
    bad = {}
    for name, v in kernels.items():
        waves = v["wg"] // 64
        alloc = -(-v["vgpr"] // VGPR_GRANULE) * VGPR_GRANULE
        # waves the register file holds per CU, in whole workgroups (a workgroup
        # of 4 or more waves spreads over the 4 SIMDs; one-wave workgroups fill
        # them one by one)
        by_regs = SIMDS_PER_CU * (VGPRS_PER_SIMD_LANE // alloc) // waves
        by_lds = LDS_PER_CU // v["lds"] if v["lds"] else 8
        want = 1 if _loader_waves(name) else min(by_lds, 8)
        if by_regs < want:
            bad[name] = dict(v, workgroups_by_registers=by_regs, workgroups_by_lds=by_lds)
    assert bad == {}


def test_loader_wave_kernels_were_found(kernels):
    assert sum(_loader_waves(k) for k in kernels if "gemm_kernel" in k) >= 8
