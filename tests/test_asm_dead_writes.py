"""No kernel of the library writes a vector register that it never reads (see
tests/asm_check.py): the pattern of a miscompile found in one instantiation,
which the library no longer builds.  From the same assembly, the register
budgets the measured launch shapes rely on.  Compiles the kernel sources to
gfx950 assembly on the CPU (about 45 s)."""
import os

import pytest

import asm_check


@pytest.fixture(scope="module")
def compiled():
    return asm_check.check_with_metadata()


@pytest.fixture(scope="module")
def kernels(compiled):
    return compiled[0]


def _regs(meta, name):
    """Registers a lane of the kernel holds (VGPRs and AGPRs share one file of
    512), rounded up to the allocation granule of 8."""
    m = meta[name]
    n = m["vgpr_count"] + m.get("agpr_count", 0)
    return -(-n // 8) * 8


def test_every_kernel_reads_what_it_writes(kernels):
    assert len(kernels) > 50  # every kernel source was compiled and scanned
    bad = [(src, fn, dead) for src, fn, _, dead in kernels if dead]
    assert not bad, "dead vector-register writes (a dropped copy?): " + "; ".join(
        f"{src} {fn}: " + ", ".join(f"{r[0]}{r[1]} <- {d}" for r, d in sorted(dead.items())[:3])
        for src, fn, dead in bad)


def test_the_miscompiled_instantiation_is_not_built(kernels):
    names = {fn for _, fn, _, _ in kernels}
    # ua_decode_sk_kernel<256, 32, bf16 or f16, 16-bit K/V, QQ bias>
    assert not any(n.startswith("_ZN2ua19ua_decode_sk_kernelILi256ELi32E") and n.endswith("Lb0ELi2EEEv14UaKernelParams")
                   for n in names)
    # its fp8 sibling and the other score transforms at d = 256 still are
    assert any(n.startswith("_ZN2ua19ua_decode_sk_kernelILi256ELi32E") and "Lb1ELi2E" in n for n in names)
    assert any(n.startswith("_ZN2ua19ua_decode_sk_kernelILi256ELi32E") and "Lb0ELi1E" in n for n in names)


def test_the_scan_flags_a_dropped_copy(tmp_path):
    """A planted kernel body in the pattern found: a copy to v254 that no
    instruction reads, while the MFMA reads v2."""
    asm = tmp_path / "k.s"
    asm.write_text(
        "_ZN2ua1kEv:\n"
        "\tglobal_load_dwordx4 v[4:7], v[2:3], off\n"
        "\tv_mov_b32_e32 v253, v7\n"
        "\tv_mov_b32_e32 v254, v6\n"
        "\tscratch_store_dwordx2 off, v[4:5], off offset:96\n"
        "\tds_read_b128 v[0:3], v85\n"
        "\tv_mov_b32_e32 v3, v253\n"
        "\tscratch_load_dwordx2 v[0:1], off, off offset:96\n"
        "\tv_fmac_f32_e32 v9, v8, v8\n"
        "\tv_permlane32_swap_b32_e32 v10, v11\n"
        "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[0:3], a[0:15]\n"
        "\tglobal_store_dwordx4 v[2:3], a[0:3], off\n"
        ".Lfunc_end0:\n")
    [(fn, spills, dead)] = list(asm_check.scan(str(asm)))
    assert fn == "_ZN2ua1kEv" and spills == 1
    assert set(dead) == {("v", 254)}


# the kernels of the measured launch shapes (head dim, Q type, K/V type, score transforms)
WIDE_FP8_D256 = "_ZN2ua14ua_attn_kernelILi256ELi4ELi32EDF16_Lb1ELb0ELi1EEEv14UaKernelParams"
DECODE16_FP8_D256 = "_ZN2ua18ua_decode16_kernelILi256EDF16_Lb1ELi1ELb1EEEv14UaKernelParams"
RING_D128 = "_ZN2ua18ua_attn_lds_kernelILi128EDF16bLb0ELi0EEEv14UaKernelParams"
RING_D128_CAP = "_ZN2ua18ua_attn_lds_kernelILi128EDF16bLb0ELi3EEEv14UaKernelParams"
DECODE_SK_D128 = "_ZN2ua19ua_decode_sk_kernelILi128ELi32EDF16bLb0ELi0EEEv14UaKernelParams"


def test_class_split_kernels_fit_side_by_side(compiled):
    """In a class split (the fp8 d = 256 mix: ALiBi, sinks, window) a CU that
    holds a wide workgroup, one wave per SIMD, must still hold a 16-row
    decode wave beside it on every SIMD, or the decode launch waits for the
    wide one to drain."""
    _, meta = compiled
    assert _regs(meta, WIDE_FP8_D256) + _regs(meta, DECODE16_FP8_D256) <= 512


def test_measured_kernels_budgets(compiled):
    """Occupancy and spills of the kernels behind the measured workloads: the
    d = 128 ring keeps three waves per SIMD (168 registers) and the 32-row
    decode engine two (256), all without vector spills."""
    _, meta = compiled
    assert _regs(meta, RING_D128) <= 168 and meta[RING_D128]["vgpr_spill_count"] == 0
    assert _regs(meta, RING_D128_CAP) <= 168
    assert _regs(meta, DECODE_SK_D128) <= 256 and meta[DECODE_SK_D128]["vgpr_spill_count"] == 0
    for k in (WIDE_FP8_D256, DECODE16_FP8_D256):
        assert _regs(meta, k) <= 256 and meta[k]["vgpr_spill_count"] == 0, k
