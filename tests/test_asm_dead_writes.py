"""No kernel of the library writes a vector register that it never reads (see
tests/asm_check.py): the pattern of a miscompile found in one instantiation,
which the library no longer builds.  Compiles the kernel sources to gfx950
assembly on the CPU (about 45 s)."""
import os

import pytest

import asm_check


@pytest.fixture(scope="module")
def kernels():
    return asm_check.check()


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
