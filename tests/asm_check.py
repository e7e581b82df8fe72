"""A static check of the library's own gfx950 assembly: in every kernel, a
vector register (VGPR or AGPR) that one instruction writes on its own must be
read somewhere in the same kernel.

The compiler removes dead writes, so one that survives in a kernel means the
value it holds went nowhere: a register copy whose reader was given another
register.  The check found exactly that in a build of the 32-row stream-K
kernel at d = 256 with 16-bit K/V and the QQ bias (one word of a spilled Q
fragment was copied to a register that no instruction read, and the MFMA read
a stale register in its place), so such a write is treated as a miscompile.

    python tests/asm_check.py        compile the kernel sources to assembly and
                                     print each kernel's spill stores and any
                                     dead writes
"""
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")
# the destination is also read (accumulate, lane write, preserved lanes)
_DST_READ = re.compile(r"fmac|_mac_|writelane|_dpp|_sdwa|d16|mfma|smfmac|dot\dc")


def _regs(text):
    out = []
    for m in _REG.finditer(text):
        if m.group(1):
            out.append((m.group(1), int(m.group(2))))
        else:
            out.extend((m.group(3), i) for i in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def _writes_first_operand(mn: str) -> bool:
    """Whether the instruction's first operand is a vector destination."""
    if "store" in mn or mn.startswith(("ds_write", "s_", "exp")):
        return False
    if "_lds" in mn:  # global/buffer loads straight into LDS: the operand is an address
        return False
    if "atomic" in mn:  # only the returning forms write their first operand
        return False
    if mn.startswith("v_cmp"):
        return False
    return True


def _functions(asm_path):
    fn, body = None, []
    with open(asm_path) as f:
        for line in f:
            m = re.match(r"^(_Z\w+):", line)
            if m:
                fn, body = m.group(1), []
                continue
            if fn and line.startswith(".Lfunc_end"):
                yield fn, body
                fn = None
                continue
            if fn:
                body.append(line)


def scan(asm_path):
    """Yield (kernel, spill stores, {register: first dead write}) per kernel."""
    for fn, body in _functions(asm_path):
        defs, uses, spills = {}, set(), 0
        for line in body:
            t = line.split(";")[0].strip()
            if not t or t.startswith(".") or t.endswith(":"):
                continue
            parts = t.split(None, 1)
            mn, ops = parts[0], parts[1] if len(parts) > 1 else ""
            if mn.startswith("scratch_store"):
                spills += 1
            opl = [o.strip() for o in re.split(r",(?![^\[]*\])", ops)] if ops else []
            if "swap" in mn:  # v_swap, v_permlane*_swap: both operands read and written
                for o in opl:
                    uses.update(_regs(o))
                continue
            if not opl or not _writes_first_operand(mn) or "glc" in ops and "atomic" in mn:
                for o in opl:
                    uses.update(_regs(o))
                continue
            dst = _regs(opl[0])
            for o in opl[1:]:
                uses.update(_regs(o))
            if _DST_READ.search(mn) or "dst_unused" in ops:
                uses.update(dst)
            if len(dst) == 1:
                defs.setdefault(dst[0], t)
        dead = {r: d for r, d in defs.items() if r not in uses}
        yield fn, spills, dead


def compile_asm(out_dir):
    """Device-only gfx950 assembly of every kernel source, as the library builds them."""
    from varlen_attention_serving_amd import build as bld
    srcs = [s for s in bld.SOURCES if s.endswith(".hip")]

    def one(src):
        out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
        cmd = [bld.HIPCC, *bld.COMMON, "--offload-device-only", "-S", "-x", "hip",
               os.path.join(bld.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"assembly of {src} failed:\n{r.stderr[-3000:]}")
        return out

    with ThreadPoolExecutor(len(srcs)) as ex:
        return list(ex.map(one, srcs))


_ENTRY = re.compile(r"^  - \.(\w+):\s*(\S*)")
_FIELD = re.compile(r"^    \.(\w+):\s*(\S*)")


def metadata(asm_path):
    """{kernel: {vgpr_count, agpr_count, vgpr_spill_count, ...}} from the code
    object metadata at the end of an assembly file (one list entry per
    kernel; its argument descriptions are nested deeper and skipped)."""
    out, entry, inside = {}, None, False

    def close():
        if entry and "name" in entry:
            out[entry.pop("name")] = entry

    with open(asm_path) as f:
        for line in f:
            if line.startswith("amdhsa.kernels:"):
                inside = True
                continue
            if not inside:
                continue
            m = _ENTRY.match(line) or _FIELD.match(line)
            if not m:
                if line and not line.startswith(" "):
                    break  # the end of the kernels list
                continue
            if line.startswith("  - "):
                close()
                entry = {}
            key, val = m.group(1), m.group(2)
            entry[key] = val if key == "name" else (int(val) if val.isdigit() else val)
    close()
    return out


def check_with_metadata(out_dir=None):
    """check()'s rows and every kernel's metadata, from one compile."""
    rows, meta = [], {}
    with tempfile.TemporaryDirectory() as tmp:
        for path in compile_asm(out_dir or tmp):
            for fn, spills, dead in scan(path):
                rows.append((os.path.basename(path), fn, spills, dead))
            meta.update(metadata(path))
    return rows, meta


def check(out_dir=None):
    """[(source, kernel, spill stores, dead writes)] over the library's kernels."""
    return check_with_metadata(out_dir)[0]


def main():
    rows = check()
    bad = 0
    for src, fn, spills, dead in rows:
        if spills or dead:
            print(f"{src} {fn} spill_stores={spills} dead_writes={len(dead)}")
        for r, d in sorted(dead.items()):
            bad += 1
            print(f"    {r[0]}{r[1]}: {d}")
    print(f"{len(rows)} kernels, {bad} dead writes")
    sys.exit(1 if bad else 0)


if __name__ == "__main__":
    main()
