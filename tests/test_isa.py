"""Machine-code checks on the CPU: hipcc cross-compiles every fused instantiation, and
the two forward units (every output, chunk-state and preparation kernel of both dtypes),
for gfx950 to assembly, and the assembly is checked for

- register spills: a spilled value reloaded after long-latency loads waits for all of
  them (the vector-memory counter is in order), so the kernel is kept spill-free;
- 16- and 12-byte buffer stores whose data registers are rewritten by one of the next
  three instructions.  Such a store has been seen to send the rewritten values on gfx950
  when it uses an SGPR offset, and the compiler inserts no wait there; the kernel fences
  each such store itself.
"""
import os
import re
import shutil
import subprocess

import pytest

from ssd_chunked_scan_03_amd import build

INSTANCES = [(64, 64), (128, 64), (256, 64), (64, 128), (128, 128), (256, 128)]


def _hipcc():
    return build.HIPCC if (os.path.exists(build.HIPCC) or shutil.which(build.HIPCC)) else None


@pytest.fixture(scope="module")
def fused_asm(tmp_path_factory):
    if _hipcc() is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa")
    src = d / "fused_inst.hip"
    refs = "\n".join(f"    (void*)&ssd::k_fused<{q}, {n}>," for q, n in INSTANCES)
    src.write_text('#include "fused.hpp"\nvoid* fused_kernels[] = {\n' + refs + "\n};\n")
    out = d / "fused_inst.s"
    cmd = [build.HIPCC, *build.CFLAGS, "--cuda-device-only", "-S", str(src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out.read_text()


def _vregs(spec):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", spec)
    return {int(m.group(1))} if m else set()


def exposed_wide_stores(asm, window=3):
    """(store line, instruction that rewrites its data) for every 12/16-byte buffer store
    whose data VGPRs are written by one of the next `window` instructions (an s_nop or
    inline-asm block in between ends the search)."""
    ins = [l.strip() for l in asm.splitlines()]
    ins = [l for l in ins if l and not l.startswith((";", ".", "//")) and not l.endswith(":")]
    found = []
    for k, line in enumerate(ins):
        m = re.match(r"buffer_store_dwordx[34]\s+(v\[\d+:\d+\])", line)
        if not m:
            continue
        data = _vregs(m.group(1))
        for nxt in ins[k + 1:k + 1 + window]:
            if nxt.startswith(("s_nop", ";;#ASMSTART")):
                break
            op = nxt.split()
            if len(op) > 1 and op[0].startswith("v_") and _vregs(op[1].rstrip(",")) & data:
                found.append((line, nxt))
                break
    return found


def test_scanner_flags_a_rewritten_store_and_passes_a_fenced_one():
    bad = "buffer_store_dwordx4 v[70:73], v81, s[16:19], s86 offen\n v_cndmask_b32_e32 v71, v0, v76, vcc\n"
    ok = "buffer_store_dwordx4 v[70:73], v81, s[16:19], s86 offen\n s_nop 4\n v_cndmask_b32_e32 v71, v0, v76, vcc\n"
    far = ("buffer_store_dwordx4 v[70:73], v81, s[16:19], s86 offen\n v_add_u32 v1, v2, v3\n"
           " v_add_u32 v4, v2, v3\n v_add_u32 v5, v2, v3\n v_mov_b32 v72, 0\n")
    assert len(exposed_wide_stores(bad)) == 1
    assert exposed_wide_stores(ok) == [] and exposed_wide_stores(far) == []


def test_fused_kernels_do_not_spill(fused_asm):
    meta = re.findall(r"\.name:\s+(\S*k_fused\S*)\s*\n(?:.*\n)*?\s*\.vgpr_spill_count:\s+(\d+)", fused_asm)
    assert len(meta) == len(INSTANCES), meta
    assert all(int(n) == 0 for _, n in meta), meta


def test_fused_wide_stores_are_fenced(fused_asm):
    assert re.search(r"buffer_store_dwordx4", fused_asm), "the fused kernels store y with 16-byte stores"
    assert exposed_wide_stores(fused_asm) == []


@pytest.fixture(scope="module")
def forward_units_asm(tmp_path_factory):
    """The forward instantiation units compiled to gfx950 assembly, both at once."""
    if _hipcc() is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa_units")
    procs = []
    for unit in ("inst_bf16.hip", "inst_f32.hip"):
        out = d / (unit + ".s")
        cmd = [build.HIPCC, *build.CFLAGS, "--cuda-device-only", "-S", os.path.join(build.CSRC, unit), "-o", str(out)]
        procs.append((unit, out, subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True)))
    texts = {}
    for unit, out, p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err[-4000:]
        texts[unit] = out.read_text()
    return texts


def kernel_spills(asm, prefix):
    """(mangled kernel name, vgpr spill count) of every kernel whose name holds prefix."""
    out = []
    for blk in re.split(r"\n\s*- \.", asm):
        name = re.search(r"\.name:\s+(\S+)", blk)
        spill = re.search(r"\.vgpr_spill_count:\s+(\d+)", blk)
        if name and spill and prefix in name.group(1) and not name.group(1).endswith(".kd"):
            out.append((name.group(1), int(spill.group(1))))
    return out


@pytest.mark.parametrize("kernel", ["k_out", "k_state", "k_prep", "k_scan"])
def test_forward_kernels_do_not_spill(forward_units_asm, kernel):
    """Every (dtype, headdim, dstate) instantiation of the split schedule's kernels is
    spill-free (float32 output tiles at headdim 128 are the tightest)."""
    found = []
    for unit, asm in forward_units_asm.items():
        found += [(unit, n, s) for n, s in kernel_spills(asm, kernel)]
    assert len(found) >= (12 if kernel == "k_scan" else 20), found
    assert all(s == 0 for _, _, s in found), [f for f in found if f[2]]
