"""Assembly lint of the direct-to-LDS loads (no GPU).

The ping-pong kernels write m0 (the LDS address of a direct-to-LDS load) one
MFMA ahead of the load that uses it, in two separate inline-assembly
statements: the compiler does not know that the load reads m0.  That is
correct only while, in the compiled code,

* every `buffer_load_dword* ... lds` follows an m0 write with at least one
  instruction between them (the wait state an m0 write needs before an LDS
  DMA reads it), and
* no m0 write in those kernels comes from outside inline assembly (a write
  of the compiler's own between a split pair would redirect the load).

tests/asm/dma_kernels.hip instantiates the kernels that use the split form;
this test compiles it to gfx950 assembly with the library's flags and checks
both rules per kernel.  The checker itself is tested on small listings.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
SRC = os.path.join(ROOT, "tests", "asm", "dma_kernels.hip")


def kernels(text):
    """Yields (kernel symbol, [lines]) of every kernel body in a listing."""
    name, cur = None, None
    for line in text.splitlines():
        m = re.match(r"^(_Z\S*):", line)
        if m:
            name, cur = m.group(1), []
            continue
        if cur is not None:
            cur.append(line)
            if "s_endpgm" in line:
                yield name, cur
                cur = None


def lint(lines):
    """Problems of one kernel body: a list of (instruction, reason)."""
    bad, in_asm, wrote, since, n = [], False, False, 0, 0
    for raw in lines:
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        t = t.split(";")[0].strip()
        if not t or t.endswith(":") or t.startswith("."):
            continue
        if re.match(r"^\S+\s+m0,", t):
            if not in_asm:
                bad.append((t, "m0 written outside inline assembly"))
            wrote, since = True, 0
            continue
        if t.split()[0].startswith("buffer_load_dword") and t.endswith(" lds"):
            n += 1
            if not wrote:
                bad.append((t, "LDS-DMA load with no m0 write before it"))
            elif since < 1:
                bad.append((t, "LDS-DMA load right after its m0 write"))
        since += 1
    return bad, n


def test_lint_flags_the_two_mistakes():
    good = [";;#ASMSTART", "s_add_u32 m0, s4, 0x1000", ";;#ASMEND",
            "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
            ";;#ASMSTART", "buffer_load_dwordx4 v1, s[8:11], s2 offen lds", ";;#ASMEND"]
    assert lint(good) == ([], 1)
    adjacent = [";;#ASMSTART", "s_add_u32 m0, s4, 0x1000",
                "buffer_load_dwordx4 v1, s[8:11], s2 offen lds", ";;#ASMEND"]
    assert [r for _, r in lint(adjacent)[0]] == ["LDS-DMA load right after its m0 write"]
    compiler = [";;#ASMSTART", "s_add_u32 m0, s4, 0", ";;#ASMEND", "s_mov_b32 m0, s7",
                "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
                ";;#ASMSTART", "buffer_load_dwordx4 v1, s[8:11], s2 offen lds", ";;#ASMEND"]
    assert [r for _, r in lint(compiler)[0]] == ["m0 written outside inline assembly"]
    assert [r for _, r in lint(["buffer_load_dword v1, s[8:11], 0 offen lds"])[0]] == \
        ["LDS-DMA load with no m0 write before it"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_split_m0_kernels_keep_their_m0(tmp_path):
    out = str(tmp_path / "dma_kernels.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    with open(out) as f:
        found = dict(kernels(f.read()))
    assert len(found) == 9, sorted(found)
    for name, body in found.items():
        bad, n = lint(body)
        assert n > 0, f"{name}: no direct-to-LDS loads found"
        assert not bad, f"{name}: {bad[:5]}"
