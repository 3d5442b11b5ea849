"""Properties of the generated gfx950 code that the sources rely on.

The attention kernels issue their global-to-LDS tile loads as inline
assembly that sets M0 (the LDS destination) and lists it as clobbered.  M0
is a reserved register: the compiler does not save or restore it around the
asm, so the kernels are only correct while no compiler-generated
instruction reads or writes M0.  This test compiles the attention source
for gfx950 (host only, no GPU) and checks that every M0 reference is one of
the asm pairs: ``s_mov_b32 m0, sN`` followed at once by a
``buffer_load_dwordx4 ... lds``.
"""
import os
import re
import subprocess

import pytest

from spatiotemporal_attention_vx_amd import build

SRC = os.path.join(build.CSRC, "flash_attn.hip")


@pytest.fixture(scope="module")
def attention_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "flash_attn.s"
    flags = [f for f in build.FLAGS if f != "-fPIC"]
    r = subprocess.run([build.hipcc(), *flags, "--cuda-device-only", "-S", SRC, "-o", str(out)],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _instructions(text):
    for line in text.splitlines():
        code = line.split(";")[0].strip()
        if code and not code.startswith(".") and not code.endswith(":"):
            yield code


def test_m0_is_only_set_for_the_tile_dma(attention_asm):
    insts = list(_instructions(attention_asm))
    m0 = re.compile(r"\bm0\b")
    uses = [i for i, s in enumerate(insts) if m0.search(s)]
    assert uses, "the attention kernels should set M0 for their tile loads"
    for i in uses:
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", insts[i]), insts[i]
        nxt = insts[i + 1]
        assert nxt.startswith("buffer_load_dwordx4") and nxt.endswith(" lds"), nxt


def test_every_bf16_attention_kernel_is_present(attention_asm):
    for d in (64, 128):
        for pad in (0, 1):
            assert f"fa_fwd_bf16_dma_kernelILi{d}ELb{pad}E" in attention_asm
