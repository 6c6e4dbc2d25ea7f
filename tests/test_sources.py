"""Source checks of the decode kernels (CPU only).

Inline asm that writes a VGPR is invisible to the compiler's hazard checks:
a code operand rebuilt by such an instruction right after the matrix op that
reads it changed under that op (wrong sums at head_dim 96, and NaN outputs
under another instruction schedule).  The kernels therefore write VGPRs from
asm only where no matrix op can be in flight: the one-time materialisation of
the magic constant at kernel entry.  DMA and wait asm write no VGPR.
"""
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "decode_attention_int4_amd", "csrc")
KERNEL_SOURCES = ["rq_decode.hip", "rq_gqa.hip", "rq_stage.h"]


def _asm_statements(text):
    # asm(...) / asm volatile(...) statements, up to their closing ");"
    return re.findall(r"\basm\s*(?:volatile\s*)?\((.*?)\);", text, re.S)


def test_no_vgpr_writing_asm_besides_the_magic_constant():
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name)) as f:
            text = f.read()
        for body in _asm_statements(text):
            if '"=v"' not in body and '"+v"' not in body:
                continue
            assert re.match(r'\s*"v_mov_b32 %0, %1"\s*:\s*"=v"\(magic\)\s*:\s*"i"\(kMagic\)', body), \
                f"{name}: inline asm writes a VGPR: {body.strip()[:80]}"


def test_decode_sources_use_the_iterative_ilp_schedule():
    from decode_attention_int4_amd import build
    for src in ("rq_decode.hip", "rq_gqa.hip"):
        assert "-amdgpu-sched-strategy=iterative-ilp" in build.SOURCE_FLAGS[src]
    assert "-amdgpu-atomic-optimizer-strategy=None" in build.FLAGS
