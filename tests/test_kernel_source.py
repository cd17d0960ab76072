"""Static checks of the HIP sources (no GPU, no compiler run).

Vector-memory instructions written as inline assembly are invisible to the compiler's
hazard checks.  Their SGPR operands (buffer offset, resource) are usually produced by
v_readfirstlane right before them, and a vector-memory read of an SGPR that a VALU
instruction wrote needs five wait states on this architecture; with fewer, a load read a
stale offset and returned zeros.  Every such asm statement must therefore begin with the
BAM_VMEM_SGPR_NOPS prefix (s_nop 4)."""
import os
import re

CSRC = os.path.join(os.path.dirname(__file__), "..", "positional_prior_bias_amd", "csrc")


def _sources():
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name)) as f:
                yield name, f.read()


def test_nop_prefix_is_five_wait_states():
    hdr = open(os.path.join(CSRC, "bam_device.h")).read()
    m = re.search(r'#define BAM_VMEM_SGPR_NOPS "s_nop (\d+)\\n\\t"', hdr)
    assert m, "BAM_VMEM_SGPR_NOPS must be an s_nop prefix"
    assert int(m.group(1)) + 1 >= 5       # s_nop N inserts N + 1 wait states


def test_every_asm_vector_memory_instruction_has_the_prefix():
    found = 0
    for name, src in _sources():
        # each asm statement: from 'asm volatile(' to the first string's end
        for m in re.finditer(r'asm\s+volatile\s*\(\s*((?:BAM_VMEM_SGPR_NOPS\s*)?)"([^"]*)"', src):
            text = m.group(2)
            if re.search(r"\b(buffer|global|flat|scratch)_(load|store|atomic)", text):
                found += 1
                line = src[:m.start()].count("\n") + 1
                assert m.group(1).strip() == "BAM_VMEM_SGPR_NOPS", f"{name}:{line} lacks the wait-state prefix"
    assert found >= 3    # the two direct-to-LDS helpers and the Q loads of the forward
