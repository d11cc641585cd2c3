"""Regression test (CPU only): inline asm that writes SCC must declare it.

The prefill body sets m0 for its direct-to-LDS tile loads with s_add_u32
inside an asm block; s_add_u32 writes SCC.  Without an "scc" clobber the
compiler once split a 64-bit address add around such a block, so the high
half lost its carry and a load faulted on the GPU.  This test compiles the
attention source for gfx950 to assembly and checks that after every such
block the first instruction touching SCC writes it (a comparison, an ALU op)
rather than reading it (add-with-carry, conditional branch or select)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_varlen_flashattention_amd", "csrc")

READERS = ("s_addc_u32", "s_subb_u32", "s_cbranch_scc0", "s_cbranch_scc1", "s_cselect_b32",
           "s_cselect_b64", "s_cmov_b32", "s_cmov_b64", "s_cmovk_i32")
WRITERS = ("s_add_", "s_sub_", "s_cmp", "s_and_", "s_or_", "s_xor_", "s_andn2", "s_orn2", "s_nand",
           "s_nor", "s_xnor", "s_lshl", "s_lshr", "s_ashr", "s_bfe", "s_min", "s_max", "s_abs", "s_not",
           "s_mul_hi", "s_bitcmp", "s_addk", "s_bcnt", "s_quadmask", "s_wqm")


def scc_violations(asm_text: str):
    bad, blocks = [], 0
    lines = [l.strip() for l in asm_text.split("\n")]
    for k, line in enumerate(lines):
        if not line.startswith("s_add_u32 m0"):
            continue
        blocks += 1
        for nxt in lines[k + 1:k + 400]:
            if not nxt or nxt.startswith((";", ".")) or nxt.endswith(":"):
                continue
            op = nxt.split()[0]
            if op in READERS:
                bad.append((line, nxt))
                break
            if op.startswith(WRITERS):
                break
    return blocks, bad


def test_scc_checker_finds_a_planted_reader():
    planted = "s_add_u32 s6, s14, s6\ns_add_u32 m0, s99, 0\nglobal_load_lds_dwordx4 v1, s[8:9]\ns_addc_u32 s7, s90, s7\n"
    assert scc_violations(planted) == (1, [("s_add_u32 m0, s99, 0", "s_addc_u32 s7, s90, s7")])
    clean = "s_add_u32 m0, s99, 0\nglobal_load_lds_dwordx4 v1, s[8:9]\ns_cmp_eq_u32 s1, 0\ns_cbranch_scc1 .L1\n"
    assert scc_violations(clean) == (1, [])


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_scc_reader_after_m0_asm(tmp_path):
    from paged_varlen_flashattention_amd import build as b
    out = tmp_path / "attn.s"
    subprocess.check_call([b.hipcc(), *b.HIPCC_FLAGS, "-Wno-inline-asm", "-I", b.INCLUDE, "-I", CSRC, "-x", "hip",
                           "--offload-device-only", "-S", os.path.join(CSRC, "ua_attention.hip"), "-o", str(out)],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    blocks, bad = scc_violations(out.read_text())
    assert blocks > 0, "no s_add_u32 m0 blocks found: the check no longer covers the tile loads"
    assert not bad, f"{len(bad)} SCC readers follow an m0 asm block, first: {bad[0]}"
