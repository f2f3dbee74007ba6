"""The build's check for MFMA accumulator chains that switch MFMA shape.

gfx950 does not order an MFMA's accumulator (srcC) read after a just-issued
MFMA of another shape that writes it, and the compiler adds no wait states for
that case; the build scans the emitted assembly and fails on it.
"""
import glob
import os

from gated_delta_rule_46_amd.isa_check import mixed_mfma_chains

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

BAD = """
_Zkernel:
	v_mfma_f32_16x16x32_bf16 v[98:101], v[182:185], v[66:69], v[106:109]
	v_mfma_f32_16x16x16_bf16 v[98:101], v[156:157], v[128:129], v[98:101]
	s_endpgm
"""

SAME_SHAPE = """
_Zkernel:
	v_mfma_f32_16x16x32_bf16 v[98:101], v[182:185], v[66:69], v[106:109]
	v_mfma_f32_16x16x32_bf16 v[98:101], v[156:159], v[128:131], v[98:101]
	s_endpgm
"""

REWRITTEN = """
_Zkernel:
	v_mfma_f32_16x16x16_bf16 v[34:37], v[42:43], v[22:23], 0
	v_cvt_pk_bf16_f32 v33, v36, v37
	v_mfma_f32_16x16x32_bf16 v[34:37], v[26:29], v[38:41], v[66:69]
	v_mfma_f32_16x16x32_bf16 v[38:41], v[30:33], v[38:41], v[34:37]
	s_endpgm
"""

FAR = "\n_Zkernel:\n\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0\n" + \
      "\ts_nop 7\n" * 5 + "\tv_mfma_f32_16x16x16_bf16 v[12:15], v[16:17], v[18:19], v[0:3]\n"


def test_flags_shape_switch():
    hits = mixed_mfma_chains(BAD)
    assert len(hits) == 1 and hits[0][4] == 1


def test_same_shape_chain_and_overwrites_pass():
    assert mixed_mfma_chains(SAME_SHAPE) == []
    assert mixed_mfma_chains(REWRITTEN) == []
    assert mixed_mfma_chains(FAR) == []          # 40 wait states apart
    assert len(mixed_mfma_chains(FAR, window=64)) == 1


def test_built_listings_are_clean():
    """Every HIP source of the built library has its listing, the engine's
    listings hold MFMAs, and none chains accumulators across shapes."""
    import pytest
    pkg = os.path.join(ROOT, "gated_delta_rule_46_amd")
    if not os.path.exists(os.path.join(pkg, "libkda.so")):
        pytest.skip("library not built (gated_delta_rule_46_amd/build.py emits the listings)")
    sources = sorted(glob.glob(os.path.join(pkg, "csrc", "*.hip")))
    assert sources
    for src in sources:
        p = os.path.join(pkg, "_build", os.path.basename(src) + ".s")
        assert os.path.exists(p), f"no listing for {src}"
        with open(p) as f:
            text = f.read()
        if os.path.basename(src).startswith("kda_chunk_"):
            assert "v_mfma_f32_16x16x" in text, p
        assert mixed_mfma_chains(text) == [], p
