"""The decode MFMA kernel's DMA pipeline survives compilation.

The kernel streams K/V tiles into LDS with global-to-LDS DMA written as inline
assembly, and orders each slot with explicit vmcnt waits, so that one pass is
in flight while the previous one is computed.  The compiler does not see those
DMAs.  When it believes some ordinary vector load may still be outstanding
(say, the shared-partition path's query loads, carried round the unit loop) it
adds its own `s_waitcnt vmcnt(0)` before the register is reused, and that wait
also drains every DMA in flight: the pipeline then runs one pass deep.  This
compiles the kernel's device code as the build does and checks that no score
MFMA has such a wait in front of it, and that no decode kernel uses scratch
(private) memory.
"""
import re
import subprocess

import pytest

from paged_kv_cache_179_amd import build as B

KERNEL = re.compile(r"^(_ZN2pa12_GLOBAL__N_118decode_mfma_kernel\S*):")
SCORE_MFMA = re.compile(r"\bv_mfma_f32_16x16x32_(bf16|f16)\b")
WINDOW = 25  # instructions before a score MFMA that must hold no full drain


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "decode_mfma.s"
    cmd = [hipcc, *B.HIPCC_FLAGS, *B.EXTRA_FLAGS.get("decode_mfma.hip", []), "--cuda-device-only", "-S",
           str(B.CSRC / "decode_mfma.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text().split("\n")


def drained_score_mfmas(lines):
    """Kernels with a full vmcnt wait among the WINDOW instructions before a score MFMA."""
    starts = [(i, m.group(1)) for i, l in enumerate(lines) if (m := KERNEL.match(l))]
    assert len(starts) >= 12, "decode kernels not found in the device assembly"
    bad = []
    for n, (begin, name) in enumerate(starts):
        end = starts[n + 1][0] if n + 1 < len(starts) else len(lines)
        body = [l.strip() for l in lines[begin:end]]
        insts = [l for l in body if l and not l.startswith((";", ".")) and not l.endswith(":")]
        mfmas = 0
        for j, ins in enumerate(insts):
            if not SCORE_MFMA.search(ins):
                continue
            mfmas += 1
            if any(x.startswith("s_waitcnt") and "vmcnt(0)" in x for x in insts[max(0, j - WINDOW):j]):
                bad.append(name)
        assert mfmas > 0, name
    return sorted(set(bad))


def test_no_compiler_drain_before_score_mfma(device_asm):
    bad = drained_score_mfmas(device_asm)
    assert not bad, "full vmcnt drain before a score MFMA in: " + ", ".join(bad[:6])


def test_checker_sees_a_drain():
    """The check itself: a wait placed just before a score MFMA is found."""
    asm = ["_ZN2pa12_GLOBAL__N_118decode_mfma_kernelX:"] * 1 + [
        "\ts_waitcnt vmcnt(4)", "\tds_read_b128 v[0:3], v4", "\ts_waitcnt vmcnt(0)",
        "\tv_mfma_f32_16x16x32_bf16 v[4:7], v[0:3], v[8:11], 0"]
    assert drained_score_mfmas(asm * 12) == ["_ZN2pa12_GLOBAL__N_118decode_mfma_kernelX"]
    ok = [l for l in asm if "vmcnt(0)" not in l]
    assert drained_score_mfmas(ok * 12) == []



def test_no_scratch(device_asm):
    """No decode kernel spills to scratch memory (its metadata gives a private
    segment of 0 bytes)."""
    seen = 0
    for i, line in enumerate(device_asm):
        if ".name:" in line and "decode_mfma_kernel" in line:
            for follow in device_asm[i + 1:i + 12]:
                if ".private_segment_fixed_size:" in follow:
                    seen += 1
                    assert int(follow.split(":")[1]) == 0, line.split()[-1]
                    break
    assert seen >= 12
