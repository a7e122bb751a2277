"""Code-generation checks (no GPU): the kernels are compiled to gfx950 assembly
with the package's own flags, and the loops whose throughput rests on how the
compiler scheduled them are read back.

- Prefill GEMM main loops (the four loops with MFMAs: FP8 and precise heads,
  one- and two-tile CTAs). Each stage waits once for its own loads, at a
  vector-memory count that leaves the later stages' loads in flight:
  (kPrefetch - 1) x the loads a stage issues. A lower wait inside the loop
  drains every load issued ahead; the compiler once put one there to widen a
  loaded byte at its load.
- Precise heads' steps: their 16 weight-operand LDS reads run ahead of the
  MFMAs, so only a stage's last MFMA waits for every LDS read.
- Decode GEMV without a publisher: the whole weight stream (four 16-byte loads
  per 128-wide k chunk) is issued before the first MFMA, not sunk next to the
  MFMAs that take it.
"""

import os
import re
import subprocess
import tempfile

import pytest

from kv_residual_add_amd import build as pa_build

CSRC = pa_build.CSRC


def _assembly(source: str) -> str:
    try:
        hipcc = pa_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not available")
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", pa_build.INCLUDE, "-I", CSRC, os.path.join(CSRC, source), "-o", out]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        assert proc.returncode == 0, proc.stderr[-2000:]
        with open(out) as f:
            return f.read()


def _functions(text: str) -> dict:
    return {m.group(1): m.group(2).split("\n")
            for m in re.finditer(r"^(_Z\S+):[^\n]*\n(.*?)^\.Lfunc_end", text, re.S | re.M)}


def _instructions(lines):
    return [x.split(";")[0].strip() for x in lines if x.strip() and not x.strip().startswith((".", ";"))]


def _loops(lines):
    """Bodies of the loops the compiler marks with a header comment."""
    out = []
    for i, line in enumerate(lines):
        if "Loop Header" not in line:
            continue
        label = line.split(":")[0]
        for j in range(i + 1, len(lines)):
            t = lines[j].strip()
            if t.startswith("s_cbranch") and t.endswith(label):
                out.append(_instructions(lines[i:j + 1]))
                break
    return out


@pytest.fixture(scope="module")
def prefill_asm():
    return _functions(_assembly("pa_prefill.hip"))


@pytest.fixture(scope="module")
def decode_asm():
    return _functions(_assembly("pa_decode.hip"))


def _gemm_loops(funcs):
    loops = {}
    for name, body in funcs.items():
        m = re.search(r"prefill_gemmILi(\d)E", name)
        if not m:
            continue
        for loop in _loops(body):
            n_fp8 = sum(x.startswith("v_mfma_scale_f32_32x32x64_f8f6f4") for x in loop)
            n_bf16 = sum(x.startswith("v_mfma_f32_32x32x16_bf16") for x in loop)
            if n_fp8 or n_bf16:
                loops[(int(m.group(1)), "precise" if n_bf16 else "fp8")] = loop
    return loops


# loads a stage issues per wave: one k step (two in one-tile FP8 CTAs) of the
# weight tile's LDS copies (FP8 2, bf16 4), the FP8 weight-scale dword, and per
# 32-token tile two activation loads and a scale byte; kPrefetch = 3 stages
STAGE_LOADS = {(1, "fp8"): 2 * (2 + 1 + 3), (2, "fp8"): 2 + 1 + 6, (1, "precise"): 4 + 3, (2, "precise"): 4 + 6}


def test_prefill_main_loops_wait_only_at_stage_barriers(prefill_asm):
    loops = _gemm_loops(prefill_asm)
    assert set(loops) == set(STAGE_LOADS), sorted(loops)
    for key, loop in loops.items():
        waits = [int(re.search(r"vmcnt\((\d+)\)", x).group(1)) for x in loop
                 if x.startswith("s_waitcnt") and "vmcnt" in x]
        assert waits == [2 * STAGE_LOADS[key]] * 4, (key, waits)  # four stages per loop iteration
        assert sum(x == "s_barrier" for x in loop) == 4, key


def test_precise_steps_read_the_weight_operand_ahead(prefill_asm):
    loops = _gemm_loops(prefill_asm)
    for ntw in (1, 2):
        loop = loops[(ntw, "precise")]
        mfmas = sum(x.startswith("v_mfma") for x in loop)
        assert mfmas == 4 * 16 * ntw
        # MFMAs issued right after a wait for every LDS read: one a stage (the last)
        drained = sum(1 for a, b in zip(loop, loop[1:])
                      if b.startswith("v_mfma") and a.startswith("s_waitcnt") and "lgkmcnt(0)" in a)
        assert drained <= 4, (ntw, drained)


def test_decode_gemv_issues_the_weight_stream_first(decode_asm):
    seen = 0
    for name, body in decode_asm.items():
        m = re.search(r"(decode_gemv_epiILi(\d)ELi\dELb0E|decode_gemvILi(\d)ELi\dE)", name)
        if not m:
            continue
        cpc = int(m.group(2) or m.group(3))
        ins = _instructions(body)
        first = next(i for i, x in enumerate(ins) if x.startswith("v_mfma"))
        weights = sum(1 for x in ins[:first] if x.startswith("global_load_dwordx4") and x.endswith(" nt"))
        assert weights == 4 * cpc, (name, weights)
        seen += 1
    assert seen == 16  # CPC 1..4 x two token-tile counts, with and without the fused epilogue
