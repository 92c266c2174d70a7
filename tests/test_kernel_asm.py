"""Checks on the generated gfx950 assembly of the GEMM kernels (CPU; hipcc
cross-compiles).  The rings of 64-byte stages (the FP8 rowwise tiles: four
slots at 256 x 256, three at 256 x 384) issue their direct-to-LDS loads from
inline assembly and order the LDS reads with their own counted vmcnt waits,
which is only sound while:

* no other vector-memory instruction (register loads, stores, spill traffic)
  sits among the ring's loads, where it would shift the counts;
* every such load takes its global base from a scalar register pair that
  holds the address itself (a sign-extended low half once turned a valid
  base into an unmapped one);
* the compiler adds no waits of its own before the fragment reads (the
  reason for the assembly), so the only vmcnt waits in the K loop are the
  ring's."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp4_grouped_gemm_quantize_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

VMEM = re.compile(r"^\s*(global_load|global_store|global_atomic|buffer_|scratch_|flat_)")
KERNEL = re.compile(r"^(_Z\S*grouped_gemm_kernel\S*):")
TILE = re.compile(r"TileILi(\d+)ELi(\d+)ELi(\d)ELi(\d)ELi(\d)ELi(\d)ELb(\d)ELi(\d+)(?:ELb(\d))?EEELi(\d)ELb(\d)ELb(\d)")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.fail("hipcc is required to compile the GEMM kernels")
    out = str(tmp_path_factory.mktemp("asm") / "gemm.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "gemm.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    lines = open(out).read().splitlines()
    starts = [(i, m.group(1)) for i, l in enumerate(lines) if (m := KERNEL.match(l))]
    ks = {}
    for (a, name), (b, _) in zip(starts, starts[1:] + [(len(lines), None)]):
        ks[name] = lines[a:b]
    return ks


def asm_rings(kernels):
    """The kernels whose ring streams 64-byte stages (assembly loads)."""
    out = {}
    for name, body in kernels.items():
        m = TILE.search(name)
        if m and m.group(8) == "64":
            out[m.groups()] = body
    return out


def test_asm_ring_kernels_exist(kernels):
    fs = asm_rings(kernels)
    # FP8 rowwise: 256 x 256 in four slots and 256 x 384 in three, each on
    # row-major and on prepared weights
    shapes = sorted((k[0], k[1], k[4], k[8]) for k in fs)
    assert shapes == [("256", "256", "4", "0"), ("256", "256", "4", "1"), ("256", "384", "3", "0"),
                      ("256", "384", "3", "1")], shapes


def test_no_other_vector_memory_among_the_ring_loads(kernels):
    for tile, body in asm_rings(kernels).items():
        dma = [i for i, l in enumerate(body) if "global_load_lds" in l]
        assert dma, tile
        inside = [body[i].strip() for i in range(dma[0], dma[-1] + 1) if VMEM.match(body[i]) and "lds" not in body[i]]
        assert not inside, (tile, inside[:4])


def test_ring_loads_take_a_scalar_base_built_from_its_halves(kernels):
    for tile, body in asm_rings(kernels).items():
        for i, l in enumerate(body):
            if "global_load_lds" not in l:
                continue
            m = re.search(r"global_load_lds_dword(?:x4)?\s+v\d+,\s*s\[(\d+):(\d+)\]", l)
            assert m, (tile, l.strip())
            lo, hi = int(m.group(1)), int(m.group(2))
            assert hi == lo + 1
            pair = f"s[{lo}:{hi}]"
            # nothing in the lines before it widens or merges into the pair
            for j in range(max(0, i - 40), i):
                s = body[j].strip()
                if re.match(r"s_(bfe_i64|ashr_i64|or_b64|sext)", s) and s.split()[1].rstrip(",") == pair:
                    pytest.fail(f"{tile}: base {pair} of a ring load is rebuilt by '{s}'")


def test_no_compiler_waits_before_fragment_reads(kernels):
    for tile, body in asm_rings(kernels).items():
        mf = [i for i, l in enumerate(body) if "v_mfma" in l]
        lo, hi = mf[0], mf[-1]
        for i in range(lo, hi):
            if body[i].strip().startswith("ds_read"):
                prev = [body[j].strip() for j in range(max(lo, i - 3), i)]
                assert not any(p.startswith("s_waitcnt") and "vmcnt" in p and "lgkmcnt" not in p for p in prev), (
                    tile, i, prev)
