"""Properties of the generated gfx950 code that the kernels' speed depends
on, checked on the CPU (hipcc cross-compiles; no GPU needed).

The latent decode kernel runs at the register file's limit (256 VGPRs and
256 accumulation registers per lane, one wave per SIMD). If the compiler
moves the tile loads' per-lane offsets to scratch, every refill load is
preceded by a scratch reload and a wait for all vector memory operations,
which drains the tile prefetch and doubles the call time; an innocuous
change to the code after the streaming loop did exactly that once. The test
compiles the kernel and checks the score steps of its streaming loop (the
basic blocks with four matrix products and one tile load into LDS) for
scratch reloads."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_55_amd", "csrc")


def device_asm(src, tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not available")
    out = tmp_path / "k.s"
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-S", "--offload-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", os.path.join(CSRC, src),
           "-o", str(out)]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-2000:]
    return out.read_text()


def kernel_blocks(asm, kernel_prefix):
    start = asm.index("\n" + kernel_prefix)
    end = asm.index("s_endpgm", start)
    blocks, cur = [], []
    for line in asm[start:end].splitlines():
        if re.match(r"^\.LBB\S+:", line):
            blocks.append(cur)
            cur = []
        else:
            cur.append(line.strip())
    blocks.append(cur)
    return blocks


def test_latent_streaming_loop_has_no_scratch_reloads(tmp_path):
    asm = device_asm("latent_mfma.hip", tmp_path)
    blocks = kernel_blocks(asm, "_ZN7pagedkv12_GLOBAL__N_120latent_decode_kernel")
    steps = [b for b in blocks
             if sum("v_mfma" in x for x in b) == 4
             and sum("buffer_load_dwordx4" in x and " lds" in x for x in b) == 1]
    assert len(steps) >= 10, "the score steps with a tile refill were not found"
    bad = [i for i, b in enumerate(steps) if any(x.startswith("scratch_load") for x in b)]
    assert not bad, f"{len(bad)} of {len(steps)} score steps reload from scratch"


def kernel_metadata(asm):
    """Per kernel: the scratch bytes per lane and the VGPRs spilled, from the
    code object's metadata."""
    meta = {}
    for chunk in asm.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", chunk).group(1)
        scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", chunk).group(1))
        spills = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", chunk).group(1))
        meta[name] = (scratch, spills)
    return meta


@pytest.mark.parametrize("src,prefix,count", [
    ("decode_mfma.hip", "_ZN7pagedkv12_GLOBAL__N_127decode_mfma_balanced_kernel", 6),
    ("decode_mfma.hip", "_ZN7pagedkv12_GLOBAL__N_118decode_mfma_kernel", 2),
    ("prefill_mfma.hip", "_ZN7pagedkv12_GLOBAL__N_119prefill_mfma_kernel", 2),
    ("latent_mfma.hip", "_ZN7pagedkv12_GLOBAL__N_119latent_merge_kernel", 1),
])
def test_streaming_kernels_use_no_scratch(tmp_path, src, prefix, count):
    """The paged decode and prefill kernels keep every value in registers: a
    scratch spill inside their tile loops would put a scratch round trip and
    a full memory wait between tile loads, the stall the latent test above
    guards against."""
    meta = kernel_metadata(device_asm(src, tmp_path))
    found = {n: v for n, v in meta.items() if n.startswith(prefix)}
    assert len(found) == count, sorted(meta)
    bad = {n: v for n, v in found.items() if v != (0, 0)}
    assert not bad, f"kernels with scratch bytes or VGPR spills: {bad}"


# instructions that read M0 without naming it on gfx950 (relative moves, messages, the
# global data share and ordered counts, interpolation, and every load into LDS)
M0_READERS = ("s_movrel", "v_movrel", "s_sendmsg", "ds_gws", "ds_append", "ds_consume",
              "ds_ordered_count", "v_interp", "global_load_lds", "scratch_load_lds")


def reads_m0(line):
    return line.startswith(M0_READERS) or (line.startswith("buffer_") and line.endswith(" lds"))


@pytest.mark.parametrize("src,prefixes,load", [
    ("prefill_mfma.hip", ("_ZN7pagedkv12_GLOBAL__N_119prefill_mfma_kernelILi128",
                          "_ZN7pagedkv12_GLOBAL__N_119prefill_mfma_kernelILi64"),
     "global_load_lds_dwordx4"),
    ("latent_mfma.hip", ("_ZN7pagedkv12_GLOBAL__N_120latent_decode_kernel",), "buffer_load_dwordx4"),
])
def test_m0_holds_only_the_tile_load_destination(tmp_path, src, prefixes, load):
    """The direct-to-LDS tile loads of the chunked-prefill and latent-decode
    kernels set M0 to their LDS destination and leave it there (the
    compiler keeps M0 reserved and does not honour it as an asm clobber).
    That is correct only while nothing else in these kernels reads M0:
    every M0 write is one of those loads' and is followed by its load, and
    no other instruction that reads M0 appears."""
    asm = device_asm(src, tmp_path)
    for prefix in prefixes:
        start = asm.index("\n" + prefix)
        body = [l.strip() for l in asm[start:asm.index("s_endpgm", start)].splitlines()]
        code = [l for l in body if l and not l.startswith((";", "."))]
        writes = [i for i, l in enumerate(code) if re.match(r"s_\w+ m0,", l)]
        assert writes, "no tile loads found"
        for i in writes:
            assert code[i].startswith("s_mov_b32 m0,"), code[i]
            nxt = [l for l in code[i + 1:i + 4] if not l.startswith("s_nop")]
            assert nxt and nxt[0].startswith(load) and reads_m0(nxt[0]), code[i:i + 4]
        loads = {i + 1 + k for i in writes for k in range(3)}
        readers = [l for i, l in enumerate(code) if reads_m0(l) and
                   not (i in loads and l.startswith(load))]
        assert not readers, readers[:5]
        other = [l for l in code if re.search(r"\bm0\b", l) and not re.match(r"s_mov_b32 m0,", l)]
        assert not other, other[:5]
