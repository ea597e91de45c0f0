"""Static checks on the generated gfx950 code of the decode kernels (CPU only).

The direct-to-LDS loads are issued from inline asm that sets m0 itself; that
is only sound if nothing else in the kernels keeps a value in m0.  The
kernels must also not spill (scratch traffic would add vector-memory
operations that the hand-placed wait counts do not account for).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "kv_sharded_mla_amd", "csrc", "mla_decode.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    from kv_sharded_mla_amd.build import FLAGS, HIPCC
    out = tmp_path_factory.mktemp("asm") / "mla_decode.s"
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-S", "--cuda-device-only", SRC, "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    return out.read_text()


def _kernels(asm):
    parts = re.split(r"\n(_ZN3dcp\w*mla_decode_(?:pc_)?kernel\w*):[^\n]*\n", asm)
    # a kernel's code runs to its .Lfunc_end label (early exits put s_endpgm inside)
    return {parts[i]: parts[i + 1].split(".Lfunc_end")[0] for i in range(1, len(parts) - 1, 2)}


def test_m0_only_feeds_lds_dma(asm):
    lines = [l.strip() for l in asm.splitlines()]
    code = [l for l in lines if l and not l.startswith((";", "."))]
    uses = [i for i, l in enumerate(code) if re.search(r"\bm0\b", l.split(";")[0])]
    assert uses, "expected the LDS-DMA m0 writes"
    for i in uses:
        ins = code[i].split(";")[0]
        assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", ins), ins
        assert code[i + 1].startswith("global_load_lds_dword"), code[i + 1]


def test_decode_kernels_do_not_spill(asm):
    ks = _kernels(asm)
    # 1, 2 or 4 row blocks x bf16/e4m3 x page-aligned or not x non-temporal loads or not
    assert len(ks) == 24 and all("pc_kernel" in k for k in ks)
    for name, body in ks.items():
        assert "scratch_" not in body, name


def test_workgroup_sizes(asm):
    # bf16 blocks of 64 rows (template arguments 4, false) run 16 waves with dedicated
    # loading waves; every other instantiation 8 waves
    # (the kernel metadata lists each kernel's workgroup size just before its name)
    meta = {n: s for s, n in re.findall(r"\.max_flat_workgroup_size:\s+(\d+)\s+\.name:\s+(\S+)", asm)
            if "mla_decode_pc_kernel" in n}
    assert len(meta) == 24, sorted(meta)
    for name, size in meta.items():
        want = 1024 if "kernelILi4ELb0E" in name else 512
        assert int(size) == want, (name, size)


def test_no_compiler_vmcnt_waits_inside_decode_loop(asm):
    # every vmcnt wait of the decode kernels is one of the explicit ones: 0 (page table and
    # Q before the loop) or a whole number of stages of one wave's loads, at most two
    # stages ahead.  A stage is 36 KB: 36 loads, 9 per loading wave, plus one scale load
    # per wave for e4m3 (64 rows of 576 bytes).  A wait the compiler placed for Q inside
    # the loop would show up as a count such as 17, 16, ... 1.
    # Waits before the first direct-to-LDS load (reading seq_len for the work plan, Q
    # and the page table) cannot interfere with the ring and are not checked.
    allowed = {0, 9, 18, 10}
    for name, body in _kernels(asm).items():
        first_dma = body.find("global_load_lds")
        assert first_dma > 0, name
        waits = set(int(x) for x in re.findall(r"vmcnt\((\d+)\)", body[first_dma:]))
        assert waits <= allowed, (name, sorted(waits))


def test_no_scalar_stores_or_atomics(asm):
    # memory is written only through vector stores and vector atomics
    for name, body in _kernels(asm).items():
        bad = re.findall(r"^\s*(s_store\w*|s_buffer_store\w*|s_atomic\w*|s_buffer_atomic\w*|s_dcache_wb\w*|s_scratch_store\w*)",
                         body, re.M)
        assert not bad, (name, bad[:4])


def test_non_temporal_loads_only_in_single_row_block_kernels(asm):
    # template argument 4 (NT) of mla_decode_pc_kernel: Lb1E at the end of the mangled name
    for name, body in _kernels(asm).items():
        loads = re.findall(r"global_load_lds_dword\S*[^\n]*", body)
        assert loads, name
        nt = [l for l in loads if re.search(r"\bnt\b", l)]
        if name.endswith("Lb1EEEvNS0_12DecodeParamsE"):
            assert len(nt) == len(loads), name
        else:
            assert not nt, name


def test_no_tuning_switches_in_sources():
    # the shipped kernels have one code path: no preprocessor switches select
    # between tuning variants, and the build takes no extra flags from the environment
    csrc = os.path.join(ROOT, "kv_sharded_mla_amd", "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f)).read()
        assert not re.search(r"#\s*if(n?def)?\s+DCP_", text), f
    build = open(os.path.join(ROOT, "kv_sharded_mla_amd", "build.py")).read()
    assert "os.environ.get(\"DCP_" not in build
