"""Host-side checks of the matrix-core kernel's LDS layouts (no GPU).

tests/layout_check.cpp compiles the kernel's layout header
(dense_fp32_matrix_amd/csrc/lds_layout.hpp) as plain C++ with g++ and
proves, for every layout the tiles use, that the direct loads fetch each
element of a K-step exactly once, put it where the fragment reads look for
it, and keep every lane's read inside the matrix at the edges (the loader
coverage and index walk-throughs of "GEMM from naive to tiled", sections
五.3-五.4).  It then prints the LDS byte offsets every lane of every wave
reads in one K-step.

The bank model below turns those offsets into LDS cycles and bank-conflict
cycles, the quantities the SQ_LDS_IDX_ACTIVE and SQ_LDS_BANK_CONFLICT
counters report (the hand bank computations of "GEMM from naive to tiled"
section 五.3 and of "SGEMM 纯 CUDA 优化总结" Q7, redone for gfx950).  It is an
empirical model of gfx950's LDS, fitted to probe measurements of 69 b128
and 11 b32 address patterns (contiguous, strided, permuted, multi-row and
the kernel's own fragment reads), every one of which it reproduces exactly:
  * ds_read_b128 runs in 4 phases of 16 lanes: lane l is in phase
    (l >> 5, parity of bits 2-4 of l); a phase reads one 256-byte row of
    64 four-byte banks, so lanes of a phase that hit one bank in different
    rows take one more cycle each (the phase costs the largest number of
    distinct rows on one bank);
  * ds_read_b32 runs in 2 phases of 32 lanes (l >> 5), each over 32 banks
    of a 128-byte row, costed the same way.
The fit also admits parity of bits 1-4 for the b128 phases; the layouts
are checked under both readings.
"""
import collections
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "layout_check.cpp")
INC = os.path.join(ROOT, "dense_fp32_matrix_amd", "csrc")


@pytest.fixture(scope="module")
def layout_output(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("layout") / "layout_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", INC, "-o", exe, SRC], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    return r.returncode, r.stdout.splitlines()


def phases(width, b128_bits=0b011100):
    """Lane -> phase key of one LDS read of `width` bytes per lane."""
    if width == 16:
        return lambda l: (l >> 5, bin(l & b128_bits).count("1") & 1)
    return lambda l: (l >> 5,)


def read_cycles(offsets, width, b128_bits=0b011100):
    """(cycles, conflict cycles) of one wave's LDS read with these per-lane byte offsets."""
    row = 256 if width == 16 else 128
    per_phase = collections.defaultdict(list)
    key = phases(width, b128_bits)
    for lane, off in enumerate(offsets):
        for w in range(width // 4):
            per_phase[key(lane)].append(off + 4 * w)
    cycles = 0
    for words in per_phase.values():
        rows_on_bank = collections.defaultdict(set)
        for a in words:
            rows_on_bank[(a % row) // 4].add(a // row)
        cycles += max(len(v) for v in rows_on_bank.values())
    return cycles, cycles - len(per_phase)


def test_layouts_cover_each_element_once(layout_output):
    rc, lines = layout_output
    fails = [ln for ln in lines if ln.startswith("FAIL")]
    oks = [ln for ln in lines if ln.startswith("ok")]
    assert rc == 0 and not fails, fails
    # KC and KM, two lane widths, five (R, BK) shapes, loader coverage and
    # edge clamps, and the tile order
    assert len(oks) == 41 and "ok tile order" in oks


def test_bank_model_reproduces_probe_patterns():
    """A few of the fitted probe points, so that a change to the model shows."""
    contiguous = [16 * l for l in range(64)]
    assert read_cycles(contiguous, 16) == (4, 0)
    assert read_cycles([32 * l for l in range(64)], 16) == (8, 4)                  # 16-byte stride 2
    assert read_cycles([256 * l for l in range(64)], 16) == (64, 60)               # one bank
    assert read_cycles([16 * (l % 8) + 1024 * (l // 8) for l in range(64)], 16) == (8, 4)
    assert read_cycles([4 * l for l in range(64)], 4) == (2, 0)
    assert read_cycles([8 * l for l in range(64)], 4) == (4, 2)                    # 32 banks for b32
    # the kernel's earlier k-contiguous swizzle ((r >> 1) ^ (r >> 3)) & 3: two-way, as measured
    old = [64 * (l % 32) + 16 * ((l // 32) ^ (((l % 32) >> 1 ^ (l % 32) >> 3) & 3)) for l in range(64)]
    assert read_cycles(old, 16) == (8, 4)


def _kstep_reads(lines):
    """{(tile, ops): [(wave, width, offsets), ...]} of the fragment reads."""
    out = collections.defaultdict(list)
    for ln in lines:
        if ln.startswith("read "):
            f = ln.split()
            out[(int(f[1]), int(f[2]))].append((int(f[3]), int(f[4]), [int(x) for x in f[5:]]))
    return out


@pytest.mark.parametrize("b128_bits", [0b011100, 0b011110], ids=["phase-bits-2-4", "phase-bits-1-4"])
def test_fragment_reads_are_conflict_free(layout_output, b128_bits):
    """Every fragment read of every wave of every tile, in all four operand
    layouts, costs the minimum LDS cycles: 4 per b128 read, 2 per b32 read."""
    _, lines = layout_output
    reads = _kstep_reads(lines)
    assert set(t for t, _ in reads) == {0, 2, 3}
    bad = []
    for (tile, ops), rs in sorted(reads.items()):
        for wave, width, offs in rs:
            cyc, conf = read_cycles(offs, width, b128_bits)
            if conf:
                bad.append((tile, ops, wave, width, cyc))
    assert not bad, f"conflicting fragment reads (tile, ops, wave, width, cycles): {bad[:8]}"


def test_kstep_lds_cycles_per_wave(layout_output):
    """LDS cycles per wave per K-step that the counters should report
    (SQ_LDS_IDX_ACTIVE / (waves x K-steps)): the 256 x 256 tile with A as
    stored and B as stored issues 4 b128 A reads and 8 b128 interleaved-column
    B reads (48 cycles); the 128 x 128 tile 4 b128 and 8 b32 reads (32)."""
    _, lines = layout_output
    reads = _kstep_reads(lines)

    def per_wave(tile, ops):
        tot = collections.Counter()
        for wave, width, offs in reads[(tile, ops)]:
            tot[wave] += read_cycles(offs, width)[0]
        assert len(set(tot.values())) == 1
        return next(iter(tot.values()))

    assert per_wave(0, 0) == 48
    assert per_wave(2, 0) == 32
