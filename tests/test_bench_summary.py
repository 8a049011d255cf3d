"""Host logic of bench.py's profile summary: the SQ counter section.

summarize_sq derives, per kernel, the shader clock (GRBM_GUI_ACTIVE per die
over the dispatch duration), the matrix-core FLOPs and their rate, the
matrix-core busy fraction, vector instructions per matrix instruction and
the LDS bank-conflict ratio from a rocprofv3 counter database. This test
builds such a database by hand (the columns rocprofv3 writes that the
summary reads) with values whose derived figures are known, and checks the
table row. No GPU is needed.
"""

import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, "
                "value real, duration integer, dispatch_id integer)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_summarize_sq_derives_clock_flops_busy_and_conflicts(tmp_path):
    name = "void fa::(anonymous namespace)::fwd_bf16_kernel<128, 64, true, false>(fa::Params)"
    dur_ns = 2_000_000                      # 2 ms
    clk_ghz = 1.75
    cycles = clk_ghz * dur_ns               # per die
    mfma_instr = 1_000_000                  # 32x32x16 products
    mops = mfma_instr * 32768 / 512         # SQ_INSTS_VALU_MFMA_MOPS_BF16 counts 512 FLOP
    busy = 0.5 * bench.SIMDS * cycles       # half of all SIMD cycles
    rows = []
    for did in (1, 2):                      # two identical dispatches
        rows += [
            (name, "GRBM_GUI_ACTIVE", cycles * bench.XCDS, dur_ns, did),
            (name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops, dur_ns, did),
            (name, "SQ_VALU_MFMA_BUSY_CYCLES", busy, dur_ns, did),
            (name, "SQ_INSTS_VALU", 4.0 * mfma_instr, dur_ns, did),  # 3 vector per matrix
            (name, "SQ_LDS_IDX_ACTIVE", 1000.0, dur_ns, did),
            (name, "SQ_LDS_BANK_CONFLICT", 25.0, dur_ns, did),
        ]
    db = tmp_path / "sq.db"
    _db(str(db), rows)
    lines = bench.summarize_sq(str(db))
    row = [l for l in lines if l.startswith("| `fwd_bf16_kernel")]
    assert len(row) == 1, lines
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    # kernel, dispatches, us, clock, MFMA TFLOP, TFLOP/s, peak at clock, busy, VALU/MFMA, LDS
    assert cells[1] == "2"
    assert float(cells[2]) == 2000.0
    assert abs(float(cells[3]) - clk_ghz) < 0.01
    flop = mfma_instr * 32768
    assert abs(float(cells[4]) - flop / 1e12) < 1e-3
    assert abs(float(cells[5]) - flop / dur_ns / 1e3) < 1.0
    assert abs(float(cells[6]) - bench.SIMDS * bench.MFMA_FLOP_PER_CLK * clk_ghz / 1e3) < 1.0
    assert abs(float(cells[7]) - 0.5) < 1e-3
    assert abs(float(cells[8]) - 3.0) < 1e-2
    assert abs(float(cells[9]) - 0.025) < 1e-4


def test_summarize_sq_skips_runtime_copies(tmp_path):
    rows = [("__amd_rocclr_copyBuffer", "GRBM_GUI_ACTIVE", 1e6, 1000, 1)]
    db = tmp_path / "sq.db"
    _db(str(db), rows)
    lines = bench.summarize_sq(str(db))
    assert not [l for l in lines if "copyBuffer" in l]


def test_summarize_tcc_hit_rate(tmp_path):
    name = "void fa::(anonymous namespace)::bwd_dkdv_kernel<128, 1, true, false>(fa::Params)"
    rows = []
    for did in (1, 2):
        rows += [(name, "TCC_HIT_sum", 9.0e6, 1000, did), (name, "TCC_MISS_sum", 1.0e6, 1000, did)]
    db = tmp_path / "tcc.db"
    _db(str(db), rows)
    lines = bench.summarize_tcc(str(db))
    row = [l for l in lines if l.startswith("| `bwd_dkdv_kernel")]
    assert len(row) == 1, lines
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1] == "2" and float(cells[2]) == 10.0 and float(cells[3]) == 9.0
    assert float(cells[5]) == 0.9


def test_launch_gaps_of_backward_calls(tmp_path):
    db = tmp_path / "trace.db"
    con = sqlite3.connect(str(db))
    con.execute("create table kernels (name text, start integer, end integer)")
    pre = "void fa::(anonymous namespace)::"
    rows = []
    t = 0
    for _ in range(3):   # a forward, then prep, dK/dV, dQ with 1 us and 2 us gaps
        rows.append((pre + "fwd_bf16_d64_kernel<64, 64, 2, true, false, false>(fa::Params)", t, t + 30_000))
        t += 31_000
        rows.append(("_ZN2fa12_GLOBAL__N_115bwd_prep_kernelILi64EDF16bEEvNS_6ParamsEx", t, t + 6_000))
        t += 7_000
        rows.append((pre + "bwd_dkdv_kernel<64, 2, true, false>(fa::Params)", t, t + 50_000))
        t += 52_000
        rows.append((pre + "bwd_dq_kernel<64, 64, true, false, false>(fa::Params)", t, t + 30_000))
        t += 40_000
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.commit()
    con.close()
    lines = bench.summarize_launch_gaps(str(db))
    row = [l for l in lines if l.startswith("| `bwd_dkdv")]
    assert len(row) == 1, lines
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1] == "3" and cells[2] == "3"
    assert [float(x) for x in cells[3:9]] == [6.0, 50.0, 30.0, 86.0, 89.0, 3.0]


def test_launch_gaps_of_two_kernel_backward_calls(tmp_path):
    """The bf16 backward is two launches, dQ (with the row terms) then dK/dV."""
    db = tmp_path / "trace.db"
    con = sqlite3.connect(str(db))
    con.execute("create table kernels (name text, start integer, end integer)")
    pre = "void fa::(anonymous namespace)::"
    rows = []
    t = 0
    for _ in range(2):
        rows.append((pre + "fwd_bf16_kernel<128, 64, true, false, 8>(fa::Params)", t, t + 30_000))
        t += 31_000
        rows.append((pre + "bwd_dq_kernel<128, 64, true, false, false>(fa::Params)", t, t + 40_000))
        t += 42_500
        rows.append((pre + "bwd_dkdv_kernel<128, 1, true, false>(fa::Params)", t, t + 60_000))
        t += 70_000
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.commit()
    con.close()
    lines = bench.summarize_launch_gaps(str(db))
    row = [l for l in lines if l.startswith("| `bwd_dkdv")]
    assert len(row) == 1, lines
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1] == "2" and cells[2] == "2"
    assert [float(x) for x in cells[3:9]] == [0.0, 60.0, 40.0, 100.0, 102.5, 2.5]


def test_dkdv_kernel_names_follow_the_dispatch():
    """The roofline line names the dK/dV kernel the library picks: the 64-key
    wave kernel for d = 128 from 4096 rows, the per-dimension kernels else."""
    assert bench.dkdv_kernel_name(128, 16384) == "bwd_dkdv_wide_kernel"
    assert bench.dkdv_kernel_name(128, 4096) == "bwd_dkdv_wide_kernel"
    assert bench.dkdv_kernel_name(128, 2048) == "bwd_dkdv_kernel"
    assert bench.dkdv_kernel_name(64, 1024) == "bwd_dkdv_d64_kernel"
    assert bench.dkdv_kernel_name(256, 8192) == "bwd_dkdv_d256_kernel"
    pre = "void fa::(anonymous namespace)::"
    assert bench._short(pre + "bwd_dkdv_wide_kernel<true>(fa::Params)") == \
        "bwd_dkdv_wide_kernel<true>"
    assert bench._short(pre + "bwd_dkdv_kernel<128, 1, true, false>(fa::Params)") == \
        "bwd_dkdv_kernel<128, 1, true, false>"
