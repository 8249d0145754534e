"""bench.py's reading of rocprofv3 counter rows (CPU): the flash kernel's
HBM bytes scaled by the copy calibration of the same run, the counted bytes
of the HBM-bound stage kernels, and the MFMA busy fraction with the shader
clock. Synthetic rows with known answers."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

FLASH = "void slr::k_flash_tiled<32, 1, false, false>(slr::FlashArgs, int const*, unsigned short const*)"
DENSE = "void slr::k_flash_tiled<32, 0, true, false>(slr::FlashArgs, int const*, unsigned short const*)"
COPY = "__amd_rocclr_copyBuffer"
ROPE = "void slr::k_rope_pool<unsigned short, 128, 64, true, true>(...)"
SUMM = "slr::k_lr_summary_bf16_pf(unsigned short const*, ...)"   # plain kernels carry no "void "


def _row(name, value, did=0, counter="X", t0=0, t1=1):
    return {"Kernel_Name": name, "Counter_Value": str(value), "Dispatch_Id": str(did), "Counter_Name": counter,
            "Start_Timestamp": str(t0), "End_Timestamp": str(t1)}


def test_traffic_scales_by_the_copies_of_the_same_run():
    gib_kib = 2 ** 30 / 1024
    # the copy reads half its bytes in FETCH_SIZE KiB (factor 2), all of them in WRITE_SIZE (factor 1)
    fetch = [_row(COPY, gib_kib / 2)] * 3 + [_row(COPY, 10.0)] + [_row(FLASH, 1000.0), _row(FLASH, 3000.0),
                                                                 _row(DENSE, 9e9), _row(ROPE, 50.0), _row(SUMM, 7.0)]
    write = [_row(COPY, gib_kib)] * 3 + [_row(FLASH, 100.0), _row(ROPE, 20.0), _row(SUMM, 1.0)]
    tb, detail, mfma, stages = bench.counters_from_rows(fetch, write, "no sq run")
    assert tb == (2000.0 * 2 + 100.0) * 1024          # mean over the sparse launches only
    assert detail["fetch_bytes"] == 2000 * 2 * 1024 and detail["write_bytes"] == 100 * 1024
    assert detail["counters"]["FETCH_SIZE"]["scale"] == 2.0 and detail["counters"]["WRITE_SIZE"]["scale"] == 1.0
    assert stages == {"rope_pool": (50.0 * 2 + 20.0) * 1024, "lowrank_summary": (7.0 * 2 + 1.0) * 1024}
    assert mfma is None


def test_missing_runs_fall_back_without_numbers():
    tb, detail, mfma, stages = bench.counters_from_rows("FETCH_SIZE run failed", "FETCH_SIZE run failed", "x")
    assert tb is None and stages is None and mfma is None and "failed" in detail
    # copies missing: no scale, so no traffic
    tb, detail, _, _ = bench.counters_from_rows([_row(FLASH, 1.0)], [_row(FLASH, 1.0)], "x")
    assert tb is None and "missing" in detail


def test_mfma_busy_fraction_and_clock():
    # 1024 SIMDs busy half of 2e6 shader cycles per XCD (GRBM_COUNT sums 8 XCDs), over 1 ms
    sq = [_row(FLASH, 0.5 * 1024 * 2e6, did=7, counter="SQ_VALU_MFMA_BUSY_CYCLES", t0=0, t1=1_000_000),
          _row(FLASH, 8 * 2e6, did=7, counter="GRBM_COUNT", t0=0, t1=1_000_000),
          _row(DENSE, 1e12, did=8, counter="SQ_VALU_MFMA_BUSY_CYCLES"), _row(DENSE, 1.0, did=8, counter="GRBM_COUNT")]
    _, _, mfma, _ = bench.counters_from_rows("x", "x", sq)
    assert mfma["busy_frac"] == 0.5
    assert mfma["clock_MHz"] == 2000
