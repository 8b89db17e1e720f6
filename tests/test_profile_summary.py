"""profile_summary.py on synthetic rocpd-shaped databases (CPU only)."""
import hashlib
import json
import os
import sqlite3
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import profile_summary as ps  # noqa: E402

GU = "void mxmoe::(anonymous namespace)::k_gemm_stream<0, 1, true, 3, 1, 2>(mxmoe::GemmParams, int, int)"
FIN = "void mxmoe::(anonymous namespace)::k_finalize<1, false>(void const*, int, int, int, unsigned short*)"


def _trace_db(path, rows):
    os.makedirs(path)
    c = sqlite3.connect(os.path.join(path, "run_results.db"))
    c.execute("create table kernels (name text, duration int, grid_x int, grid_y int, grid_z int, "
              "workgroup_x int, workgroup_y int, workgroup_z int, lds_size int)")
    c.executemany("insert into kernels values (?,?,?,?,?,?,?,?,?)", rows)
    c.commit()


def _pmc_db(path, counter, rows):
    os.makedirs(path)
    c = sqlite3.connect(os.path.join(path, "run_results.db"))
    c.execute("create table counters_collection (id integer primary key, kernel_name text, "
              "grid_size int, counter_name text, value real)")
    c.executemany("insert into counters_collection (kernel_name, grid_size, counter_name, value) "
                  "values (?,?,?,?)", [(n, 1, counter, v) for n, v in rows])
    c.commit()


def test_trace_and_traffic(tmp_path):
    src, out = tmp_path / "src", tmp_path / "out"
    out.mkdir()
    wl = "decode_mxfp8"
    _trace_db(str(src / f"prof_trace_{wl}"), [
        (GU, 46000, 1024, 1, 1, 64, 1, 1, 0), (GU, 48000, 1024, 1, 1, 64, 1, 1, 0),
        (FIN, 4000, 256, 1, 1, 256, 1, 1, 0),
        ("void mxmoe::(anonymous namespace)::k_prepack_codes<0>(int)", 9000, 1, 1, 1, 1, 1, 1, 0),
        ("at::native::some_torch_kernel(int)", 1000, 1, 1, 1, 1, 1, 1, 0)])
    copy = "__amd_rocclr_copyBuffer"
    # 512 MiB copies: FETCH_SIZE reads half (factor 2), WRITE_SIZE all (factor 1)
    _pmc_db(str(src / f"prof_pmc_FETCH_SIZE_{wl}"), "FETCH_SIZE",
            [(copy, 262144)] * 3 + [(GU, 1000.0), (GU, 1200.0), (FIN, 10.0)])
    _pmc_db(str(src / f"prof_pmc_WRITE_SIZE_{wl}"), "WRITE_SIZE",
            [(copy, 524288)] * 3 + [(GU, 5.0), (GU, 7.0), (FIN, 2.0)])
    ps.main([str(src), "--out", str(out), "--traffic", f"{wl}=k_gemm_stream<0, 1, true, 3, 1, 2>"])
    md = (out / f"kernels_{wl}.md").read_text()
    assert "| `k_gemm_stream<0, 1, true, 3, 1, 2>` | 2 | 47.00 | 46.00 | 48.00 |" in md
    assert "k_prepack" not in md and "some_torch_kernel" not in md
    assert "51.0 us per forward call" in md   # 47 + 4
    rec = json.loads((out / "traffic.json").read_text())[wl]
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["read_bytes"] == pytest.approx(1100.0 * 2 * 1024)
    assert rec["write_bytes"] == pytest.approx(6.0 * 1024)
    # keyed by the GEMM kernels' sources, the same hash bench.py checks before it reports traffic
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_dev.h", "device.h"):
        h.update(open(os.path.join(ps.ROOT, "mx_quantized_grouped_amd", "csrc", f), "rb").read())
    assert rec["gemm_src_sha"] == h.hexdigest()[:16]
    import bench
    assert rec["gemm_src_sha"] == bench.gemm_source_hash()
