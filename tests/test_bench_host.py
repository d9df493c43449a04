"""bench.py's host logic without a GPU: the parity comparison of the suite lines, and the
attribution of rocprofv3 dispatches to workloads in --summarize-configs (on synthetic rocpd
databases with the kernel-trace and counter views it reads)."""

import json
import os
import sqlite3

import numpy as np
import pytest

import bench


def test_compare_bf16_and_f32():
    want = np.array([1.0, -2.5, 0.0, 3.0e-3, np.nan])
    bits = (want.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert bench._compare(bits, want) == (0, 0)
    one = bits.copy()
    one[1] += 1  # one ulp
    assert bench._compare(one, want) == (1, 0)
    two = bits.copy()
    two[0] += 2
    assert bench._compare(two, want) == (2, 1)
    nan_for_num = bits.copy()
    nan_for_num[2] = 0x7FC0
    assert bench._compare(nan_for_num, want)[1] == 1
    w32 = np.array([1.0, 1e-7, -4.0])
    g32 = w32.astype(np.float32)
    assert bench._compare(g32, w32) == (0, 0)
    g32b = g32.copy()
    g32b[0] *= 1.0 + 2e-5  # past 1e-5 relative
    mu, over = bench._compare(g32b, w32)
    assert over == 1 and mu > 100


def _fake_db(path, rows, counter=None):
    con = sqlite3.connect(path)
    if counter is None:
        con.execute("create table kernels (name, duration, vgpr_count, accum_vgpr_count, lds_size, "
                    "scratch_size, workgroup_x, workgroup_y, workgroup_z, dispatch_id)")
        for i, (name, dur) in enumerate(rows):
            con.execute("insert into kernels values (?,?,?,?,?,?,?,?,?,?)",
                        (name, dur * 1000.0, 24, 0, 64, 0, 512, 1, 1, i))
    else:
        con.execute("create table counters_collection (kernel_name, counter_name, value, dispatch_id)")
        for i, (name, val) in enumerate(rows):
            # two partial records per dispatch (the view's rows are summed per dispatch)
            con.execute("insert into counters_collection values (?,?,?,?)", (name, counter, val / 2, i))
            con.execute("insert into counters_collection values (?,?,?,?)", (name, counter, val / 2, i))
        con.execute("insert into counters_collection values (?,?,?,?)", ("torch_kernel", counter, 5.0, 999))
    con.commit()
    con.close()


def test_summarize_configs_attributes_dispatches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "SUITE_TRAFFIC_FILE", str(tmp_path / "t.json"))
    monkeypatch.setattr(bench, "SUITE_MD", str(tmp_path / "t.md"))
    meta = bench._case_meta()
    ids = bench.CONFIG_IDS + bench.NEXT_IDS

    def seq(calls, value):
        out = [("void nrm::copy16_kernel(...)", value("cal"))] * calls
        for cid in ids:
            nd = bench.dispatches_per_call(cid)
            for _ in range(calls):
                if cid in bench.DISPATCHES_PER_CALL:  # the backward: its kernel, then column sums
                    out.append((f"void nrm::kernel_{cid}(nrm::Args)", value(cid)))
                    out.append(("void nrm::vjp_colsum<true>(double const*)", 1.0))
                else:  # a row call split into nd launches, each a share of the call's bytes
                    out += [(f"void nrm::kernel_{cid}(nrm::Args)", value(cid) / nd)] * nd
        return out

    # the calibration copy reads half its bytes on FETCH_SIZE (scale 2) and all on WRITE_SIZE
    cal_kib = bench.CAL_BYTES / 1024
    fetch = lambda cid: cal_kib / 2 if cid == "cal" else meta[cid]["bytes"] / 2 / 1024 / 2
    write = lambda cid: cal_kib if cid == "cal" else meta[cid]["bytes"] / 2 / 1024
    _fake_db(tmp_path / "tr.db", seq(20, lambda cid: 100.0))
    _fake_db(tmp_path / "f.db", seq(3, fetch), "FETCH_SIZE")
    _fake_db(tmp_path / "w.db", seq(3, write), "WRITE_SIZE")
    bench.summarize_configs(str(tmp_path / "tr.db"), str(tmp_path / "f.db"), str(tmp_path / "w.db"))
    t = json.load(open(tmp_path / "t.json"))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    for cid in ids:
        c = t["cases"][cid]
        assert c["kernel"].startswith(f"kernel_{cid}")
        assert c["dispatches_per_call"] == bench.dispatches_per_call(cid)
        colsum = 2 * 1.0 * 1024 / 1e6 if cid in bench.DISPATCHES_PER_CALL else 0.0
        assert c["fetch_MB"] == pytest.approx(meta[cid]["bytes"] / 2 / 1e6 + colsum, abs=0.011)
        assert c["write_MB"] == pytest.approx(meta[cid]["bytes"] / 2 / 1e6 + colsum / 2, abs=0.011)
    # a run that does not match the case list is refused
    _fake_db(tmp_path / "bad.db", seq(3, fetch)[:-1], "FETCH_SIZE")
    with pytest.raises(SystemExit, match="not a multiple"):
        bench.summarize_configs(str(tmp_path / "tr.db"), str(tmp_path / "bad.db"), str(tmp_path / "w.db"))


def test_row_call_launches():
    """The library's split of row calls over 1 GiB, as the counter attribution counts it: the
    1 GiB headline call is one launch; the larger at-scale calls are several."""
    assert bench.row_call_launches(16384, 8192, 2, 4) == 1         # exactly 1 GiB
    assert bench.row_call_launches(16385, 8192, 2, 4) == 2         # one row more
    assert bench.row_call_launches(16384, 8192, 4, 4) == 2         # 8192 rows a piece
    assert bench.row_call_launches(65536, 5120, 2, 4) == 3         # 26214 rows a piece
    assert bench.row_call_launches(65536, 5120, 4, 4) == 6         # 13106 rows a piece
    assert bench.row_call_launches(65539, 8192, 2, 2) == 3         # 32768, 32768, 3
    assert bench.row_call_launches(3, 2 ** 28, 2, 4) == 2          # rows over 1 GiB: two a piece
    assert [bench.dispatches_per_call(c) for c in ("5a", "5b", "5c", "5d", "6a", "9a")] == \
        [1, 2, 3, 6, 2, 1]


def test_committed_counters_match_the_sources():
    """The committed counter summaries were taken on the current sources, so the bench's
    `traffic` and the per-configuration traffic table are not silently dropped as stale:
    any source or flag change has to come with retaken counters."""
    with open(bench.TRAFFIC_FILE) as f:
        assert json.load(f)["kernel_source_hash"] == bench.kernel_source_hash()
    with open(bench.SUITE_TRAFFIC_FILE) as f:
        assert json.load(f)["library_source_hash"] == bench.library_source_hash()
    assert bench.stored_traffic(0) is not None
