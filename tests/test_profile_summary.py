"""The profile summaries that turn rocprofv3 result databases into the figures
of profiles/ and of the bench line's `traffic` field, checked on small
databases with the same tables (kernels: name, duration in ns;
counters_collection: kernel_name, counter_name, value)."""

import re
import sqlite3

import pytest

from fp8_quantized_skinny_amd import profile_summary as ps

STREAM = "_ZN6skinny12_GLOBAL__N_112nvfp4_streamILi5ELi1EEEvNS0_9Nvfp4ArgsE"
FINAL = "_ZN6skinny12_GLOBAL__N_115finalize_splitsILb0EEEvPKfiiiS3_PDF16_Py"
COPY = "__amd_rocclr_copyBuffer"


def _trace_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, duration integer)")
    con.executemany("insert into kernels values (?, ?)", rows)
    con.commit()
    con.close()
    return str(path)


def _counter_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?)", rows)
    con.commit()
    con.close()
    return str(path)


def test_kernel_names_keep_their_template_arguments():
    assert ps._short(STREAM) == "skinny::nvfp4_stream<5, 1>"
    assert ps._short(FINAL) == "skinny::finalize_splits<false>"
    assert ps._short(COPY) == COPY


def test_trace_statistics_in_microseconds(tmp_path, capsys):
    durs = [10_000, 11_000, 12_000, 13_000, 50_000]          # ns
    db = _trace_db(tmp_path / "t.db", [(STREAM, d) for d in durs] + [(FINAL, 4_500)])
    rows = ps.trace_rows(db, "nvfp4")
    assert list(rows) == ["skinny::nvfp4_stream<5, 1>"]
    assert rows["skinny::nvfp4_stream<5, 1>"].tolist() == [10.0, 11.0, 12.0, 13.0, 50.0]
    ps.main(["trace", db])
    out = capsys.readouterr().out.splitlines()
    stream = next(l for l in out if l.startswith("skinny::nvfp4_stream"))
    calls, mean, median = stream.split()[2:5]
    assert (int(calls), float(mean), float(median)) == (5, 19.2, 12.0)


def test_traffic_scales_each_counter_by_the_copy_calibration(tmp_path, capsys):
    # A copy of 512 MB that reads 250 000 and writes 500 000 counts makes one
    # FETCH_SIZE count 2048 bytes and one WRITE_SIZE count 1024 bytes.
    f = _counter_db(tmp_path / "f.db", [(STREAM, "FETCH_SIZE", v) for v in (100.0, 110.0, 120.0)])
    w = _counter_db(tmp_path / "w.db", [(STREAM, "WRITE_SIZE", 16.0)] * 3)
    cf = _counter_db(tmp_path / "cf.db", [(COPY, "FETCH_SIZE", 250_000.0)])
    cw = _counter_db(tmp_path / "cw.db", [(COPY, "WRITE_SIZE", 500_000.0)])
    ps.main(["traffic", f, w, cf, cw, "--match", "nvfp4_stream", "--copy-bytes", "512000000"])
    out = dict(re.findall(r"^(\w+_bytes_per_launch): (\d+)$", capsys.readouterr().out, re.M))
    assert int(out["hbm_read_bytes_per_launch"]) == 110 * 2048          # median count x bytes per count
    assert int(out["hbm_write_bytes_per_launch"]) == 16 * 1024
    assert int(out["traffic_bytes_per_launch"]) == 110 * 2048 + 16 * 1024


def test_traffic_refuses_an_ambiguous_kernel_match(tmp_path):
    f = _counter_db(tmp_path / "f.db", [(STREAM, "FETCH_SIZE", 1.0), (FINAL, "FETCH_SIZE", 2.0)])
    w = _counter_db(tmp_path / "w.db", [(STREAM, "WRITE_SIZE", 1.0)])
    cf = _counter_db(tmp_path / "cf.db", [(COPY, "FETCH_SIZE", 1.0)])
    cw = _counter_db(tmp_path / "cw.db", [(COPY, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        ps.main(["traffic", f, w, cf, cw, "--match", "skinny"])


def test_sources_hash_is_stable_hex():
    h = ps.sources_sha256()
    assert re.fullmatch(r"[0-9a-f]{64}", h) and h == ps.sources_sha256()


def test_sources_hash_ignores_comments_not_code():
    a = "int f(int x) {  // doubles\n  return 2 * x;  /* the\n result */\n}\n"
    b = "int f(int x) {\n\n    return 2 * x;\n}\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert ps._code_only(a) == ps._code_only(b)
    assert ps._code_only(a) != ps._code_only(c)
