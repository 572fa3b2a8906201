"""Host logic of the rocprofv3 summaries that bench.py's roofline reads."""
import os

from sparse_mla_attention_score_amd import rocprof_summary as rs


def test_short_names():
    assert rs.short_name("void hs::(anonymous namespace)::index_score_kernel<4, true>"
                         "(unsigned short const*, float const*)") == "index_score_kernel<4, true>"
    assert rs.short_name("hs::(anonymous namespace)::resolve_kernel(int const*, int)") == "resolve_kernel"


def _write_csv(path, header, rows):
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(f'"{x}"' if isinstance(x, str) else str(x) for x in r) + "\n")


def test_stats_and_traffic_roundtrip(tmp_path):
    trace = tmp_path / "trace"
    trace.mkdir()
    name = "void hs::(anonymous namespace)::index_score_kernel<4, true>(float*)"
    _write_csv(trace / "p_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [[name, 1000, 401000], [name, 500000, 1000000], ["void hs::topk_select_kernel(int)", 0, 90000]])
    st = rs.kernel_stats(str(trace))
    assert st[0][0] == "index_score_kernel<4, true>" and st[0][1] == 2
    assert abs(st[0][2] - 450.0) < 1e-9 and abs(st[0][3] - 400.0) < 1e-9
    for counter, val, sub in (("FETCH_SIZE", 550000.0, "f"), ("WRITE_SIZE", 135000.0, "w")):
        d = tmp_path / sub
        d.mkdir()
        _write_csv(d / "p_counter_collection.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"],
                   [[name, counter, val], [name, counter, val + 2], ["void hs::decode(int)", counter, 1.0]])
    out = tmp_path / "traffic.txt"
    import contextlib, io
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        rs.main(["traffic", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
                 "--kernel", "index_score"])
    out.write_text("# a comment: ignored\n" + buf.getvalue())
    want = int(round(550001.0 * 1024 * 2 + 135001.0 * 1024))
    assert rs.read_traffic(str(out)) == want
    # a figure measured on other sources is not reported
    out.write_text(buf.getvalue().replace(rs.source_fingerprint("index_score_kernel"), "0" * 16))
    assert rs.read_traffic(str(out)) is None
    assert rs.read_traffic(str(tmp_path / "missing.txt")) is None
