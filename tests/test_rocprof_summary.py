"""The profile summarizer: copy-calibrated traffic from two counter databases,
the staleness check that keeps a reading only while the library code is the
one it was taken on, and the comment-blind code text that check hashes."""

import os
import sqlite3

from fp8_mixture_experts_amd import rocprof_summary as R

EXPERT = "void mega_moe::moe_expert_ffn<2, 128, 0>(mega_moe::MoeArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _db(dirname, counter, rows):
    os.makedirs(dirname)
    con = sqlite3.connect(os.path.join(dirname, "run_results.db"))
    con.execute("create table counters_collection "
                "(dispatch_id int, kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)",
                    [(d, k, counter, v) for d, k, v in rows])
    con.commit()
    con.close()
    return dirname


def test_traffic_is_calibrated_by_the_copy(tmp_path):
    copy_bytes = 1 << 20
    # the copy reads 1 MiB but FETCH_SIZE reports half of it: factor 2;
    # WRITE_SIZE reports it whole: factor 1
    fetch = _db(str(tmp_path / "f"), "FETCH_SIZE",
                [(1, EXPERT, 100.0), (2, EXPERT, 120.0), (3, COPY, 512.0), (4, COPY, 8.0)])
    write = _db(str(tmp_path / "w"), "WRITE_SIZE",
                [(1, EXPERT, 10.0), (2, EXPERT, 30.0), (3, COPY, 1024.0)])
    out = str(tmp_path / "traffic.txt")
    R.traffic(fetch, write, out, "decode", "cmd", copy_bytes)
    want = 110.0 * 1024 * 2 + 20.0 * 1024 * 1
    assert R.read_traffic(out, "decode") == want
    assert R.read_traffic(out, "prefill") is None
    text = open(out).read()
    assert "fetch_factor: 2.0000" in text and "write_factor: 1.0000" in text
    assert "(dispatches: 2)" in text
    # a reading taken on other code is stale
    stale = str(tmp_path / "stale.txt")
    with open(stale, "w") as f:
        f.write(text.replace(R.sources_sha256(), "0" * 64))
    assert R.read_traffic(stale, "decode") is None
    assert R.read_traffic(str(tmp_path / "missing.txt"), "decode") is None


def test_code_text_ignores_comments_and_layout_only():
    a = 'int a = 1; // note\n/* block\n comment */ const char* s = "x // y /* z */";\n'
    b = 'int a = 1;\nconst char* s = "x // y /* z */";  /* another */\n'
    assert R.code_text(a) == R.code_text(b) == 'int a = 1; const char* s = "x // y /* z */";'
    assert R.code_text("int a = 1;") != R.code_text("int a = 2;")
    assert R.code_text("char c = '/'; // x") == "char c = '/';"
