"""The measured dispatch table: the library follows the table file it is
given, interpolates between the measured M as the file's ranges say, falls
back to the built-in rules for shapes it does not list, and ignores lines it
cannot use.  Each case runs in a fresh process (the table is read once)."""
from __future__ import annotations

import json
import os
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "quantized_skinny_gemm_amd", "dispatch_table.txt")
TYPES = {"f32": 0, "f16": 1, "q4_0": 2, "q4_0r": 4}


def _dispatch(table_text, queries, extra_env=None):
    """[mm_dispatch(...)[0] for each (type, M, N, K)] in a subprocess that reads
    table_text (None: the committed file beside the library)."""
    env = dict(os.environ)
    path = None
    if table_text is not None:
        import tempfile
        fd, path = tempfile.mkstemp(suffix=".txt")
        with os.fdopen(fd, "w") as fh:
            fh.write(textwrap.dedent(table_text))
        env["MM_DISPATCH_TABLE"] = path
    else:
        env.pop("MM_DISPATCH_TABLE", None)
    env.update(extra_env or {})
    code = ("import json, sys; sys.path.insert(0, %r)\n"
            "import quantized_skinny_gemm_amd as qs\n"
            "q = json.loads(sys.argv[1])\n"
            "print(json.dumps([qs.dispatch(t, m, n, k)[0] for t, m, n, k in q]))\n") % ROOT
    try:
        r = subprocess.run([sys.executable, "-c", code, json.dumps(queries)], env=env,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        return json.loads(r.stdout.strip().splitlines()[-1]), r.stderr
    finally:
        if path:
            os.unlink(path)


def test_table_choices_are_followed():
    table = """
        # a made-up table: the wide kernel from M = 3, the narrow one below
        q4_0 4096 4096 1 2 1
        q4_0 4096 4096 3 2147483647 2
        f16 4096 4096 1 5 1
        f16 4096 4096 6 2147483647 3
    """
    q = [[2, 1, 4096, 4096], [2, 2, 4096, 4096], [2, 3, 4096, 4096], [2, 17, 4096, 4096],
         [1, 5, 4096, 4096], [1, 6, 4096, 4096], [1, 300, 4096, 4096],
         # not in the table: the built-in rules (skinny for Q4_0 at M = 8)
         [2, 8, 4096, 8192], [2, 8, 4096, 4096 + 32]]
    got, _ = _dispatch(table, q)
    assert got == [1, 1, 2, 2, 1, 3, 3, 3, 3]


def test_unusable_lines_are_ignored_and_logged():
    table = """
        q4_0 4096 4096 1 8 7
        f32 4096 4096 1 8 2
        q4_0r 4096 4096 1 8 1
        q4_0 4096 4096 9 4
        q4_0 4096 4096 1 8 2 extra
        bogus 4096 4096 1 8 2
    """
    got, err = _dispatch(table, [[2, 4, 4096, 4096], [0, 4, 4096, 4096], [4, 4, 4096, 4096]],
                         {"MM_VERBOSE": "1"})
    # rules: Q4_0 M = 4 skinny, F32 M = 4 skinny, repacked M = 4 skinny; the
    # line with a trailing field is read (sscanf reads the first six)
    assert got == [2, 3, 3]
    assert "ignored" in err and "dispatch table" in err


def test_missing_table_means_rules():
    got, err = _dispatch(None, [[2, 1, 4096, 4096]], {"MM_DISPATCH_TABLE": "/nonexistent/x.txt",
                                                      "MM_VERBOSE": "1"})
    assert got == [1]
    assert "not found" in err


def test_committed_table_is_followed():
    """Every range of the committed table, at its ends and middle."""
    if not os.path.exists(TABLE):
        return
    rows = []
    for line in open(TABLE):
        line = line.split("#")[0].split()
        if len(line) == 6:
            t, n, k, lo, hi, v = line
            rows.append((TYPES[t], int(n), int(k), int(lo), min(int(hi), 4096), int(v)))
    assert rows, "the committed table is empty"
    q, want = [], []
    for t, n, k, lo, hi, v in rows:
        for m in sorted({lo, hi, (lo + hi) // 2}):
            q.append([t, m, n, k])
            want.append(v)
    got, _ = _dispatch(None, q)
    assert got == want
