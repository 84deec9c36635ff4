"""Host logic that ties the committed rocprofv3 summaries to the code they were taken with."""
import os
import re

from sparse_weight_direct_amd import rocprof_summary as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _digest_of(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    return rs._code_only(str(p))


def test_code_digest_ignores_comments_but_not_code(tmp_path):
    base = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\nint g = 2;\n"
    a = _digest_of(tmp_path, "a.cpp", base)
    # comments reworded, a blank line and trailing blanks added: the same code
    b = _digest_of(tmp_path, "b.cpp", base.replace("// one more", "// the successor").replace(
        "/* block\n comment */", "/* another\n block */") + "\n   \n")
    assert a == b
    # a changed constant, a string that holds "//" after code: different code
    assert _digest_of(tmp_path, "c.cpp", base.replace("x + 1", "x + 2")) != a
    s = 'const char* k = "a//b";\n'
    assert _digest_of(tmp_path, "d.cpp", s) == s.rstrip("\n").encode()
    py = "x = 1\n# note\ny = x  # trailing\n"
    assert _digest_of(tmp_path, "e.py", py) == _digest_of(tmp_path, "f.py", "x = 1\n# other note\ny = x  # trailing\n")


def test_stored_traffic_summary_has_the_keys_the_bench_reads():
    path = os.path.join(ROOT, "profiles", "sc_baked_imb95_traffic.txt")
    kv = {}
    for line in open(path):
        m = re.match(r"^(\w+):\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    assert kv["workload"] == "imb95" and kv["kernel"] == "sc_baked"
    assert re.fullmatch(r"[0-9a-f]{16}", kv["kernel_digest"])
    fetch, write, total = (float(kv[k]) for k in ("fetch_bytes_per_launch", "write_bytes_per_launch",
                                                  "traffic_bytes_per_launch"))
    assert abs(fetch + write - total) <= 2
    # at least the compulsory bytes of the layer (input and output once), at most twice them
    alg = 2 * 8 * 128 * 112 * 112 * 4
    assert alg <= total <= 2 * alg
