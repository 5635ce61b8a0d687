"""The counter records in profiles/traffic.json are tied to the code they were
taken on by a hash of the kernel sources' comment-free text (CPU only)."""
import json
import os

from matrix_core_scheduling_amd import profiling as pr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_text_drops_comments_and_keeps_strings():
    src = 'int a = 1; // one\n/* two\n lines */ int b = 2;\nconst char *s = "//x /*y*/"; char c = \'/\';\n'
    assert pr.code_text(src) == 'int a = 1; int b = 2; const char *s = "//x /*y*/"; char c = \'/\';'
    assert pr.code_text("a  \n\t b") == "a b"
    assert pr.code_text("x /* unterminated") == "x"


def test_comment_edits_keep_the_hash_and_code_edits_change_it(tmp_path, monkeypatch):
    for name in ("k.hip", "device.h", "internal.h"):
        (tmp_path / name).write_text("int f() { return 1; } // note\n")
    monkeypatch.setattr(pr, "CSRC", str(tmp_path))
    monkeypatch.setitem(pr.KERNEL_SOURCES, "probe", ("k.hip", "device.h", "internal.h"))
    h0 = pr.kernel_code_hash("probe")
    (tmp_path / "k.hip").write_text("// a new comment\nint f() {\n  return 1;  /* same code */\n}\n")
    assert pr.kernel_code_hash("probe") == h0
    (tmp_path / "k.hip").write_text("int f() { return 2; }\n")
    assert pr.kernel_code_hash("probe") != h0


def test_every_record_names_a_known_kernel_and_has_its_fields():
    data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert data
    for key, rec in data.items():
        sched = key.split("@")[1] if "@" in key else "pipelined"
        assert sched in pr.KERNEL_SOURCES, key
        assert len(rec["kernel_code_sha256"]) == 64, key
        assert abs(rec["hbm_bytes_per_launch"] - rec["fetch_bytes_per_launch"] - rec["write_bytes_per_launch"]) <= 1, key
