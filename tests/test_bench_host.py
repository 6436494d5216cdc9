"""Host-side pieces of bench.py: the code hash that decides whether a committed HBM-counter
summary still describes the kernel and planner sources."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _text(tmp_path, src):
    p = tmp_path / "k.hip"
    p.write_text(src)
    return bench.code_text(str(p))


def test_code_text_drops_comments_and_blank_lines(tmp_path):
    a = _text(tmp_path, "int a = 1;  // one\n\n/* block\n comment */int b = 2;\n")
    b = _text(tmp_path, "int a = 1;\n// another comment\nint b = 2;   \n")
    assert a == b == "int a = 1;\nint b = 2;"


def test_code_text_keeps_literals_and_sees_code_changes(tmp_path):
    a = _text(tmp_path, 'const char *s = "a // not a comment"; char c = \'/\';\n')
    assert "// not a comment" in a and "'/'" in a
    assert _text(tmp_path, "int x = 1;\n") != _text(tmp_path, "int x = 2;\n")
    # an escaped quote does not end the literal
    e = _text(tmp_path, 'const char *s = "q\\" // still text"; // gone\n')
    assert "still text" in e and "gone" not in e


def test_source_hash_is_stable():
    assert bench.source_hash() == bench.source_hash()
    assert len(bench.source_hash()) == 16


def test_more_than_one_gpu_is_refused_before_any_gpu_work(capsys):
    """The benchmark measures one GPU: --gpus N > 1 exits with status 2 and a message,
    before torch or the library is imported."""
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err
