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


def test_floor_tile_lists_cover_each_key_once():
    """The read-floor probe's tile lists: per kv head, the first key of every 16-key tile of
    every request (each key of the call in exactly one tile), and the same tiles as whole
    token rows (row r of the whole-row list is row r * Hkv + h of the per-head one)."""
    import numpy as np
    import workloads as W
    b = W.make_batch([1, 16, 17, 300, 33], page_size=16, num_qo_heads=4, num_kv_heads=2, head_dim=64,
                     dtype="bf16", num_pages=64, seed=3)
    per_head, whole = bench.tile_rows(b), bench.whole_row_tiles(b)
    assert len(whole) == sum(-(-int(n) // 16) for n in b.kv_lens)
    # per-head list: request by request, kv head by kv head
    expect, i = [], 0
    for r, n in enumerate(b.kv_lens):
        t = -(-int(n) // 16)
        for h in range(b.num_kv_heads):
            expect.extend(whole[i:i + t].astype(np.int64) * b.num_kv_heads + h)
        i += t
    assert np.array_equal(per_head, np.array(expect, dtype=np.int32))
    # every token of every request lies in the tile starting at its 16-aligned position
    for r, n in enumerate(b.kv_lens):
        for t in range(int(n)):
            page = b.kv_indices[b.kv_indptr[r] + t // b.page_size]
            first = page * b.page_size + (t - t % 16) % b.page_size
            assert first in whole
