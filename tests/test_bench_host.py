"""Host logic of bench.py (no GPU): the source hash that ties a recorded
traffic measurement to the kernel code it was taken on."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _files(text):
    names = bench.KERNEL_SOURCES["mfma"]
    base = {n: open(os.path.join(bench.CSRC, n), encoding="utf-8").read() for n in names}
    return base, (lambda n: text(n, base[n]))


def test_comment_edits_keep_the_hash():
    base, read = _files(lambda n, t: t.replace("\n", "  // a remark\n", 3) + "\n/* more\n words */\n")
    assert bench.kernel_source_hash("mfma", read) == bench.kernel_source_hash("mfma", base.get)


def test_code_edits_change_the_hash():
    first = sorted(bench.KERNEL_SOURCES["mfma"])[0]
    base, read = _files(lambda n, t: t + "\nint kvd_unused_symbol;\n" if n == first else t)
    assert bench.kernel_source_hash("mfma", read) != bench.kernel_source_hash("mfma", base.get)


def test_code_text_strips_comments_only():
    src = "int a = 1; // one\n/* two\n three */ int b = 2;\n"
    assert bench.code_text(src) == "int a = 1; int b = 2;"


def test_traffic_needs_the_same_kernel_form(tmp_path, monkeypatch):
    """A traffic record counts only for the kernel source and the kernel
    form (RoPE and append fused into the split kernel, or not) it was
    taken on."""
    import json
    rec = {"kernel_match": "decode_mfma_kernel<128, false, true>", "kernel_source_hash": "abc",
           "hbm_bytes_per_launch": 123}
    (tmp_path / "traffic_w.json").write_text(json.dumps(rec))
    rec2 = dict(rec, kernel_match="decode_i8_kernel_wide<128, false>")
    (tmp_path / "traffic_v.json").write_text(json.dumps(rec2))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.load_traffic("w", "abc", True) == 123
    assert bench.load_traffic("w", "abc", False) is None
    assert bench.load_traffic("w", "abd", True) is None
    assert bench.load_traffic("v", "abc", False) == 123
    assert bench.load_traffic("v", "abc", True) is None
    assert bench.load_traffic("missing", "abc", False) is None
