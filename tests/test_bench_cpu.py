"""Host logic of bench.py: committed profile summaries are read only while the
kernel sources they were taken on are unchanged."""
import os

import bench


def _summary(tmp_path, sha, extra="- gateup_narrow_avg_us: 25.00\n"):
    p = tmp_path / "summary.md"
    p.write_text("# a summary\n\ntext\n\n" + extra + f"- source_sha256: `{sha}`\n")
    return str(p)


def test_source_sha_covers_every_file(tmp_path, monkeypatch):
    a, b = tmp_path / "a.h", tmp_path / "b.hip"
    a.write_bytes(b"one")
    b.write_bytes(b"two")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_sha256(("a.h", "b.hip"))
    b.write_bytes(b"two!")
    assert bench.source_sha256(("a.h", "b.hip")) != h
    assert bench.source_sha256(("b.hip", "a.h")) != bench.source_sha256(("a.h", "b.hip"))


def test_profile_fields_match_and_mismatch(tmp_path, monkeypatch):
    (tmp_path / "k.hip").write_bytes(b"kernel v1")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.source_sha256(("k.hip",))
    f = bench.profile_fields(_summary(tmp_path, sha), ("k.hip",))
    assert f is not None and f["gateup_narrow_avg_us"] == "25.00" and f["source_sha256"] == sha
    (tmp_path / "k.hip").write_bytes(b"kernel v2")
    assert bench.profile_fields(_summary(tmp_path, sha), ("k.hip",)) is None
    assert bench.profile_fields(str(tmp_path / "absent.md"), ("k.hip",)) is None


def test_committed_summaries_name_the_narrow_sources():
    """The committed T=1 summaries carry a sha and name the files it covers."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for name in ("decode_t1_kernels.md", "gateup_narrow_decode_t1_traffic.md"):
        text = open(os.path.join(root, "profiles", name)).read()
        assert "- source_sha256: `" in text
        for src in bench.NARROW_SRC:
            assert src in text, (name, src)
