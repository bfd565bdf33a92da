"""Pins for the oracle of the routing history (oracle/usage.py).

Page "colibrì 路由遥测全解析：.coli_usage专家历史、ROUTE_TRACE追踪流与route_trace.h统一格式":
the printed engine hash, the printed header records, the printed four-field example
that an old reader misreads, the 5-versus-305 totals of a legacy file with
out-of-range records, and the contract points its test list names (empty history =
zero bytes, exactly three fields per record, identity and geometry refusals, trusted
reads, dropped rows, the dense IKU1 layout, decay that keeps count-1 experts).
"""
import os
import struct

import numpy as np
import pytest

from oracle import usage as U

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "usage_engine_hash.txt")


def test_engine_hash_is_the_printed_value():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    for name, h in rows:
        assert U.fnv1a32(name) == int(h)
        assert int(h) > 2 ** 31 - 1  # the page's point: above INT_MAX, hence the third field


def test_empty_history_is_zero_bytes(tmp_path):
    p = tmp_path / ".coli_usage"
    U.save(str(p), [[0] * 8 for _ in range(5)], "glm_moe_dsa")
    assert p.exists() and p.stat().st_size == 0


def test_header_records_and_sparse_triples(tmp_path):
    counts = [[0] * 8 for _ in range(5)]
    counts[0][3] = 2
    counts[4][7] = 9
    p = tmp_path / ".coli_usage"
    U.save(str(p), counts, "kimi_k3")
    lines = p.read_text().splitlines()
    assert lines[0] == "-1 5 8"  # the page's Case 2: "-1 5 8" is the first record
    assert lines[1] == f"-2 1 {U.fnv1a32('kimi_k3')}"
    assert lines[2:] == ["0 3 2", "4 7 9"]  # only non-zero counters
    assert all(len(l.split()) == 3 for l in lines)  # exactly three fields
    assert all(all(t.lstrip("-").isdigit() for t in l.split()) for l in lines)  # all numeric
    assert not list(tmp_path.glob("*.tmp*"))  # the temporary file was renamed away


def test_round_trip_and_old_reader(tmp_path):
    rng = np.random.default_rng(0)
    counts = [[int(v) for v in rng.integers(0, 4, 16)] for _ in range(3)]
    p = tmp_path / "u"
    U.save(str(p), counts, "glm_moe_dsa")
    got, total = U.read(p.read_bytes(), 3, 16, "glm_moe_dsa")
    assert got == counts and total == sum(map(sum, counts))
    # the legacy loop reads the same file: headers skipped, same records and totals
    old, n = U.legacy_read(p.read_text(), 3, 16)
    assert old == counts and n == sum(1 for r in counts for c in r if c)


def test_four_field_record_misleads_the_old_reader():
    """The page's example: an old reader of '3 2 5 | -3 7 12 99 | 4 1 8' admits
    3 2 5, skips -3 7 12, then admits 99 4 1 made of the leftover 99 and two fields
    of the next line; the real 4 1 8 is lost."""
    text = "3 2 5\n-3 7 12 99\n4 1 8\n"
    assert U.triples(text) == [(3, 2, 5), (-3, 7, 12), (99, 4, 1)]
    counts, n = U.legacy_read(text, 100, 10)
    assert n == 2 and counts[3][2] == 5 and counts[99][4] == 1 and counts[4][1] == 0


def test_legacy_file_accepted_and_out_of_range_not_counted():
    """A header-less legacy file is accepted as it is; a record past the model's
    layers is discarded and does not inflate the total (5, not 305)."""
    text = b"0 1 2\n1 0 3\n7 0 300\n"
    counts, total = U.read(text, 2, 4, "glm_moe_dsa")
    assert total == 5
    assert counts[0][1] == 2 and counts[1][0] == 3


def test_crlf_history():
    counts, total = U.read(b"-1 2 4\r\n-2 1 3815245270\r\n1 3 7\r\n", 2, 4, "glm_moe_dsa")
    assert total == 7 and counts[1][3] == 7


def test_refusals_and_trusted_reads():
    good = U.history_text([[1, 0], [0, 2]], "kimi_k3").encode()
    with pytest.raises(U.Rejected):
        U.read(good, 3, 2, "kimi_k3")  # other dimensions
    with pytest.raises(U.Rejected):
        U.read(good, 2, 2, "glm_moe_dsa")  # another engine's history
    counts, total = U.read(good, 2, 2, "glm_moe_dsa", trusted=True)  # trust relaxes identity
    assert total == 3
    with pytest.raises(U.Rejected):
        U.read(good, 3, 2, "glm_moe_dsa", trusted=True)  # but never the geometry
    future = good.replace(b"-2 1 ", b"-2 2 ")
    with pytest.raises(U.Rejected):
        U.read(future, 2, 2, "kimi_k3", trusted=True)  # nor a future version


def test_dropped_rows_take_no_counts():
    text = U.history_text([[4, 0], [0, 5], [6, 0]], "olmoe").encode()
    counts, total = U.read(text, 3, 2, "olmoe", dropped={1})
    assert total == 10 and counts[1] == [0, 0]
    # and a dropped row is not written back
    assert "1 1 5" not in U.history_text([[4, 0], [0, 5], [6, 0]], "olmoe", dropped={1})


def test_iku1_dense_layout():
    dense = struct.pack("<III", U.IKU1_MAGIC, 2, 3) + struct.pack("<6I", 1, 0, 2, 0, 0, 3)
    with pytest.raises(U.Rejected):
        U.read(dense, 2, 3, "glm_moe_dsa")  # refused by name for every other engine
    counts, total = U.read(dense, 2, 3, "inkling")  # placed by position for inkling
    assert counts == [[1, 0, 2], [0, 0, 3]] and total == 6
    with pytest.raises(U.Rejected):
        U.read(dense, 3, 3, "inkling")


def test_decay_keeps_count_one_experts():
    assert U.history_text([[1, 1000, 50, 0]], "x", decay=0.99).splitlines()[2:] == \
        ["0 0 1", "0 1 990", "0 2 50"]
    # 1.0 and values outside (0, 1] leave the counts as they are
    for d in (1.0, 0.0, 1.5, -0.3):
        assert U.history_text([[3, 7]], "x", decay=d) == U.history_text([[3, 7]], "x")


def test_count_routes_is_bincount():
    rng = np.random.default_rng(3)
    idx = rng.integers(-2, 20, size=(50, 6))
    c = U.count_routes(idx, 4, 16, 2)
    flat = idx.reshape(-1)
    ref = np.bincount(flat[(flat >= 0) & (flat < 16)], minlength=16)
    assert c[2] == ref.tolist() and all(sum(r) == 0 for i, r in enumerate(c) if i != 2)
