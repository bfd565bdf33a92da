"""The library's routing-history writer and reader (host functions of libcoli.so)
against the oracle (oracle/usage.py), byte for byte and record for record; page
"colibrì 路由遥测全解析：.coli_usage专家历史、ROUTE_TRACE追踪流与route_trace.h统一格式"."""
import os
import struct

import numpy as np
import pytest

import int4_grouped_expert_amd as coli
from oracle import usage as U


def lib_save(path, counts, engine, decay=1.0, dropped=None):
    coli.coli_usage_save(str(path), np.asarray(counts, dtype=np.uint64),
                         coli.coli_usage_engine_hash(engine), decay, dropped)


@pytest.mark.parametrize("engine", ["glm_moe_dsa", "kimi_k3", "inkling", "x"])
def test_engine_hash_matches_oracle(engine):
    assert coli.coli_usage_engine_hash(engine) == U.fnv1a32(engine)


@pytest.mark.parametrize("seed,decay,drop", [(0, 1.0, ()), (1, 0.99, ()), (2, 0.5, (1,)),
                                            (3, 1.0, (0, 3)), (4, 2.0, ())])
def test_save_matches_oracle_bytes(tmp_path, seed, decay, drop):
    rng = np.random.default_rng(seed)
    L, E = 4, 32
    counts = rng.integers(0, 5, (L, E)) * (rng.random((L, E)) < 0.3)
    counts[0, 0] = 1  # a count of one, kept alive by the decay's rounding
    dropped = np.array([l in drop for l in range(L)], dtype=np.uint8)
    lib_save(tmp_path / "c", counts, "glm_moe_dsa", decay, dropped)
    U.save(str(tmp_path / "o"), counts.tolist(), "glm_moe_dsa", decay, set(drop))
    assert (tmp_path / "c").read_bytes() == (tmp_path / "o").read_bytes()
    assert not list(tmp_path.glob("*.tmp*"))


def test_empty_history_zero_bytes(tmp_path):
    lib_save(tmp_path / "e", np.zeros((5, 8), dtype=np.uint64), "glm_moe_dsa")
    assert (tmp_path / "e").stat().st_size == 0
    c, tot = coli.coli_usage_load(str(tmp_path / "e"), 5, 8, U.fnv1a32("glm_moe_dsa"))
    assert tot == 0 and not c.any()


def test_round_trip_both_ways(tmp_path):
    rng = np.random.default_rng(7)
    counts = rng.integers(0, 1000, (3, 64)) * (rng.random((3, 64)) < 0.2)
    h = U.fnv1a32("glm_moe_dsa")
    lib_save(tmp_path / "c", counts, "glm_moe_dsa")
    oc, ot = U.read((tmp_path / "c").read_bytes(), 3, 64, "glm_moe_dsa")
    assert oc == counts.tolist() and ot == int(counts.sum())
    U.save(str(tmp_path / "o"), counts.tolist(), "glm_moe_dsa")
    lc, lt = coli.coli_usage_load(str(tmp_path / "o"), 3, 64, h)
    assert np.array_equal(lc, counts) and lt == int(counts.sum())


@pytest.mark.parametrize("case", ["legacy", "out_of_range", "crlf", "other_engine",
                                  "other_engine_trusted", "dims", "dims_trusted", "future",
                                  "unknown_record", "dropped", "iku1_glm", "iku1_inkling",
                                  "four_fields"])
def test_reader_matches_oracle(tmp_path, case):
    n_layers, n_experts, engine, trusted, dropped = 3, 8, "glm_moe_dsa", False, ()
    good = U.history_text([[1, 0, 0, 0, 0, 0, 0, 2], [0, 3, 0, 0, 0, 0, 0, 0],
                           [0, 0, 0, 4, 0, 0, 0, 0]], "glm_moe_dsa").encode()
    data = {
        "legacy": b"0 1 2\n1 0 3\n",
        "out_of_range": b"0 1 2\n1 0 3\n7 0 300\n2 9 50\n",
        "crlf": good.replace(b"\n", b"\r\n"),
        "other_engine": U.history_text([[1] * 8] * 3, "kimi_k3").encode(),
        "other_engine_trusted": U.history_text([[1] * 8] * 3, "kimi_k3").encode(),
        "dims": U.history_text([[1] * 8] * 2, "glm_moe_dsa").encode(),
        "dims_trusted": U.history_text([[1] * 8] * 2, "kimi_k3").encode(),
        "future": good.replace(b"-2 1 ", b"-2 3 "),
        "unknown_record": good + b"-7 1 2\n2 2 6\n",
        "dropped": good,
        "iku1_glm": struct.pack("<III", U.IKU1_MAGIC, 3, 8) + bytes(4 * 24),
        "iku1_inkling": struct.pack("<III", U.IKU1_MAGIC, 3, 8) +
                        struct.pack("<24I", *range(24)),
        "four_fields": b"0 2 5\n-3 7 1 99\n1 1 8\n",
    }[case]
    if case.endswith("trusted"):
        trusted = True
    if case == "dropped":
        dropped = (1,)
    if case == "iku1_inkling":
        engine = "inkling"
    path = tmp_path / "h"
    path.write_bytes(data)
    drop = np.array([l in dropped for l in range(n_layers)], dtype=np.uint8)
    try:
        ref = U.read(data, n_layers, n_experts, engine, trusted, set(dropped))
    except U.Rejected:
        ref = None
    if ref is None:
        with pytest.raises(coli.ColiError) as ei:
            coli.coli_usage_load(str(path), n_layers, n_experts, U.fnv1a32(engine), trusted, drop)
        assert ei.value.status == coli.COLI_EUSAGE
    else:
        got, tot = coli.coli_usage_load(str(path), n_layers, n_experts, U.fnv1a32(engine),
                                        trusted, drop)
        assert got.tolist() == ref[0] and tot == ref[1]
    if case == "out_of_range":
        assert ref[1] == 5  # the page's point: only accepted counts are totalled


def test_long_path_rejected_before_touching_the_file_system(tmp_path):
    """The temporary path must fit, or the call fails before any file is created."""
    deep = str(tmp_path / ("d" * 200))
    os.makedirs(deep)
    path = os.path.join(deep, "x" * 250) + "/" + "y" * 3900  # past the 4096-byte buffer
    before = sorted(os.listdir(deep))
    with pytest.raises(coli.ColiError) as ei:
        coli.coli_usage_save(path, np.ones((1, 4), dtype=np.uint64), 1)
    assert ei.value.status == coli.COLI_EINVAL
    assert sorted(os.listdir(deep)) == before


def test_unwritable_directory_is_eio(tmp_path):
    with pytest.raises(coli.ColiError) as ei:
        coli.coli_usage_save(str(tmp_path / "no" / "such" / "dir" / "u"),
                             np.ones((1, 4), dtype=np.uint64), 1)
    assert ei.value.status == coli.COLI_EIO
