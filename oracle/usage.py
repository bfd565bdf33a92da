"""The oracle of the routing-history file ``.coli_usage`` and of its counters.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``): only the test
suite may import it; the product never imports it.

Source: page "colibrì 路由遥测全解析：.coli_usage专家历史、ROUTE_TRACE追踪流与
route_trace.h统一格式", sections 历史文件 .coli_usage、stats.txt 与 PIN=file,
头部记录为什么长这样, 以后再加头部记录：三条铁律, 空历史 = 零字节文件,
仍然兼容读取的旧布局, 可信读取, 运行时环境变量一览 (COLI_USAGE_DECAY) and
测试与 CI 保障.  Written from the description, in plain Python:

* the counters: per (layer, expert), the number of routing decisions that chose
  the expert (every (token, slot) pair counts once);
* the file is text, one record per line, three numeric fields: first
  ``-1 n_layers n_experts``, then ``-2 format_version engine_hash``, then one
  ``layer expert count`` triple per non-zero counter (sparse), layers and experts
  ascending; a history whose counts are all zero is a zero-byte file (no
  header); the file is replaced atomically (a temporary file, then rename);
* the engine is identified by a 32-bit hash of its name in the third field of
  the ``-2`` record; the page prints the hash of ``glm_moe_dsa`` as 3815245270,
  which is the 32-bit FNV-1a hash;
* readers: the legacy loop reads three numbers at a time while three are read,
  keeps records whose layer and expert are in range and skips the rest (so the
  negative header records are skipped by old readers); the full reader also
  checks the header: the dimensions must match, the version must be known, and
  the engine hash must match unless the read is trusted (trust relaxes only the
  identity check); legacy files without a header are accepted as they are; a
  dense binary layout with the magic ``IKU1`` is read only by the engine
  ``inkling``; rows dropped by the engine (layers with no router) never absorb
  counts; the total reported is the sum of the accepted counts only;
* decay (optional, in (0, 1]; other values are ignored): each count becomes
  round(count * decay), except that a non-zero count never rounds to 0.
"""
from __future__ import annotations

import os
import struct

FORMAT_VERSION = 1
IKU1_MAGIC = 0x31554B49
U32_MAX = 0xFFFFFFFF


class Rejected(Exception):
    """The history file was refused (identity, geometry or version)."""


def fnv1a32(name: str) -> int:
    h = 0x811C9DC5
    for b in name.encode():
        h ^= b
        h = (h * 0x01000193) & 0xFFFFFFFF
    return h


def apply_decay(count: int, decay: float) -> int:
    if not (0.0 < decay <= 1.0) or decay == 1.0:
        return count
    v = int(count * decay + 0.5)
    return 1 if (count > 0 and v == 0) else v


def count_routes(idx, n_layers: int, n_experts: int, layer: int, counts=None):
    """Counters [n_layers][n_experts] plus one count per (token, slot) pair of idx
    routed at `layer` (ids outside [0, n_experts) are not counted)."""
    if counts is None:
        counts = [[0] * n_experts for _ in range(n_layers)]
    for row in idx:
        for e in row:
            e = int(e)
            if 0 <= e < n_experts:
                counts[layer][e] += 1
    return counts


def history_text(counts, engine: str, decay: float = 1.0, dropped=()) -> str:
    """The file's bytes (as text) for the counters; '' when every count is zero."""
    n_layers = len(counts)
    n_experts = len(counts[0]) if n_layers else 0
    rows = []
    for l in range(n_layers):
        if l in dropped:
            continue
        for e in range(n_experts):
            c = min(apply_decay(int(counts[l][e]), decay), U32_MAX)
            if c:
                rows.append(f"{l} {e} {c}\n")
    if not rows:
        return ""
    head = f"-1 {n_layers} {n_experts}\n-2 {FORMAT_VERSION} {fnv1a32(engine)}\n"
    return head + "".join(rows)


def save(path: str, counts, engine: str, decay: float = 1.0, dropped=()) -> None:
    tmp = f"{path}.tmp.{os.getpid()}"
    with open(tmp, "w", newline="\n") as f:
        f.write(history_text(counts, engine, decay, dropped))
    os.replace(tmp, path)


def triples(text: str):
    """Three numbers at a time, as the legacy loop reads them (stops at the first
    token that is not a number or when fewer than three remain)."""
    toks = text.split()
    out = []
    i = 0
    while i + 3 <= len(toks):
        try:
            a, b, c = int(toks[i]), int(toks[i + 1]), int(toks[i + 2])
        except ValueError:
            break
        out.append((a, b, c))
        i += 3
    return out


def legacy_read(text: str, n_layers: int, n_experts: int):
    """The legacy reader: every record with 0 <= layer < n_layers and 0 <= expert <
    n_experts is added; everything else (headers included) is skipped."""
    counts = [[0] * n_experts for _ in range(n_layers)]
    n = 0
    for l, e, c in triples(text):
        if 0 <= l < n_layers and 0 <= e < n_experts:
            counts[l][e] += c
            n += 1
    return counts, n


def read(data: bytes, n_layers: int, n_experts: int, engine: str, trusted: bool = False,
         dropped=()):
    """The full reader.  Returns (counts, accepted_total); raises Rejected."""
    counts = [[0] * n_experts for _ in range(n_layers)]
    if len(data) == 0:
        return counts, 0
    if len(data) >= 4 and struct.unpack_from("<I", data, 0)[0] == IKU1_MAGIC:
        if engine != "inkling":
            raise Rejected("IKU1 history belongs to inkling")
        if len(data) < 12:
            raise Rejected("IKU1 header truncated")
        _, nl, ne = struct.unpack_from("<III", data, 0)
        if nl != n_layers or ne != n_experts or len(data) < 12 + 4 * nl * ne:
            raise Rejected("IKU1 geometry differs")
        total = 0
        for l in range(nl):
            for e in range(ne):
                c = struct.unpack_from("<I", data, 12 + 4 * (l * ne + e))[0]
                if l in dropped:
                    continue
                counts[l][e] += c
                total += c
        return counts, total
    text = data.decode("ascii", errors="replace")
    total = 0
    for l, e, c in triples(text):
        if l == -1:
            if e != n_layers or c != n_experts:
                raise Rejected("dimensions differ")
            continue
        if l == -2:
            if e != FORMAT_VERSION:
                raise Rejected("unknown format version")
            if (c & U32_MAX) != fnv1a32(engine) and not trusted:
                raise Rejected("written by another engine")
            continue
        if l < 0:
            continue  # a record type this reader does not know
        if l >= n_layers or e < 0 or e >= n_experts or l in dropped:
            continue
        counts[l][e] += c
        total += c
    return counts, total
