"""GPU parity of the quantiser and planar packer (bit-exact bytes and scale bits).

Rule: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战", section 权重转换.
Every case compares coli_quant_int4_g64 with the oracle on the same fp32 input.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._golden import load_quant_case
from tests.harness import log

pytestmark = pytest.mark.gpu


def gpu_quant(w_host: np.ndarray):
    import int4_grouped_expert_amd as coli
    rows, cols = w_host.shape
    G = -(-cols // 64)
    w = torch.from_numpy(np.ascontiguousarray(w_host)).cuda()
    packed = torch.full((max(rows, 1), G * 32), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((max(rows, 1), G), 7.0, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    coli.coli_quant_int4_g64(w, packed, scales, status)
    torch.cuda.synchronize()
    return packed.cpu().numpy()[:rows], scales.cpu().numpy()[:rows], int(status.item())


def assert_same(w):
    p, s, st = gpu_quant(w)
    pr, sr, str_ = oracle.quant_int4_g64(w)
    assert st == str_
    assert np.array_equal(p, pr)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))


@pytest.mark.parametrize("name", ["quant_E1.txt", "quant_E2.txt", "quant_E3.txt",
                                  "quant_E4.txt"])
def test_golden(name):
    log(f"quant golden {name}")
    w, want, scale = load_quant_case(name)
    p, s, st = gpu_quant(w)
    assert st == 0
    assert bytes(p[0]) == want
    assert int(s[0, 0:1].view(np.uint32)[0]) == scale


@pytest.mark.parametrize("rows,cols", [(1, 64), (7, 200), (33, 1), (5, 63), (3, 65),
                                       (16, 130), (64, 6144), (300, 2048), (2, 4098)])
def test_random_shapes(rows, cols):
    log(f"quant random {rows}x{cols}")
    rng = np.random.default_rng(rows * 1000 + cols)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    assert_same(w)


def test_ties_and_scales():
    """Exact ties after division for many power-of-two and non-power-of-two scales."""
    rng = np.random.default_rng(1)
    rows = 512
    q = rng.integers(-7, 8, size=(rows, 64)).astype(np.float64)
    q[:, 0] = 7
    half = rng.random((rows, 64)) < 0.3
    q = np.where(half, q + 0.5 * np.sign(rng.standard_normal((rows, 64))), q)
    q[:, 0] = 7
    s = rng.uniform(1e-3, 1.0, size=(rows, 1))
    s[: rows // 2] = 2.0 ** rng.integers(-12, 3, size=(rows // 2, 1))
    w = (q * s).astype(np.float32)
    assert_same(w)


def test_quotients_near_rounding_boundaries():
    """Quotients w/s within a few ulp of every half-integer in [-6.5, 6.5] (inside the
    band where the library divides) and about 2^-17 from it (the edge of that band),
    for scales spanning 2^-60 .. 2^60: every nibble is rint(fl32(w/s)) as the oracle
    rounds it."""
    rng = np.random.default_rng(5)
    rows = 4096
    amax = rng.uniform(1e-6, 1e3, size=rows).astype(np.float32)
    amax[:1024] = (2.0 ** rng.integers(-60, 60, size=1024) *
                   rng.uniform(1.0, 2.0, size=1024)).astype(np.float32)
    s = (amax / np.float32(7.0)).astype(np.float32)
    half = rng.integers(-7, 7, size=(rows, 63)).astype(np.float64) + 0.5
    band = np.where(rng.random((rows, 63)) < 0.5, -1.0, 1.0) * 2.0 ** -17
    band *= rng.uniform(0.9, 1.1, size=(rows, 63))
    quot = np.where(np.arange(rows)[:, None] < rows // 4, half + band, half)
    t = (quot * s[:, None].astype(np.float64)).astype(np.float32)
    ulps = rng.integers(-6, 7, size=(rows, 63)).astype(np.int32)
    ulps[: rows // 4] = 0
    t = (t.view(np.int32) + ulps).view(np.float32)
    w = np.empty((rows, 64), dtype=np.float32)
    w[:, 0] = amax
    w[:, 1:] = t
    assert np.all(np.abs(w[:, 1:]) < amax[:, None])
    assert_same(w)


@pytest.mark.parametrize("H,I", [(200, 72), (64, 33), (6144, 2048)])
def test_expert_finish_group_major_copies(H, I):
    """coli_quant_expert fills the blob's group-major and 8-row blocked scale copies:
    sT[g][o] = s[o][g], sB[o // 8][g][o % 8] = s[o][g] (zero past the last row)."""
    import int4_grouped_expert_amd as coli
    from tests.harness import device_sections
    blob = torch.zeros(coli.coli_expert_blob_bytes(H, I), dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(H * 7 + I)
    wg = torch.randn((I, H), generator=g, device="cuda")
    wu = torch.randn((I, H), generator=g, device="cuda")
    wd = torch.randn((H, I), generator=g, device="cuda")
    coli.coli_quant_expert(blob.data_ptr(), H, I, wg, wu, wd)
    torch.cuda.synchronize()
    sec = device_sections(blob.cpu().numpy(), H, I)
    from tests.harness import blocked8
    for k in ("gs", "us", "ds"):
        assert np.array_equal(sec[k + "T"].view(np.uint32), sec[k].T.view(np.uint32)), k
        assert np.array_equal(sec[k + "B"].view(np.uint32), blocked8(sec[k]).view(np.uint32)), k
    ref = oracle.quant_int4_g64(wd.cpu().numpy())
    assert np.array_equal(sec["ds"].view(np.uint32), ref[1].view(np.uint32))


def test_subnormal_and_extreme_magnitudes():
    rng = np.random.default_rng(2)
    bits = rng.integers(1, 0x7F7FFFFF, size=(256, 64), dtype=np.uint32)
    bits[:64] = rng.integers(1, 0x00800000, size=(64, 64), dtype=np.uint32)  # subnormal
    w = bits.view(np.float32) * np.where(rng.random((256, 64)) < 0.5, -1, 1).astype(np.float32)
    assert_same(w)


def test_nonfinite_groups_set_status():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    w[1, 70] = np.nan
    w[2, 255] = np.inf
    w[3, 0] = -np.inf
    p, s, st = gpu_quant(w)
    assert st == 1
    pr, sr, _ = oracle.quant_int4_g64(w)
    assert np.array_equal(p, pr)
    assert np.array_equal(np.isnan(s), np.isnan(sr))
    fin = ~np.isnan(sr)
    assert np.array_equal(s[fin].view(np.uint32), sr[fin].view(np.uint32))
    # finite input leaves the flag at 0
    _, _, st2 = gpu_quant(w[0:1])
    assert st2 == 0


def test_zero_rows_is_noop():
    import int4_grouped_expert_amd as coli
    w = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    packed = torch.full((1, 32), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((1, 1), 7.0, device="cuda")
    coli.coli_quant_int4_g64(w, packed, scales)
    torch.cuda.synchronize()
    assert torch.all(packed == 0x5A) and torch.all(scales == 7.0)


def test_unaligned_rows_scalar_path():
    """cols % 4 != 0 rows are not 16-byte aligned: the scalar load path."""
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((9, 131)) * 0.1).astype(np.float32)
    assert_same(w)


def test_deterministic_twice():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((128, 512)) * 0.02).astype(np.float32)
    a = gpu_quant(w)
    b = gpu_quant(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("n,rows,cols,offset", [(5, 96, 320, 0), (3, 33, 200, 1), (12, 256, 6144, 0)])
def test_many_matrices_in_one_launch(n, rows, cols, offset):
    """coli_quant_int4_g64_many: every matrix's bytes and scale bits equal the oracle's
    (and so the single-matrix calls'); one matrix starts 4 bytes past 16-byte
    alignment when offset is set (the element-load path inside the batched launch);
    a non-finite element in one matrix sets the status flag."""
    import int4_grouped_expert_amd as coli
    log(f"quant many n {n} rows {rows} cols {cols} offset {offset}")
    rng = np.random.default_rng(n * 1000 + rows + cols)
    ws = [(rng.standard_normal((rows, cols)) * 0.02 * 2.0 ** rng.integers(-8, 8)).astype(np.float32)
          for _ in range(n)]
    ws[0][1, 3] = np.nan
    G = -(-cols // 64)
    buf = torch.empty(n * rows * cols + 4, dtype=torch.float32, device="cuda")
    wd = []
    for i, w in enumerate(ws):
        base = i * rows * cols + (1 if (offset and i == n - 1) else 0)
        t = buf[base:base + rows * cols].view(rows, cols)
        t.copy_(torch.from_numpy(w))
        wd.append(t)
    packed = [torch.full((rows, G * 32), 0x5A, dtype=torch.uint8, device="cuda")
              for _ in range(n)]
    scales = [torch.full((rows, G), 7.0, dtype=torch.float32, device="cuda") for _ in range(n)]
    ptr = lambda ts: torch.tensor([t.data_ptr() for t in ts], dtype=torch.int64, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    coli.coli_quant_int4_g64_many(ptr(wd), ptr(packed), ptr(scales), n, rows, cols, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 1
    for i, w in enumerate(ws):
        pr, sr, _ = oracle.quant_int4_g64(w)
        assert np.array_equal(packed[i].cpu().numpy(), pr), i
        assert np.array_equal(scales[i].cpu().numpy().view(np.uint32), sr.view(np.uint32)), i
