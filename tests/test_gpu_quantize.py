"""GPU parity of mxfp8_quantize against the CPU oracle: codes and scales
bit-exact, dbias within its summation-depth bound (exact on integers)."""

import numpy as np
import pytest

import mxfp8_block_scaled_quantize_amd as mx
import oracle
import workloads
from gpu_util import bf16_to_f64, log, need_gpu, to_dev, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu

ROW, COL, DB = mx.MXFP8_ROWWISE, mx.MXFP8_COLWISE, mx.MXFP8_DBIAS


def gpu_quantize(bits, flags, ld=None, canary=False):
    """Run mxfp8_quantize on BF16 bits [R, C] (optionally inside a wider ld);
    returns host arrays.  With canary=True every output sits inside a guard
    band of 0xA5 bytes that must come back untouched."""
    torch = need_gpu()
    R, C = bits.shape
    ld = C if ld is None else ld
    src = np.zeros((R, ld), dtype=np.uint16)
    src[:, :C] = bits
    x = to_dev_bf16(src)
    G = 4096 if canary else 0

    def buf(n, dtype=torch.uint8):
        t = torch.full((n + 2 * G,), 0xA5 if dtype == torch.uint8 else 0, dtype=dtype, device="cuda")
        return t, t[G:G + n]

    bufs = {}
    outs = {}
    if flags & ROW:
        bufs["q_row"], outs["q_row"] = buf(R * C)
        bufs["s_row"], outs["s_row"] = buf(R * (C // 32))
    if flags & COL:
        bufs["q_colT"], outs["q_colT"] = buf(R * C)
        bufs["s_colT"], outs["s_colT"] = buf(C * (R // 32))
    if flags & DB:
        bufs["dbias"], outs["dbias"] = buf(C, torch.float32)
    nws = mx.mxfp8_quantize_workspace_bytes(R, C, flags)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device="cuda")
    mx.mxfp8_quantize(x, R, C, ld, flags, outs.get("q_row"), outs.get("s_row"), outs.get("q_colT"),
                      outs.get("s_colT"), outs.get("dbias"), ws if nws else None, nws)
    torch.cuda.synchronize()
    res = {}
    if flags & ROW:
        res["q_row"] = to_host(outs["q_row"]).reshape(R, C)
        res["s_row"] = to_host(outs["s_row"]).reshape(R, C // 32)
    if flags & COL:
        res["q_colT"] = to_host(outs["q_colT"]).reshape(C, R)
        res["s_colT"] = to_host(outs["s_colT"]).reshape(C, R // 32)
    if flags & DB:
        res["dbias"] = to_host(outs["dbias"])
    if canary:
        for name, full in bufs.items():
            h = to_host(full)
            if h.dtype == np.uint8:
                assert np.all(h[:G] == 0xA5) and np.all(h[-G:] == 0xA5), name + " guard band written"
            else:
                assert np.all(h[:G] == 0) and np.all(h[-G:] == 0), name + " guard band written"
    return res


def check_against_oracle(bits, flags, res, label):
    if flags & ROW:
        q, s = oracle.quantize_rowwise(bits)
        assert np.array_equal(res["s_row"], s), label + ": rowwise scales differ"
        bad = np.argwhere(res["q_row"] != q)
        assert bad.size == 0, "%s: %d rowwise codes differ, first %s" % (label, len(bad), bad[:4].tolist())
    if flags & COL:
        qT, sT = oracle.quantize_colwise(bits)
        assert np.array_equal(res["s_colT"], sT), label + ": colwise scales differ"
        bad = np.argwhere(res["q_colT"] != qT)
        assert bad.size == 0, "%s: %d colwise codes differ, first %s" % (label, len(bad), bad[:4].tolist())
    if flags & DB:
        check_dbias(bits, res["dbias"], label)


def dbias_depth(R):
    """Length of the longest fp32 addition chain of the GPU dbias: 8 rows per
    lane, 2 cross-lane steps, 3 pairwise levels across the (up to 8) waves of
    a row tile, then 8 interleaved chains over the row tiles (tiles of at
    least 128 rows) combined pairwise in 3 levels."""
    tiles = (R + 127) // 128
    return 8 + 2 + 3 + (tiles + 7) // 8 + 3


def check_dbias(bits, got, label):
    ref = oracle.dbias(bits).astype(np.float64)
    mag = np.abs(bf16_to_f64(bits)).sum(axis=0)
    d = dbias_depth(bits.shape[0])
    tol = 1.01 * d * 2.0 ** -24 * mag + 2.0 ** -126
    err = np.abs(got.astype(np.float64) - ref)
    # the oracle itself rounds the exact sum once: allow its half ulp too
    tol += np.abs(ref) * 2.0 ** -24
    assert np.all(err <= tol), "%s: dbias off by %g (tol %g)" % (label, err.max(), tol[np.argmax(err - tol)])


# ------------------------------------------------------------------ tests

def test_tiny_config_all_copies():
    data = workloads.tiny()
    for name in ("A", "B"):
        log("tiny %s row+col+dbias" % name)
        res = gpu_quantize(data[name], ROW | COL | DB, canary=True)
        check_against_oracle(data[name], ROW | COL | DB, res, "tiny " + name)


def exhaustive_bf16_blocks():
    """Every finite BF16 value under every scale it can carry: block b of
    anchor exponent field e has first element (e << 7) | 0x7F (the largest
    magnitude of that binade) and then 31 values drawn in order from all BF16
    patterns with exponent field <= e, both signs."""
    blocks = []
    for e in range(0, 255):
        anchor = np.uint16((e << 7) | 0x7F)
        mags = np.arange(0, (e << 7) | 0x80, dtype=np.uint32).astype(np.uint16)
        vals = np.concatenate([mags, mags | 0x8000])
        pad = (-len(vals)) % 31
        vals = np.concatenate([vals, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 31)
        blk = np.empty((vals.shape[0], 32), dtype=np.uint16)
        blk[:, 0] = anchor | (0x8000 if e % 2 else 0)
        blk[:, 1:] = vals
        blocks.append(blk)
    allb = np.concatenate(blocks)
    nb = allb.shape[0]
    per_row = 128
    rows = (nb + per_row - 1) // per_row
    rows = (rows + 31) // 32 * 32
    out = np.zeros((rows * per_row, 32), dtype=np.uint16)
    out[:nb] = allb
    return out.reshape(rows, per_row * 32)


def test_exhaustive_bf16_values_and_scales_rowwise():
    bits = exhaustive_bf16_blocks()
    log("exhaustive rowwise %s" % (bits.shape,))
    res = gpu_quantize(bits, ROW)
    check_against_oracle(bits, ROW, res, "exhaustive rowwise")


def test_exhaustive_bf16_values_and_scales_colwise():
    bits = np.ascontiguousarray(exhaustive_bf16_blocks().T)   # blocks now run down the columns
    log("exhaustive colwise %s" % (bits.shape,))
    res = gpu_quantize(bits, COL)
    check_against_oracle(bits, COL, res, "exhaustive colwise")


@pytest.mark.parametrize("R,C,flags,ld", [
    (32, 32, ROW | COL | DB, None),
    (96, 160, ROW | COL | DB, None),
    (160, 96, ROW | COL, 104),
    (288, 4128, ROW | COL | DB, None),
    (1000, 224, ROW | DB, None),
    (7, 64, ROW, 72),
    (1, 32, ROW | DB, None),
    (4096, 32, COL | DB, None),
])
def test_ragged_shapes_and_strides(R, C, flags, ld):
    bits = workloads.wide_range_bf16((R, C), R * 7 + C, n_maxbf16=0 if flags & DB else 2,
                                     n_subnormal=min(64, R * C // 8),
                                     n_subnormal_blocks=1)
    log("ragged R=%d C=%d flags=%d ld=%s" % (R, C, flags, ld))
    res = gpu_quantize(bits, flags, ld=ld, canary=True)
    check_against_oracle(bits, flags, res, "ragged %dx%d" % (R, C))


def test_special_values():
    rows = []
    rows.append([0.0] * 32)
    rows.append([-0.0] * 32)
    rows.append([1.0] + [-(2.0 ** -20)] * 31)
    rows.append([448.0, 1.0, 500.0] + [0.0] * 29)
    rows.append([2.0 ** -130] * 32)
    rows.append([7.5, 1.0] + [-0.0] * 30)
    x = np.array(rows * 6, dtype=np.float32)[:32]
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    bits[0, 5] = workloads.BF16_MAX_BITS
    bits[1, 7] = 0x8000 | workloads.BF16_MAX_BITS
    bits[2, 9] = 0x0001
    bits[3, 11] = 0x8001
    log("special values")
    res = gpu_quantize(bits, ROW | COL | DB, canary=True)
    check_against_oracle(bits, ROW | COL | DB, res, "special")


def test_dbias_exact_on_integers_and_deterministic():
    rng = np.random.default_rng(5)
    ints = rng.integers(-256, 257, size=(1024, 256))
    bits = (ints.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    log("dbias integers")
    r1 = gpu_quantize(bits, ROW | COL | DB)
    r2 = gpu_quantize(bits, ROW | COL | DB)
    assert np.array_equal(r1["dbias"].astype(np.int64), ints.sum(axis=0))
    assert np.array_equal(r1["dbias"].view(np.uint32), r2["dbias"].view(np.uint32))
    heavy = workloads.student_t_bf16((2048, 384), 3)
    a = gpu_quantize(heavy, ROW | DB)
    b = gpu_quantize(heavy, ROW | DB)
    assert np.array_equal(a["dbias"].view(np.uint32), b["dbias"].view(np.uint32))
    check_dbias(heavy, a["dbias"], "heavy")


def test_empty_inputs():
    torch = need_gpu()
    db = torch.full((64,), 7.0, device="cuda")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    log("empty rows with dbias")
    mx.mxfp8_quantize(x, 0, 64, 64, ROW | DB, None, None, None, None, db, None, 0)
    torch.cuda.synchronize()
    assert torch.all(db == 0).item()
    mx.mxfp8_quantize(None, 0, 64, 64, ROW, None, None)
    mx.mxfp8_quantize(None, 64, 0, 0, ROW | COL, None, None, None, None)


# ------------------------------------------------- full workload sizes

@pytest.mark.slow
def test_full_dense_rowwise():
    data = workloads.dense_linear()
    for name in ("X", "W"):
        log("dense %s rowwise %s" % (name, data[name].shape))
        res = gpu_quantize(data[name], ROW)
        check_against_oracle(data[name], ROW, res, "dense " + name)


@pytest.mark.slow
def test_full_backward_row_col_dbias():
    data = workloads.backward()
    log("backward dY row+col+dbias")
    res = gpu_quantize(data["dY"], ROW | COL | DB)
    check_against_oracle(data["dY"], ROW | COL | DB, res, "backward dY")
    log("backward X col")
    res = gpu_quantize(data["X"], COL)
    check_against_oracle(data["X"], COL, res, "backward X")


@pytest.mark.slow
def test_full_stress_row_col():
    data = workloads.stress()
    log("stress A row+col %s" % (data["A"].shape,))
    res = gpu_quantize(data["A"], ROW | COL)
    check_against_oracle(data["A"], ROW | COL, res, "stress A")
    del res
    log("stress B row")
    res = gpu_quantize(data["B"], ROW)
    check_against_oracle(data["B"], ROW, res, "stress B")


@pytest.mark.slow
def test_full_moe_rowwise():
    """The MoE workload's operands at full size (X [16384 x 4096], the eight
    experts' W as one [114688 x 4096] tensor), byte scales, bit-exact."""
    data = workloads.moe()
    G, N, K = data["W"].shape
    for name, bits in (("X", data["X"]), ("W", data["W"].reshape(G * N, K))):
        log("moe %s rowwise %s" % (name, bits.shape))
        res = gpu_quantize(bits, ROW)
        check_against_oracle(bits, ROW, res, "moe " + name)
        del res
