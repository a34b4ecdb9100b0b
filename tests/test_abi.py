"""C-ABI checks that need no GPU: the library loads, exports every function
include/mxfp8.h declares, and rejects invalid arguments on the host before
anything is launched (these calls never reach the HIP runtime)."""

import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_quantize_amd as mx
from mxfp8_block_scaled_quantize_amd import build as mxbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")

OK, NULL, SHAPE, MISALIGNED, FLAGS, WORKSPACE, HIP, LIMIT = range(8)
ROW, COL, DB = 1, 2, 4
A16 = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mx.LIB_PATH):
        mxbuild.build()
    return mx.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("mxfp8_quantize", "mxfp8_pack_scales", "mxfp8_gemm", "mxfp8_grouped_gemm"):
        assert n in names


def test_header_constants_match_the_binding():
    """Every flag, size constant and status value the header defines has the
    same value in the Python binding (and the binding defines no such constant
    the header lacks)."""
    import re
    text = open(HEADER).read()
    flags = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (MXFP8_[A-Z_]+) (\d+)u", text)}
    assert len(flags) == 14, flags
    for name, value in flags.items():
        assert getattr(mx, name) == value, name
    binding = {n for n in dir(mx) if re.fullmatch(r"MXFP8_[A-Z_]+", n) and isinstance(getattr(mx, n), int)}
    assert binding == set(flags), binding ^ set(flags)
    status = {m.group(1): int(m.group(2)) for m in re.finditer(r"(MXFP8_(?:OK|ERR_[A-Z]+)) = (\d+)", text)}
    assert {v: k for k, v in status.items()} == mx.STATUS_NAMES


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert names and set(names) == set(mx.EXPORTED)
    for n in names:
        assert hasattr(L, n), n
    so = ctypes.CDLL(mx.LIB_PATH)
    for n in names:
        getattr(so, n)


def test_status_strings(L):
    for code, name in mx.STATUS_NAMES.items():
        assert mx.mxfp8_status_string(code).startswith(name)
    assert "unknown" in mx.mxfp8_status_string(99)


def test_workspace_and_packed_sizes(L):
    assert L.mxfp8_quantize_workspace_bytes(300, 256, ROW | DB) == 3 * 256 * 4
    assert L.mxfp8_quantize_workspace_bytes(300, 256, ROW) == 0
    assert L.mxfp8_quantize_workspace_bytes(0, 256, ROW | DB) == 0
    assert L.mxfp8_packed_scale_bytes(96, 512) == 4 * 96 * 4
    assert L.mxfp8_packed_scale_bytes(0, 512) == 0


def q(L, x=A16, rows=64, cols=64, ld=64, flags=ROW, qr=A16, sr=A16, qc=A16, sc=A16, db=A16, ws=A16, wsb=1 << 20):
    return L.mxfp8_quantize(x, rows, cols, ld, flags, qr, sr, qc, sc, db, ws, wsb, None)


def test_quantize_validation(L):
    assert q(L, flags=0) == FLAGS
    assert q(L, flags=8 | ROW) == FLAGS
    assert q(L, flags=DB) == FLAGS
    assert q(L, cols=48, ld=48) == SHAPE
    assert q(L, rows=-1) == SHAPE
    assert q(L, ld=32) == SHAPE
    assert q(L, rows=48, flags=COL) == SHAPE
    assert q(L, x=None) == NULL
    assert q(L, qr=None) == NULL
    assert q(L, sr=None) == NULL
    assert q(L, flags=COL, qc=None) == NULL
    assert q(L, flags=ROW | DB, db=None) == NULL
    assert q(L, x=A16 + 2) == MISALIGNED
    assert q(L, ld=68) == MISALIGNED
    assert q(L, qr=A16 + 8) == MISALIGNED
    assert q(L, flags=COL, qc=A16 + 4) == MISALIGNED
    assert q(L, flags=ROW | DB, db=A16 + 2) == MISALIGNED
    assert q(L, flags=ROW | DB, ws=None) == WORKSPACE
    assert q(L, flags=ROW | DB, wsb=64 * 4 - 1) == WORKSPACE
    assert q(L, flags=ROW | DB, ws=A16 + 4) == MISALIGNED
    # empty problems are no-ops that launch nothing
    assert q(L, rows=0, x=None, qr=None, sr=None) == OK
    assert q(L, cols=0, ld=0, x=None, qr=None, sr=None) == OK


def qx(L, x=A16, rows=128, cols=128, ld=128, flags=ROW, qr=A16, sr=A16, qc=A16, sc=A16, db=A16, am=A16,
       noop=None, act=A16, ws=A16, wsb=1 << 20):
    return L.mxfp8_quantize_ex(x, rows, cols, ld, flags, qr, sr, qc, sc, db, am, noop, act, ws, wsb, None)


def test_quantize_ex_validation(L):
    AMAX, PACKED = mx.MXFP8_AMAX, mx.MXFP8_PACKED_SCALES
    ACT, DACT = mx.MXFP8_ACT_SQRELU, mx.MXFP8_DACT_SQRELU
    GELU, DGELU = mx.MXFP8_ACT_GELU, mx.MXFP8_DACT_GELU
    assert qx(L, flags=512 | ROW) == FLAGS
    assert qx(L, flags=ROW | ACT | DACT) == FLAGS              # one activation at a time
    for a, b in ((ACT, GELU), (DACT, GELU), (ACT, DGELU), (GELU, DGELU), (DACT, DGELU)):
        assert qx(L, flags=ROW | a | b, act=A16) == FLAGS
    assert qx(L, flags=ROW | DGELU, act=None) == NULL
    assert qx(L, flags=COL | DGELU, act=A16 + 2) == MISALIGNED
    assert qx(L, flags=ROW | GELU, act=None, x=A16 + 2) == MISALIGNED   # act_in unused for the forward
    assert qx(L, flags=ROW | GELU | DB, act=None, ws=None) == WORKSPACE
    assert qx(L, flags=ROW | DGELU | DB, act=A16, ws=None) == WORKSPACE
    assert qx(L, flags=ACT) == FLAGS
    assert qx(L, flags=ROW | DACT, act=None) == NULL
    assert qx(L, flags=COL | DACT, act=A16 + 2) == MISALIGNED
    assert qx(L, flags=ROW | ACT, act=None, x=A16 + 2) == MISALIGNED   # act_in unused without DACT
    assert qx(L, flags=ROW | DACT | DB, act=A16, ws=None) == WORKSPACE  # stops before launching
    assert qx(L, flags=AMAX) == FLAGS                         # no copy requested
    assert qx(L, flags=ROW | AMAX, am=None) == NULL
    assert qx(L, flags=ROW | AMAX, am=A16 + 2) == MISALIGNED
    assert qx(L, noop=A16 + 2) == MISALIGNED
    assert qx(L, flags=ROW | PACKED, cols=96, ld=96) == SHAPE      # rowwise packed: cols % 128
    assert qx(L, flags=COL | PACKED, rows=96) == SHAPE             # columnwise packed: rows % 128
    # (the cases below stop at the last check, the workspace, so nothing is launched)
    assert qx(L, flags=ROW | PACKED | DB, rows=96, ws=None) == WORKSPACE   # rows free for the rowwise copy
    assert qx(L, flags=ROW | PACKED, sr=A16 + 2) == MISALIGNED
    assert qx(L, flags=COL | PACKED, sc=A16 + 2) == MISALIGNED
    assert qx(L, flags=ROW | DB, sr=A16 + 2, ws=None) == WORKSPACE   # byte scales need no alignment
    # the plain entry point keeps rejecting the extra flags
    assert q(L, flags=ROW | AMAX) == FLAGS
    assert q(L, flags=ROW | PACKED) == FLAGS
    assert q(L, flags=ROW | ACT) == FLAGS


def test_quantize_grid_limit(L):
    assert q(L, rows=1 << 36, cols=1 << 20, ld=1 << 20) == LIMIT
    assert q(L, rows=1 << 41, cols=64, ld=64) == LIMIT
    # Grids are counted in work-items (a 32-bit field of the dispatch packet).
    # Flat rowwise kernel, 4096 elements per 256-work-item workgroup: 2^36
    # elements need exactly 2^32 work-items, one too many.
    assert q(L, rows=1 << 22, cols=1 << 14, ld=1 << 14) == LIMIT
    # columnwise tiles (128 x 128, 256 work-items): 2^25 tiles need 2^33
    assert q(L, rows=1 << 20, cols=1 << 19, ld=1 << 19, flags=COL) == LIMIT
    # row+col tiles (256 x 128, 512 work-items): 2^23 tiles need 2^32, one
    # tile fewer fits (the missing workspace is then the first error found)
    assert q(L, rows=256 * (1 << 23), cols=128, ld=128, flags=ROW | COL | DB, ws=None) == LIMIT
    assert q(L, rows=256 * ((1 << 23) - 1), cols=128, ld=128, flags=ROW | COL | DB, ws=None) == WORKSPACE
    # the dbias reduce (256 work-items per 32 columns) is the larger grid here
    assert q(L, rows=32, cols=1 << 29, ld=1 << 29, flags=ROW | COL | DB, ws=None) == LIMIT
    assert q(L, rows=32, cols=(1 << 29) - 32, ld=(1 << 29) - 32, flags=ROW | COL | DB, ws=None) == WORKSPACE


def test_gemm_and_pack_grid_limits(L):
    # 256 x 256 tiles of 256 work-items: 2^24 tiles need 2^32 work-items
    assert L.mxfp8_gemm(A16, A16, A16, A16, A16, 1 << 20, 1 << 20, 1 << 20, 128, None) == LIMIT
    # tile counts whose product would overflow int64 if formed naively
    assert L.mxfp8_gemm(A16, A16, A16, A16, A16, 1 << 40, 1 << 40, 1 << 40, 128, None) == LIMIT
    # grouped: the row tiles include one spare per group
    assert L.mxfp8_grouped_gemm(A16, A16, A16, A16, A16, 1, A16, 1 << 20, 1 << 20, 1 << 20, 128, None) == LIMIT
    # packing: 64 x 64 word tiles of 256 work-items
    assert L.mxfp8_pack_scales(A16, 1 << 30, 1 << 20, 1 << 15, A16, None) == LIMIT


def test_pack_validation(L):
    P = L.mxfp8_pack_scales
    assert P(A16, 64, 100, 4, A16, None) == SHAPE
    assert P(A16, 64, 256, 4, A16, None) == SHAPE          # ld_s < k/32
    assert P(A16, -1, 256, 8, A16, None) == SHAPE
    assert P(None, 64, 256, 8, A16, None) == NULL
    assert P(A16, 64, 256, 8, None, None) == NULL
    assert P(A16 + 1, 64, 256, 8, A16, None) == MISALIGNED
    assert P(A16, 64, 256, 10, A16, None) == MISALIGNED
    assert P(A16, 0, 256, 8, None, None) == OK


def test_gemm_validation(L):
    G = L.mxfp8_gemm
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 100, None) == SHAPE      # K % 128
    assert G(A16, A16, A16, A16, A16, 48, 64, 48, 128, None) == SHAPE      # N % 32
    assert G(A16, A16, A16, A16, A16, 32, 64, 64, 128, None) == SHAPE      # ldc < N
    assert G(A16, A16, A16, A16, A16, 64, -1, 64, 128, None) == SHAPE
    assert G(None, A16, A16, A16, A16, 64, 64, 64, 128, None) == NULL
    assert G(A16, None, A16, A16, A16, 64, 64, 64, 128, None) == NULL
    assert G(A16, A16, A16, A16, None, 64, 64, 64, 128, None) == NULL
    assert G(A16 + 8, A16, A16, A16, A16, 64, 64, 64, 128, None) == MISALIGNED
    assert G(A16, A16 + 2, A16, A16, A16, 64, 64, 64, 128, None) == MISALIGNED
    assert G(A16, A16, A16, A16, A16 + 2, 64, 64, 64, 128, None) == MISALIGNED
    assert G(A16, A16, A16, A16, A16, 68, 64, 64, 128, None) == MISALIGNED  # ldc % 8
    assert G(None, None, None, None, None, 64, 0, 64, 128, None) == OK
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, (1 << 22) + 128, None) == LIMIT


def test_grouped_gemm_validation(L):
    G = L.mxfp8_grouped_gemm
    assert G(A16, A16, A16, A16, A16, 0, A16, 64, 64, 64, 128, None) == SHAPE
    assert G(A16, A16, A16, A16, A16, 70000, A16, 64, 64, 64, 128, None) == SHAPE
    assert G(A16, A16, A16, A16, None, 4, A16, 64, 64, 64, 128, None) == NULL
    assert G(A16, A16, A16, A16, A16 + 2, 4, A16, 64, 64, 64, 128, None) == MISALIGNED
    assert G(A16, A16, A16, A16, None, 4, None, 64, 0, 64, 128, None) == OK


def test_gemm_ex_flags(L):
    G = L.mxfp8_gemm_ex
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 128, 16, None) == FLAGS
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 128, 3, None) == FLAGS   # accumulate and relu^2 together
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 128, 9, None) == FLAGS   # accumulate and SwiGLU
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 128, 12, None) == FLAGS  # GELU and SwiGLU
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 100, 8, None) == SHAPE   # SwiGLU alone passes the flag check
    assert G(A16, A16, A16, A16, A16, (1 << 27) + 32, 64, (1 << 27) + 32, 128, 8, None) == LIMIT
    assert G(None, None, None, None, None, 64, 0, 64, 128, 8, None) == OK
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 128, 5, None) == FLAGS   # accumulate and GELU
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 128, 6, None) == FLAGS   # two epilogues
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 100, 4, None) == SHAPE   # GELU alone passes the flag check
    assert G(None, None, None, None, None, 64, 0, 64, 128, 4, None) == OK
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 100, 2, None) == SHAPE
    assert G(A16, A16, A16, A16, A16, 64, 64, 64, 100, 1, None) == SHAPE   # the dense checks still apply
    assert G(None, None, None, None, None, 64, 0, 64, 128, 1, None) == OK
    GG = L.mxfp8_grouped_gemm_ex
    assert GG(A16, A16, A16, A16, A16, 4, A16, 64, 64, 64, 128, 16, None) == FLAGS
    assert GG(A16, A16, A16, A16, A16, 4, A16, (1 << 27) + 32, 64, (1 << 27) + 32, 128, 8, None) == LIMIT
    assert GG(A16, A16, A16, A16, A16, 4, A16, 64, 64, 64, 128, 3, None) == FLAGS
    assert GG(A16, A16, A16, A16, A16, 4, A16, 64, 64, 64, 128, 6, None) == FLAGS
    assert GG(A16, A16, A16, A16, None, 4, None, 64, 0, 64, 128, 4, None) == OK
    assert GG(A16, A16, A16, A16, None, 4, None, 64, 0, 64, 128, 2, None) == OK
    assert GG(A16, A16, A16, A16, A16, 0, A16, 64, 64, 64, 128, 1, None) == SHAPE
    assert GG(A16, A16, A16, A16, None, 4, None, 64, 0, 64, 128, 1, None) == OK


def test_gemm_bias_validation(L):
    """The bias entry points apply the _ex rules, require a 16-byte aligned
    bias pointer, and reject accumulate (the bias belongs to a fresh output)."""
    B = L.mxfp8_gemm_bias
    assert B(A16, A16, A16, A16, None, A16, 64, 64, 64, 128, 0, None) == NULL
    assert B(A16, A16, A16, A16, A16 + 2, A16, 64, 64, 64, 128, 0, None) == MISALIGNED
    assert B(A16, A16, A16, A16, A16, A16, 64, 64, 64, 128, 1, None) == FLAGS        # accumulate
    assert B(A16, A16, A16, A16, A16, A16, 64, 64, 64, 128, 16, None) == FLAGS
    assert B(A16, A16, A16, A16, A16, A16, 64, 64, 64, 100, 4, None) == SHAPE         # K % 128
    assert B(A16, A16, A16, A16, None, A16, 64, 0, 64, 128, 0, None) == OK           # empty: nothing read
    assert B(A16, A16, A16, A16, A16, A16, (1 << 27) + 32, 64, (1 << 27) + 32, 128, 8, None) == LIMIT
    GB = L.mxfp8_grouped_gemm_bias
    assert GB(A16, A16, A16, A16, A16, 0, A16, A16, 64, 64, 64, 128, 0, None) == SHAPE
    assert GB(A16, A16, A16, A16, A16, 0, A16, A16, 64, 64, 64, 128, 16, None) == FLAGS
    assert GB(A16, A16, A16, A16, A16, 4, None, A16, 64, 64, 64, 128, 0, None) == NULL
    assert GB(A16, A16, A16, A16, A16, 4, A16 + 8, A16, 64, 64, 64, 128, 2, None) == MISALIGNED
    assert GB(A16, A16, A16, A16, A16, 4, A16, A16, 64, 64, 64, 128, 1, None) == FLAGS
    assert GB(A16, A16, A16, A16, None, 4, A16, A16, 64, 64, 64, 128, 0, None) == NULL  # offsets
    assert GB(A16, A16, A16, A16, None, 4, None, A16, 64, 0, 64, 128, 0, None) == OK


def test_gemm_mxfp8_out_validation(L):
    """The MXFP8-output GEMMs: the _ex rules with a byte-element output (row
    stride a multiple of 16 bytes), whole packed scale words (N % 128), a
    packed-scale pointer, an optional bias, and no accumulate."""
    X = L.mxfp8_gemm_mxfp8_out
    assert X(A16, A16, A16, A16, None, A16, 128, A16, 64, 128, 128, 1, None) == FLAGS      # accumulate
    assert X(A16, A16, A16, A16, None, A16, 128, A16, 64, 128, 128, 16, None) == FLAGS
    assert X(A16, A16, A16, A16, None, A16, 96, A16, 64, 96, 128, 0, None) == SHAPE       # N % 128
    assert X(A16, A16, A16, A16, None, A16, 64, A16, 64, 128, 128, 0, None) == SHAPE      # ldq < N
    assert X(A16, A16, A16, A16, None, None, 128, A16, 64, 128, 128, 0, None) == NULL     # codes
    assert X(A16, A16, A16, A16, None, A16, 128, None, 64, 128, 128, 0, None) == NULL     # packed scales
    assert X(A16, A16, A16, A16, None, A16, 136, A16, 64, 128, 128, 0, None) == MISALIGNED   # ldq % 16
    assert X(A16, A16, A16, A16, None, A16 + 8, 128, A16, 64, 128, 128, 0, None) == MISALIGNED
    assert X(A16, A16, A16, A16, None, A16, 128, A16 + 2, 64, 128, 128, 0, None) == MISALIGNED
    assert X(A16, A16, A16, A16, A16 + 2, A16, 128, A16, 64, 128, 128, 0, None) == MISALIGNED   # bias
    assert X(A16, A16, A16, A16, None, None, 128, None, 0, 128, 128, 0, None) == OK       # empty
    assert X(A16, A16, A16, A16, None, A16, (1 << 27) + 128, A16, 64, (1 << 27) + 128, 128, 8, None) == LIMIT
    XG = L.mxfp8_grouped_gemm_mxfp8_out
    assert XG(A16, A16, A16, A16, A16, 0, None, A16, 128, A16, 64, 128, 128, 0, None) == SHAPE
    assert XG(A16, A16, A16, A16, A16, 4, None, A16, 128, A16, 64, 128, 128, 1, None) == FLAGS
    assert XG(A16, A16, A16, A16, None, 4, None, A16, 128, A16, 64, 128, 128, 0, None) == NULL   # offsets
    assert XG(A16, A16, A16, A16, A16, 4, None, A16, 128, None, 64, 128, 128, 0, None) == NULL
    assert XG(A16, A16, A16, A16, A16, 4, None, A16, 160, A16, 64, 160, 128, 0, None) == SHAPE   # N % 128
    assert XG(A16, A16, A16, A16, None, 4, None, None, 128, None, 0, 128, 128, 0, None) == OK


def test_binding_raises_on_error(L):
    with pytest.raises(mx.MXFP8Error) as ei:
        mx.mxfp8_quantize(A16, 64, 48, 64, ROW, A16, A16, stream=0)
    assert ei.value.status == SHAPE and "SHAPE" in str(ei.value)


def test_noalloc_quantize_validation(L):
    """The allocation-free quantize applies mxfp8_quantize_ex's rules, then
    rejects dbias requests whose partial sums exceed the static scratch
    (MXFP8_ERR_WORKSPACE), all on the host before anything is launched."""
    def qn(x=A16, rows=128, cols=128, ld=128, flags=ROW, db=A16):
        return L.mxfp8_quantize_ex_noalloc(x, rows, cols, ld, flags, A16, A16, A16, A16, db, A16, None, A16, None)
    assert qn(flags=0) == FLAGS
    assert qn(cols=48, ld=48) == SHAPE
    assert qn(x=None) == NULL
    assert qn(flags=ROW | DB, db=None) == NULL
    assert qn(x=A16 + 2) == MISALIGNED
    limit = mx.MXFP8_NOALLOC_SCRATCH_BYTES
    # partial sums of 1024 row tiles x 2048 columns = 8 MiB fit; one more tile does not
    assert L.mxfp8_quantize_workspace_bytes(1024 * 128, 2048, ROW | DB) == limit
    assert L.mxfp8_quantize_workspace_bytes(1025 * 128, 2048, ROW | DB) > limit
    assert qn(rows=1025 * 128, cols=2048, ld=2048, flags=ROW | DB) == WORKSPACE
    assert qn(rows=1025 * 128, cols=2048, ld=2048, flags=ROW | COL | DB) == WORKSPACE


def test_calibration_library_is_separate(L):
    """The benchmark's register-only MFMA kernel lives in its own library, so
    the product library exports exactly what include/mxfp8.h declares."""
    from mxfp8_block_scaled_quantize_amd.build import CALIB_PATH
    cal = ctypes.CDLL(CALIB_PATH)
    cal.mxfp8_calib_mfma_ceiling
    assert cal.mxfp8_calib_code_words() == 4096
    assert not hasattr(ctypes.CDLL(mx.LIB_PATH), "mxfp8_calib_mfma_ceiling")


def test_header_is_plain_c_and_links(tmp_path):
    """include/mxfp8.h compiles as C99 with warnings as errors, and a C program
    linked against libmxfp8.so calls it without Python: status strings, sizes
    and host-side validation (nothing reaches the GPU)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    if not os.path.exists(mx.LIB_PATH):
        mxbuild.build()
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "mxfp8.h"
int main(void) {
    void *p = (void *)0x10000;   /* never dereferenced: every call below fails validation */
    if (strncmp(mxfp8_status_string(MXFP8_ERR_SHAPE), "MXFP8_ERR_SHAPE", 15) != 0) return 1;
    if (mxfp8_packed_scale_bytes(96, 512) != 4 * 96 * 4) return 2;
    if (mxfp8_quantize(p, 64, 48, 64, MXFP8_ROWWISE, p, p, NULL, NULL, NULL, NULL, 0, NULL) != MXFP8_ERR_SHAPE)
        return 3;
    if (mxfp8_gemm_ex(p, p, p, p, p, 64, 64, 64, 128, MXFP8_GEMM_ACCUMULATE | MXFP8_GEMM_GELU, NULL)
        != MXFP8_ERR_FLAGS) return 4;
    if (mxfp8_gemm_mxfp8_out(p, p, p, p, NULL, p, 96, p, 64, 96, 128, 0, NULL) != MXFP8_ERR_SHAPE) return 5;
    if (mxfp8_grouped_gemm(p, p, p, p, p, 0, p, 64, 64, 64, 128, NULL) != MXFP8_ERR_SHAPE) return 6;
    puts("c abi ok");
    return 0;
}
''')
    exe = tmp_path / "abi"
    libdir = os.path.dirname(mx.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-l:libmxfp8.so", "-Wl,-rpath," + libdir],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c abi ok" in r.stdout, (r.returncode, r.stdout, r.stderr)
