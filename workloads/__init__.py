"""Seeded synthetic inputs for the MXFP8 quantize + block-scaled GEMM path.

This module only draws random numbers and lays them out as BF16 bit patterns
(``numpy.uint16``).  It holds none of the method's arithmetic: no amax, no
scale, no FP8 cast, no GEMM.  Both the CPU oracle (through the tests) and the
GPU path consume exactly the bytes produced here.

Every generator is deterministic in its seed (numpy ``default_rng`` / PCG64).
Floating samples are drawn in float32 and rounded to BF16 with
round-to-nearest-even on the bit pattern.

Workload recipes (shapes and value distributions of the LLM linear-layer and
MoE workloads the MXFP8 quantize and GEMM pages discuss):

* ``tiny``      A, B BF16[256x256] ~ N(0,1), seeds 0 and 1.
* ``dense``     X BF16[8192x4096] ~ N(0,1) (seed 0), W BF16[14336x4096] ~
                N(0,0.02) (seed 1); square A[8192x8192] ~ N(0,1) (seed 2),
                B[8192x8192] ~ N(0,0.02) (seed 3).
* ``backward``  dY BF16[16384x4096] = 0.1 * Student-t(df=3) (seed 0) with 1%
                of the aligned 32x32 tiles set to zero; X BF16[16384x4096] ~
                N(0,1) (seed 1).
* ``moe``       X BF16[16384x4096] ~ N(0,1) (seed 0); W BF16[8][14336x4096] ~
                N(0,0.02) (seed 1); group sizes 32 * Multinomial(512, 1/8 each)
                (seed 2) turned into int32 offsets[9].
* ``preact``    GELU inputs: N(0,1) blocks scaled by 2^u, u in [-12, 2], with
                1/16 of the blocks uniform in [-10, -3] and 1/16 uniform in
                [3, 40], clipped below at -12 (where GELU stays inside fp32's
                normal range); parity cases only.
* ``stress``    A BF16[32768x8192]: N(0,1) with every rowwise 32-block scaled
                by 2^u, u uniform integer in [-40, 40] (seed 0), plus 64 +-max
                BF16 values, 4096 random +-subnormals and 16 all-subnormal
                blocks; B BF16[8192x8192] by the same recipe without the max
                BF16 values (seed 1).
"""

from __future__ import annotations

import numpy as np

BF16_MAX_BITS = 0x7F7F  # largest finite BF16 magnitude, about 3.39e38


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even) -> uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    lsb += 0x7FFF
    lsb += u          # finite floats stay below 2^32 (largest is 0xFF7FFFFF + 0x8000)
    lsb >>= 16
    return lsb.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 (exact: BF16 is the top half of binary32)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def normal_bf16(shape, seed: int, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(_normal_f32(rng, shape, std))


def student_t_bf16(shape, seed: int, df: float = 3.0, scale: float = 0.1,
                   zero_tile_frac: float = 0.01, tile: int = 32) -> np.ndarray:
    """Heavy-tailed values with a fraction of aligned tile x tile squares zeroed.

    Zeroing aligned 32x32 squares zeroes the same fraction of 32-blocks in
    both the rowwise and the columnwise direction.
    """
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(df, size=shape) * scale).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    r, c = shape
    tr, tc = r // tile, c // tile
    ntiles = tr * tc
    nzero = int(round(zero_tile_frac * ntiles))
    if nzero:
        pick = rng.choice(ntiles, size=nzero, replace=False)
        b3 = bits.reshape(tr, tile, tc, tile)
        b3[pick // tc, :, pick % tc, :] = 0
    return bits


def wide_range_bf16(shape, seed: int, u_lo: int = -40, u_hi: int = 40,
                    n_maxbf16: int = 64, n_subnormal: int = 4096,
                    n_subnormal_blocks: int = 16) -> np.ndarray:
    """N(0,1) with each rowwise 32-block scaled by 2^u, plus extreme values."""
    rng = np.random.default_rng(seed)
    r, c = shape
    x = _normal_f32(rng, shape, 1.0)
    u = rng.integers(u_lo, u_hi + 1, size=(r, c // 32))
    x.reshape(r, c // 32, 32)[...] *= np.ldexp(np.float32(1.0), u)[..., None].astype(np.float32)
    bits = f32_to_bf16_bits(x)
    flat = bits.reshape(-1)
    n = flat.size
    if n_maxbf16:
        pos = rng.choice(n, size=n_maxbf16, replace=False)
        sign = rng.integers(0, 2, size=n_maxbf16).astype(np.uint16) << 15
        flat[pos] = sign | BF16_MAX_BITS
    if n_subnormal:
        pos = rng.choice(n, size=n_subnormal, replace=False)
        sign = rng.integers(0, 2, size=n_subnormal).astype(np.uint16) << 15
        mant = rng.integers(1, 128, size=n_subnormal).astype(np.uint16)
        flat[pos] = sign | mant
    if n_subnormal_blocks:
        nblk = r * (c // 32)
        blk = rng.choice(nblk, size=n_subnormal_blocks, replace=False)
        sign = rng.integers(0, 2, size=(n_subnormal_blocks, 32)).astype(np.uint16) << 15
        mant = rng.integers(1, 128, size=(n_subnormal_blocks, 32)).astype(np.uint16)
        flat.reshape(nblk, 32)[blk] = sign | mant
    return bits


def preact_bf16(shape, seed: int, u_lo: int = -12, u_hi: int = 2, tail_frac: float = 1.0 / 16,
                floor: float = -12.0) -> np.ndarray:
    """Pre-activation-like values for GELU: N(0,1) with each rowwise 32-block
    scaled by 2^u (u uniform integer in [u_lo, u_hi]); a fraction tail_frac
    of the blocks is replaced by uniform values in [-10, -3] (GELU's negative
    tail) and as many by uniform values in [3, 40] (where GELU is nearly the
    identity); everything is clipped below at `floor`."""
    rng = np.random.default_rng(seed)
    r, c = shape
    x = _normal_f32(rng, shape, 1.0)
    xb = x.reshape(r * (c // 32), 32)
    u = rng.integers(u_lo, u_hi + 1, size=r * (c // 32))
    xb *= np.ldexp(np.float32(1.0), u)[:, None].astype(np.float32)
    nblk = xb.shape[0]
    k = int(round(tail_frac * nblk))
    if k:
        pick = rng.choice(nblk, size=2 * k, replace=False)
        xb[pick[:k]] = rng.uniform(-10.0, -3.0, size=(k, 32)).astype(np.float32)
        xb[pick[k:]] = rng.uniform(3.0, 40.0, size=(k, 32)).astype(np.float32)
    np.maximum(x, np.float32(floor), out=x)
    return f32_to_bf16_bits(x)


def moe_offsets(total_tokens: int, groups: int, seed: int, align: int = 32) -> np.ndarray:
    """int32 offsets[G+1] from align * Multinomial(total/align, uniform)."""
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(total_tokens // align, [1.0 / groups] * groups) * align
    off = np.zeros(groups + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    return off.astype(np.int32)


def offsets_from_counts(counts) -> np.ndarray:
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(counts, dtype=np.int64))
    return off.astype(np.int32)


# A fixed grouping with empty experts (the uniform multinomial practically never
# leaves one empty): 16384 tokens over 8 experts.
MOE_EMPTY_COUNTS = (0, 8192, 0, 0, 4096, 4096, 0, 0)


# ---------------------------------------------------------------- workloads

def tiny():
    return {"A": normal_bf16((256, 256), 0), "B": normal_bf16((256, 256), 1)}


def dense_linear():
    return {"X": normal_bf16((8192, 4096), 0),
            "W": normal_bf16((14336, 4096), 1, std=0.02)}


def dense_square():
    return {"A": normal_bf16((8192, 8192), 2),
            "B": normal_bf16((8192, 8192), 3, std=0.02)}


def mlp():
    """Squared-ReLU MLP step: tokens 8192, d_model 4096, d_ff 14336.  X and W1
    are the dense linear layer's tensors; W2 [4096 x 14336] ~ N(0, 0.02);
    dY [8192 x 4096] ~ N(0, 1)."""
    d = dense_linear()
    return {"X": d["X"], "W1": d["W"], "W2": normal_bf16((4096, 14336), 5, std=0.02),
            "dY": normal_bf16((8192, 4096), 6)}


def mlp_hidden():
    """Stand-ins for the MLP step's BF16 GEMM outputs at full size: H = X W1^T
    and dA = dY W2 are sums of 4096 (14336) products of N(0,1) and
    N(0,0.02) values, i.e. N(0, 1.28^2) and N(0, 2.39^2)."""
    return {"H": normal_bf16((8192, 14336), 7, std=1.28),
            "dA": normal_bf16((8192, 14336), 8, std=2.39)}


def backward():
    return {"dY": student_t_bf16((16384, 4096), 0),
            "X": normal_bf16((16384, 4096), 1)}


def moe(empty_groups: bool = False):
    x = normal_bf16((16384, 4096), 0)
    w = normal_bf16((8, 14336, 4096), 1, std=0.02)
    off = offsets_from_counts(MOE_EMPTY_COUNTS) if empty_groups else moe_offsets(16384, 8, 2)
    return {"X": x, "W": w, "offsets": off}


def moe_fc2():
    """The MoE block's second projection: per expert W2 [4096][7168] (d_model
    x the SwiGLU output width of the first projection), N(0, 0.02)."""
    return {"W2": normal_bf16((8, 4096, 7168), 5, std=0.02)}


def stress():
    return {"A": wide_range_bf16((32768, 8192), 0),
            "B": wide_range_bf16((8192, 8192), 1, n_maxbf16=0)}
