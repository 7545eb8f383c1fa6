"""Oracle for the NF4 storage format with double-quantised absmax (plain numpy, CPU).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the product path.

What the pages fix, and what this module reads into the gaps
------------------------------------------------------------
"Can You Fine-Tune a 27B Model on a Laptop? (I Did the Math)", transcript @2:19-2:29: the
base is stored in a 4-bit format built for normally distributed weights, so that the
quantisation levels sit where the values are, and the per-block constants of that first
pass are themselves quantised by a second pass.  "An 8B Fine-Tune Now Fits in 4 GB of
VRAM" names the format (NF4) and links QLoRA (arXiv 2305.14314), whose construction the
codebook below follows.  The pages print no constants, so these are readings:

* codebook: 16 ascending levels, 7 negative, an exact zero at index 7, 8 positive, equal
  to standard-normal quantiles at evenly spaced probabilities between P_MAX and 1/2,
  normalised so the end levels are exactly -1 and +1;
* first pass: blocks of 64 consecutive row-major elements of W[out][in], each scaled by its
  absolute maximum c_b and given the code of the nearest level (ties to the lower level);
* second pass: the c_b minus their mean mu, in groups of 256 blocks, each group scaled by
  its absolute maximum s2 (fp32) and rounded to a symmetric linear int8 code v/127;
* packing: byte j holds element 2j in the high nibble and element 2j+1 in the low nibble.

Every fp32 operation below is a single IEEE-rounded numpy float32 operation (numpy never
fuses a multiply and an add), so each line states one rounding step.
"""

from __future__ import annotations

import statistics

import numpy as np

BLOCK = 64            # weights per first-level absmax block
GROUP = 256           # first-level blocks per second-level scale
P_MAX = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))   # reading: midpoint of the two end-quantile rules


# --------------------------------------------------------------------------------------
# codebook (reading of the transcript @2:19: levels at normal quantiles)
# --------------------------------------------------------------------------------------

def _linspace(start: float, stop: float, num: int) -> list[float]:
    """`num` fp64 points from start to stop inclusive."""
    step = (stop - start) / (num - 1)
    return [start + i * step for i in range(num)]


def codebook_fp64() -> np.ndarray:
    """The 16 NF4 levels in fp64, before rounding to fp32.

    Positive levels: Phi^-1 at 9 evenly spaced probabilities from P_MAX down to 1/2, with 1/2
    dropped (8 levels).  Negative levels: -Phi^-1 at 8 evenly spaced probabilities from P_MAX
    down to 1/2, with 1/2 dropped (7 levels).  Plus an exact zero.  All divided by Phi^-1(P_MAX).
    """
    inv = statistics.NormalDist().inv_cdf
    z_max = inv(P_MAX)
    positive = [inv(p) for p in _linspace(P_MAX, 0.5, 9)[:-1]]
    negative = [-inv(p) for p in _linspace(P_MAX, 0.5, 8)[:-1]]
    levels = sorted(negative + [0.0] + positive)
    return np.array([lv / z_max for lv in levels], dtype=np.float64)


def codebook() -> np.ndarray:
    """q[0..15]: the NF4 levels rounded to fp32 (q[0] = -1, q[7] = 0, q[15] = +1)."""
    return codebook_fp64().astype(np.float32)


def code_thresholds() -> np.ndarray:
    """m[0..14] = fl32((q_i + q_{i+1}) / 2), the mean taken in fp64."""
    q = codebook().astype(np.float64)
    return ((q[:-1] + q[1:]) / 2.0).astype(np.float32)


def int8_levels() -> np.ndarray:
    """code8[v] = fl32(v / 127) for v = -127 .. 127 (index v + 127)."""
    v = np.arange(-127, 128, dtype=np.float32)
    return v / np.float32(127.0)


def int8_thresholds() -> np.ndarray:
    """t[v] = fl32((code8[v] + code8[v+1]) / 2) for v = -127 .. 126, mean in fp64."""
    c = int8_levels().astype(np.float64)
    return ((c[:-1] + c[1:]) / 2.0).astype(np.float32)


# --------------------------------------------------------------------------------------
# bf16 round-to-nearest-even
# --------------------------------------------------------------------------------------

def bf16_rne(f: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16, nearest-even; returns the uint16 bit patterns.

    Adds 0x7FFF plus the lowest kept bit to the fp32 bit pattern and keeps the upper 16
    bits (inputs are finite; denormals are kept).
    """
    bits = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    return ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the fp32 values they denote (exact)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------
# pack: first pass, then the second pass over its constants (transcript @2:19-2:29)
# --------------------------------------------------------------------------------------

def _count_greater(x: np.ndarray, thresholds: np.ndarray) -> np.ndarray:
    """For each x, the number of thresholds t with x > t (an exact tie counts as not greater)."""
    count = np.zeros(x.shape, dtype=np.int32)
    for t in thresholds:
        count += (x > t)
    return count


def check_shape(rows: int, cols: int) -> None:
    if rows <= 0 or cols <= 0 or cols % BLOCK != 0 or (rows * cols) % (BLOCK * GROUP) != 0:
        raise ValueError(f"NF4 needs cols % {BLOCK} == 0 and rows*cols % {BLOCK * GROUP} == 0, "
                         f"got {rows}x{cols}")


def first_pass(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Blockwise absmax quantisation of fp32 W.

    Returns (code per element as uint8 0..15 in row-major order, c_b per block as fp32).
    c_b = max |w| over the 64 elements (exact); x = fl32(w / c_b) (x = 0 when c_b = 0);
    code = number of level midpoints m_i with x > m_i.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    blocks = w.reshape(-1, BLOCK)
    c = np.abs(blocks).max(axis=1)
    x = np.zeros_like(blocks)
    np.divide(blocks, c[:, None], out=x, where=c[:, None] > 0)
    codes = _count_greater(x, code_thresholds()).astype(np.uint8)
    return codes.reshape(-1), c


def second_pass(c: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.float32]:
    """Double quantisation of the block constants c_b.

    mu = fl32(S / n_b) with S the left-to-right fp64 sum of the c_b;  d_b = fl32(c_b - mu);
    per group g of 256 blocks s2_g = max |d_b| and y = fl32(d_b / s2_g) (0 when s2_g = 0);
    v_b = -127 + number of int8 midpoints t with y > t.
    Returns (qabsmax int8[n_b], absmax2 fp32[n_b / 256], mu fp32).
    """
    c = np.ascontiguousarray(c, dtype=np.float32)
    n_b = c.size
    S = np.add.accumulate(c.astype(np.float64))[-1]        # sequential sum, left to right
    mu = np.float32(S / np.float64(n_b))
    d = c - mu
    groups = d.reshape(-1, GROUP)
    s2 = np.abs(groups).max(axis=1)
    y = np.zeros_like(groups)
    np.divide(groups, s2[:, None], out=y, where=s2[:, None] > 0)
    v = -127 + _count_greater(y.reshape(-1), int8_thresholds())
    return v.astype(np.int8), s2.astype(np.float32), mu


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Byte j = code[2j] << 4 | code[2j+1]."""
    codes = codes.astype(np.uint8).reshape(-1, 2)
    return ((codes[:, 0] << 4) | codes[:, 1]).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: the per-element codes in row-major order."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed >> 4
    out[1::2] = packed & 0x0F
    return out


def pack(w: np.ndarray) -> dict:
    """NF4-pack fp32 W[rows][cols]: codes u8[n/2], qabsmax i8[n/64], absmax2 f32[n/16384], mean."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    check_shape(rows, cols)
    codes, c = first_pass(w)
    qabsmax, absmax2, mu = second_pass(c)
    return {"rows": rows, "cols": cols, "codes": pack_nibbles(codes), "qabsmax": qabsmax,
            "absmax2": absmax2, "mean": np.float32(mu)}


# --------------------------------------------------------------------------------------
# dequantise
# --------------------------------------------------------------------------------------

def decode_absmax(qabsmax: np.ndarray, absmax2: np.ndarray, mean) -> np.ndarray:
    """c'_b = fl32( fl32(code8[v_b] * s2_g) + mu ), two separately rounded fp32 operations."""
    code8 = int8_levels()[np.asarray(qabsmax, dtype=np.int32) + 127]
    s2 = np.repeat(np.asarray(absmax2, dtype=np.float32), GROUP)
    scaled = code8 * s2
    return scaled + np.float32(mean)


def dequant_f32(p: dict) -> np.ndarray:
    """fl32(q[code] * c'_b) for every element, as fp32 [rows, cols]."""
    q = codebook()
    codes = unpack_nibbles(p["codes"]).reshape(-1, BLOCK)
    cprime = decode_absmax(p["qabsmax"], p["absmax2"], p["mean"])
    w_hat = q[codes] * cprime[:, None]
    return w_hat.reshape(p["rows"], p["cols"])


def dequant_bf16(p: dict) -> np.ndarray:
    """bf16_RNE(fl32(q[code] * c'_b)) as uint16 bit patterns [rows, cols]."""
    return bf16_rne(dequant_f32(p))
