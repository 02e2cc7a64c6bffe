"""W12: lossless 12-bit storage of bf16 weights (oracle encoder and decoder).

Source: SpecPilot summary (onedev.kr), section 무엇과 다른가 ("how it
differs").  Each output channel keeps the 16 consecutive binades in which most
of its weights lie.  A weight inside that window is stored in 12 bits: its
sign, its exponent as a 4-bit offset from the window's lowest exponent, and
its 7 mantissa bits.  Everything else -- values outside the window, zeros and
subnormals -- is kept exactly in a per-channel sparse list of escapes.

Readings of points the page leaves open (the plainest ones the rest supports):

* a channel is one row of the ``[out, in]`` weight (an output channel);
* the window ``[base, base+15]`` covers normal exponents only, so
  ``1 <= base <= 239``; it is the one holding the most weights, the smallest
  ``base`` on ties; +-0, subnormals (exponent 0), +-inf and NaN (exponent
  255) always escape;
* a record is ``sign << 11 | (exp - base) << 7 | mantissa`` (sign first);
  an escaped slot holds record 0;
* records are stored as two planes per channel: ``hi = record >> 4`` (one
  byte per weight: sign, offset and the top three mantissa bits) and the low
  four bits packed two per byte, even ``k`` in the low nibble, odd ``k_in``
  padded with a zero nibble;
* escapes are CSR over channels: ``esc_ptr`` (uint32, ``n_out + 1``),
  ``esc_idx`` (uint16 column, ascending within a channel) and ``esc_val``
  (uint16, the raw bf16 bits).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

WINDOW = 16
BASE_MIN, BASE_MAX = 1, 254 - WINDOW + 1  # 1 .. 239


@dataclass
class W12Tensor:
    n_out: int
    k_in: int
    hi: np.ndarray       # uint8  [n_out, k_in]
    lo: np.ndarray       # uint8  [n_out, ceil(k_in/2)]
    base: np.ndarray     # uint8  [n_out]
    esc_ptr: np.ndarray  # uint32 [n_out + 1]
    esc_idx: np.ndarray  # uint16 [n_esc]
    esc_val: np.ndarray  # uint16 [n_esc]

    @property
    def n_esc(self) -> int:
        return int(self.esc_ptr[-1])

    def nbytes(self) -> int:
        """Bytes of the format: planes + base + esc_ptr + 4 per escape."""
        return (self.hi.size + self.lo.size + self.base.size + 4 * self.esc_ptr.size
                + 2 * self.esc_idx.size + 2 * self.esc_val.size)

    def bits_per_weight(self) -> float:
        return 8.0 * self.nbytes() / float(self.n_out * self.k_in)


def exponent_histogram(w: np.ndarray) -> np.ndarray:
    """Per-channel counts of each biased exponent value, normal exponents only."""
    n, k = w.shape
    e = ((w >> 7) & 0xFF).astype(np.int64)
    flat = e + 256 * np.arange(n, dtype=np.int64)[:, None]
    hist = np.bincount(flat.ravel(), minlength=256 * n).reshape(n, 256)
    hist[:, 0] = 0
    hist[:, 255] = 0
    return hist


def choose_base(hist: np.ndarray) -> np.ndarray:
    """Lowest exponent of the 16-binade window holding the most weights (smallest on ties)."""
    cs = np.concatenate([np.zeros((hist.shape[0], 1), np.int64), np.cumsum(hist, axis=1)], axis=1)
    b = np.arange(BASE_MIN, BASE_MAX + 1)
    counts = cs[:, b + WINDOW] - cs[:, b]  # counts[:, j] = sum(hist[:, b_j : b_j + 16])
    return (BASE_MIN + np.argmax(counts, axis=1)).astype(np.uint8)


def encode(w_bits: np.ndarray) -> W12Tensor:
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    if w.ndim != 2:
        raise ValueError("weights must be [n_out, k_in]")
    n, k = w.shape
    base = choose_base(exponent_histogram(w))
    sign = (w >> 15).astype(np.uint16)
    exp = ((w >> 7) & 0xFF).astype(np.int32)
    man = (w & 0x7F).astype(np.uint16)
    b = base.astype(np.int32)[:, None]
    inside = (exp >= b) & (exp <= b + WINDOW - 1)
    off = np.where(inside, exp - b, 0).astype(np.uint16)
    rec = np.where(inside, (sign << 11) | (off << 7) | man, 0).astype(np.uint16)
    hi = (rec >> 4).astype(np.uint8)
    nib = (rec & 0xF).astype(np.uint8)
    if k % 2:
        nib = np.concatenate([nib, np.zeros((n, 1), np.uint8)], axis=1)
    lo = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    esc = ~inside
    counts = esc.sum(axis=1)
    esc_ptr = np.zeros(n + 1, dtype=np.uint32)
    esc_ptr[1:] = np.cumsum(counts)
    rows, cols = np.nonzero(esc)  # row-major: channel, then ascending k
    if k > 65536:
        raise ValueError("k_in > 65536 does not fit uint16 escape indices")
    return W12Tensor(n, k, hi, lo, base, esc_ptr, cols.astype(np.uint16),
                     w[rows, cols].astype(np.uint16))


def records(t: W12Tensor) -> np.ndarray:
    """The 12-bit records (uint16) reassembled from the two planes."""
    lo = np.empty((t.n_out, 2 * t.lo.shape[1]), dtype=np.uint16)
    lo[:, 0::2] = t.lo & 0xF
    lo[:, 1::2] = t.lo >> 4
    return (t.hi.astype(np.uint16) << 4) | lo[:, : t.k_in]


def decode(t: W12Tensor) -> np.ndarray:
    """Exact bf16 bit patterns ``[n_out, k_in]``."""
    r = records(t)
    base = t.base.astype(np.uint16)[:, None]
    exp = ((r >> 7) & 0xF) + base  # <= 254: never reaches the sign bit
    out = (((r >> 11) & 1) << 15) | (exp << 7) | (r & 0x7F)
    out = out.astype(np.uint16)
    counts = np.diff(t.esc_ptr.astype(np.int64))
    rows = np.repeat(np.arange(t.n_out), counts)
    out[rows, t.esc_idx.astype(np.int64)] = t.esc_val
    return out


def decode_hi8(t: W12Tensor) -> np.ndarray:
    """The weights seen through the 8-bit leading view of each record, as bf16
    bit patterns ``[n_out, k_in]`` (SpecPilot summary, section 무엇과 다른가:
    two-level verification runs its Q pass on the 8-bit view of the front of
    the W12 records).

    Reading: the view is the ``hi`` plane, ``record >> 4`` (sign, exponent
    offset and the top three mantissa bits); the weight it stands for is the
    record with its low four mantissa bits cleared, decoded with the
    channel's window, i.e. the bf16 value truncated toward zero to three
    mantissa bits.  Escaped slots are not records: they keep their exact
    values from the escape list, which is part of the format.
    """
    r = t.hi.astype(np.uint16) << 4
    base = t.base.astype(np.uint16)[:, None]
    exp = ((r >> 7) & 0xF) + base
    out = ((((r >> 11) & 1) << 15) | (exp << 7) | (r & 0x7F)).astype(np.uint16)
    counts = np.diff(t.esc_ptr.astype(np.int64))
    rows = np.repeat(np.arange(t.n_out), counts)
    out[rows, t.esc_idx.astype(np.int64)] = t.esc_val
    return out
