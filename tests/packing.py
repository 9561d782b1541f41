"""Block *encoders* used by the tests to build blocks from chosen field values.

They state the ggml block layouts in the encoding direction (fields -> bytes),
written independently of the oracle's decoder and of the GPU kernels, so that a
block built here with known fields has a known, closed-form set of weights.

Layout (byte offsets within one block):
  Q4_0 (32 weights, 18 B): fp16 d @0; quant byte j (0..15) @2+j holds weight j in
      its low nibble and weight j+16 in its high nibble.
  Q4_K (256 weights, 144 B): fp16 d @0, fp16 dmin @2, 12 scale bytes @4, quant
      bytes @16.  Weight i: chunk c = i // 64, j = i % 64; j < 32 -> low nibble of
      quant byte 32c + j (sub-block 2c); else high nibble of 32c + j - 32
      (sub-block 2c + 1).  Scale bytes: for s < 4, byte s = sc_s | (sc_{s+4} >> 4) << 6,
      byte s+4 = m_s | (m_{s+4} >> 4) << 6, byte s+8 = (sc_{s+4} & 15) | (m_{s+4} & 15) << 4.
  Q6_K (256 weights, 210 B): ql @0 (128 B), qh @128 (64 B), int8 scales @192 (16),
      fp16 d @208.  Weight i: h = i // 128, r = i % 128, g = r // 32, l = r % 32;
      low 4 bits -> ql[64h + l + 32(g % 2)] (low nibble if g < 2, else high);
      high 2 bits -> bits 2g..2g+1 of qh[32h + l]; scale index 8h + r // 16.
  Q5_K (256 weights, 176 B): Q4_K's 16-byte header, 32 fifth-bit bytes @16,
      Q4_K's 128 quant bytes @48 (low four bits as in Q4_K).  Weight i
      (c = i // 64, j = i % 64): fifth bit = bit 2c + (j >= 32) of qh[j % 32].
"""
from __future__ import annotations

import numpy as np


def f16_bits(v: float) -> int:
    return int(np.array([v], np.float16).view(np.uint16)[0])


def pack_q4_0(d_bits: int, q) -> np.ndarray:
    q = [int(v) for v in q]
    assert len(q) == 32 and all(0 <= v < 16 for v in q)
    b = np.zeros(18, np.uint8)
    b[0], b[1] = d_bits & 0xFF, d_bits >> 8
    for j in range(16):
        b[2 + j] = q[j] | (q[j + 16] << 4)
    return b


def pack_q4_k(d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    q = [int(v) for v in q]
    assert len(sc) == 8 and len(m) == 8 and len(q) == 256
    assert all(0 <= v < 64 for v in sc + m) and all(0 <= v < 16 for v in q)
    b = np.zeros(144, np.uint8)
    b[0], b[1] = d_bits & 0xFF, d_bits >> 8
    b[2], b[3] = dmin_bits & 0xFF, dmin_bits >> 8
    for s in range(4):
        b[4 + s] = (sc[s] & 63) | ((sc[s + 4] >> 4) << 6)
        b[4 + s + 4] = (m[s] & 63) | ((m[s + 4] >> 4) << 6)
        b[4 + s + 8] = (sc[s + 4] & 15) | ((m[s + 4] & 15) << 4)
    for i in range(256):
        c, j = divmod(i, 64)
        if j < 32:
            b[16 + 32 * c + j] |= q[i]
        else:
            b[16 + 32 * c + j - 32] |= q[i] << 4
    return b


def pack_q6_k(d_bits: int, sc, q) -> np.ndarray:
    sc = [int(v) for v in sc]
    q = [int(v) for v in q]
    assert len(sc) == 16 and len(q) == 256
    assert all(-128 <= v < 128 for v in sc) and all(0 <= v < 64 for v in q)
    b = np.zeros(210, np.uint8)
    for i in range(256):
        h, r = divmod(i, 128)
        g, l = divmod(r, 32)
        li = 64 * h + l + 32 * (g % 2)
        if g < 2:
            b[li] |= q[i] & 15
        else:
            b[li] |= (q[i] & 15) << 4
        b[128 + 32 * h + l] |= (q[i] >> 4) << (2 * g)
    b[192:208] = np.array(sc, np.int8).view(np.uint8)
    b[208], b[209] = d_bits & 0xFF, d_bits >> 8
    return b


def q4_0_sub(i: int) -> int:
    return 0


def q4_k_sub(i: int) -> int:
    """Sub-block (0..7) of weight i in a Q4_K block (32 consecutive weights)."""
    return i // 32


def q6_k_sub(i: int) -> int:
    """Scale index (0..15) of weight i in a Q6_K block (16 consecutive weights)."""
    return i // 16


def pack_q5_k(d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 32 for v in q)
    base = pack_q4_k(d_bits, dmin_bits, sc, m, [v & 15 for v in q])
    b = np.zeros(176, np.uint8)
    b[0:16] = base[0:16]
    b[48:176] = base[16:144]
    for i in range(256):
        c, j = divmod(i, 64)
        if q[i] >> 4:
            b[16 + j % 32] |= 1 << (2 * c + (j >= 32))
    return b
