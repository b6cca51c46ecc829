"""Reference INT8 and INT4 K/V pages: quantised append and fill, decode attention on them.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources: "Building an LLM inference engine from scratch: KV cache, operator
fusion and quantisation practice", section 5.1 (the KV cache may be stored as
INT8, or lower, and dequantised back to the compute precision before
attention; this halves the cache memory at some cost in accuracy) and section
3.4 (symmetric quantisation: the scale is the largest magnitude divided by
2^(bits-1) - 1; a value's code is its quotient by the scale, rounded and
clamped to the signed range; dequantisation widens the code to float32 and
multiplies it by the scale).

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* Granularity: one scale per (token, KV head) row of ``D`` values, separately
  for K and for V.  The pages' example quantises a whole tensor with one
  scale; the cache grows by one token per step, and a row scale is the one
  granularity that never needs an earlier token's codes to be redone.
* Arithmetic of the quantiser: the BF16 inputs are widened to FP32 (exact);
  the largest magnitude is exact; the scale is the FP32 quotient of it by 127
  (round to nearest even); each code is the FP32 quotient of the value by the
  scale, rounded to the nearest integer with ties to even (the rounding of
  the pages' ``round``), then clamped to [-128, 127].  The pages' dequantiser
  multiplies by the scale in float32, which fixes the scale as an FP32
  number.
* A row of zeros would divide zero by zero; it stores scale 0 and codes 0
  (it dequantises to zeros, the only sensible result).
* The dequantised value is ``code * scale`` taken exactly (float64 holds the
  product of an 8-bit integer and an FP32 number exactly); attention on the
  dequantised cache is then the plain definition of the BF16 oracle.
* Inputs are finite.
* INT4 pages (section 5.1: INT8 "or even INT4") use the same quantiser with
  ``bits = 4``: scale = max|x| / 7, codes clamped to [-8, 7].  Two codes
  share a byte, stored offset by 8 (``u = code + 8`` in 0..15): byte ``j`` of
  a 64-value row holds dim ``2j`` in its low nibble and dim ``2j + 1`` in its
  high nibble.

Layout (the library's format, which these functions also define):

* ``k_codes``, ``v_codes``: int8 ``[num_pages][Hkv][P][D]``: within a page,
  each KV head's 16 token rows of 64 codes are one contiguous 1 KiB block;
* INT4: ``k_codes``, ``v_codes``: uint8 ``[num_pages][Hkv][P][D/2]`` (packed as
  above): each KV head's 16 token rows are one contiguous 512-byte block;
* ``scales``: float32 ``[num_pages][Hkv][2][P]``: for page ``p`` and KV head
  ``g``, the 16 K scales of the page's slots, then the 16 V scales.

Parity pins for every function here live in the oracle tests; none is
"parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

from .paged_decode import attention_one_query, bf16_bits_to_f64, kv_head_of

QMAX = 127                      # 2^(8-1) - 1
QMIN = -128
QMAX4 = 7                       # 2^(4-1) - 1
QMIN4 = -8


# ---------------------------------------------------------------------------
# The quantiser (section 3.4, one row at a time)
# ---------------------------------------------------------------------------
def quantize_rows(bits, nbits: int = 8):
    """Symmetric quantisation of BF16 rows along the last axis to ``nbits``
    (8 or 4) signed bits.

    Returns ``(codes int8 [..., D], scale float32 [...])``.  Every step is an
    FP32 operation of numpy, which rounds to nearest even like IEEE hardware.
    """
    qmax, qmin = (QMAX, QMIN) if nbits == 8 else (QMAX4, QMIN4)
    b = np.asarray(bits, dtype=np.uint16)
    x = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)    # exact widening
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(qmax)).astype(np.float32)
    zero = scale == 0
    safe = np.where(zero, np.float32(1), scale).astype(np.float32)
    ratio = (x / safe[..., None]).astype(np.float32)                 # FP32 quotient
    codes = np.clip(np.rint(ratio), qmin, qmax)                       # ties to even
    codes = np.where(zero[..., None], 0, codes).astype(np.int8)
    return codes, scale


def pack_q4(codes) -> np.ndarray:
    """INT4 codes ``[..., D]`` (in [-8, 7]) -> bytes ``[..., D/2]``: dim 2j in the
    low nibble of byte j, dim 2j+1 in its high nibble, each stored as code + 8."""
    u = (np.asarray(codes, np.int16) + 8).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_q4(packed) -> np.ndarray:
    """Bytes ``[..., D/2]`` -> INT4 codes ``[..., D]`` (int8)."""
    b = np.asarray(packed, np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = (b & 0x0F).astype(np.int16) - 8
    out[..., 1::2] = (b >> 4).astype(np.int16) - 8
    return out


def dequantize(codes, scale) -> np.ndarray:
    """``code * scale`` in float64 (exact); ``scale`` broadcasts over the last axis."""
    return np.asarray(codes, np.float64) * np.asarray(scale, np.float64)[..., None]


# ---------------------------------------------------------------------------
# Writing into the pages
# ---------------------------------------------------------------------------
def _write_token(k_codes, v_codes, scales, physical, slot, k_row_bits, v_row_bits, nbits=8):
    kc, ks = quantize_rows(k_row_bits, nbits)     # [Hkv][D], [Hkv]
    vc, vs = quantize_rows(v_row_bits, nbits)
    if nbits == 4:
        kc, vc = pack_q4(kc), pack_q4(vc)
    k_codes[physical, :, slot] = kc
    v_codes[physical, :, slot] = vc
    scales[physical, :, 0, slot] = ks
    scales[physical, :, 1, slot] = vs


def append_kv_q8(k_codes, v_codes, scales, k_new_bits, v_new_bits, block_tables, seq_lens,
                 nbits: int = 8):
    """Quantise each sequence's new K/V row into its page slot; return new pools.

    As the BF16 append (token ``L-1`` goes to logical page ``(L-1) // P``,
    slot ``(L-1) % P``; idle slots write nothing), with each (token, head)
    row stored as its codes and its scale (``nbits`` 8 or 4).
    """
    kc, vc, sc = (np.array(a, copy=True) for a in (k_codes, v_codes, scales))
    page_size = kc.shape[2]
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        if L == 0:
            continue
        pos = L - 1
        physical = int(block_tables[b][pos // page_size])
        _write_token(kc, vc, sc, physical, pos % page_size, k_new_bits[b], v_new_bits[b], nbits)
    return kc, vc, sc


def fill_kv_q8(k_codes, v_codes, scales, k_rows_bits, v_rows_bits, block_table_row, start: int,
               nbits: int = 8):
    """Quantise tokens ``start .. start+T-1`` of one sequence into their pages."""
    kc, vc, sc = (np.array(a, copy=True) for a in (k_codes, v_codes, scales))
    page_size = kc.shape[2]
    for j in range(len(k_rows_bits)):
        t = start + j
        physical = int(block_table_row[t // page_size])
        _write_token(kc, vc, sc, physical, t % page_size, k_rows_bits[j], v_rows_bits[j], nbits)
    return kc, vc, sc


# ---------------------------------------------------------------------------
# Reading the pages back and attending
# ---------------------------------------------------------------------------
def gather_sequence_q8(codes, scales, which: int, block_table_row, seq_len: int,
                       nbits: int = 8) -> np.ndarray:
    """Dequantised ``[L][Hkv][D]`` float64 rows of one sequence (which: 0 = K, 1 = V)."""
    codes = np.asarray(codes)
    hkv, page_size, d = codes.shape[1:]
    if nbits == 4:
        d *= 2
    rows = []
    for t in range(seq_len):
        physical = int(block_table_row[t // page_size])
        slot = t % page_size
        c = codes[physical, :, slot]
        if nbits == 4:
            c = unpack_q4(c)
        rows.append(dequantize(c, scales[physical, :, which, slot]))
    if not rows:
        return np.zeros((0, hkv, d), dtype=np.float64)
    return np.stack(rows)


def decode_attention_q8(q_bits, k_codes, v_codes, scales, block_tables, seq_lens, scale: float,
                        sequences=None, nbits: int = 8) -> np.ndarray:
    """Paged GQA decode attention over dequantised INT8 pages, in float64.

    The cache is dequantised first (section 5.1: dequantise before the
    attention), then each query head attends as in the BF16 definition.
    Returns ``[B][Hq][D]`` (idle rows zero).
    """
    q_all = np.asarray(q_bits)
    B, Hq, D = q_all.shape
    Hkv = np.asarray(k_codes).shape[1]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    todo = range(B) if sequences is None else sequences
    for b in todo:
        L = int(seq_lens[b])
        if L == 0:
            continue
        K = gather_sequence_q8(k_codes, scales, 0, block_tables[b], L, nbits)
        V = gather_sequence_q8(v_codes, scales, 1, block_tables[b], L, nbits)
        q = bf16_bits_to_f64(q_all[b])
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h] = attention_one_query(q[h], K[:, g, :], V[:, g, :], scale)[0]
    return out


# ---------------------------------------------------------------------------
# How far quantisation can move the output
# ---------------------------------------------------------------------------
def quantisation_error_bound(q, K, K_hat, V, V_hat, scale: float) -> np.ndarray:
    """Bound on ``|attn(q, K_hat, V_hat) - attn(q, K, V)|`` per output dim (float64).

    With scores ``s_t = scale q.k_t``, weights ``w = softmax(s)`` and
    ``eps = max_t |scale q.(k_hat_t - k_t)|``, every weight moves by a factor
    in ``[e^-2eps, e^2eps]`` (its numerator and the normaliser each by at most
    ``e^eps``), so ``|w_hat_t - w_t| <= w_t (e^2eps - 1)``.  Writing
    ``o_hat - o = sum_t (w_hat_t - w_t) v_hat_t + sum_t w_t (v_hat_t - v_t)``:

        |o_hat_d - o_d| <= (e^2eps - 1) sum_t w_t |v_hat_td| + sum_t w_t |v_hat_td - v_td|.

    ``q`` ``[D]``, ``K``/``K_hat``/``V``/``V_hat`` ``[L][D]``, all float64.
    """
    if len(K) == 0:
        return np.zeros(np.shape(V)[1:], dtype=np.float64)
    s = scale * (K @ q)
    e = np.exp(s - s.max())
    w = e / e.sum()
    eps = float(np.max(np.abs(scale * ((K_hat - K) @ q))))
    grow = math.expm1(2.0 * eps)
    return grow * (w @ np.abs(V_hat)) + w @ np.abs(V_hat - V)
