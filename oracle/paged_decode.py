"""Float64 reference for paged GQA decode attention and the one-token append.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Layout of the inputs, as the caller hands them over (all little-endian):

* ``q``            uint16 BF16 bits ``[B][Hq][D]``  -- one new query per sequence
* ``k_pool``       uint16 BF16 bits ``[num_pages][P][Hkv][D]``
* ``v_pool``       same layout as ``k_pool``
* ``block_tables`` int32 ``[B][max_blocks]`` -- logical page -> physical page
* ``seq_lens``     int32 ``[B]`` -- attention length of each sequence

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* Query head ``h`` reads KV head ``h // (Hq // Hkv)`` (consecutive groups).
  The pages name grouped-query attention only; this is the usual grouping.
* Token ``t`` of a sequence sits in physical page ``block_tables[b][t // P]``
  at slot ``t % P`` (the pages: one shared pool, a block table per sequence,
  16 tokens per page).
* A sequence of length ``L`` attends tokens ``0 .. L-1``, the new token
  included; a decode query sits at the last position, so the causal mask of
  the attention definition removes nothing.
* ``L == 0`` marks an idle batch slot: its output row is zero.

Parity pins for every function here live in the oracle tests; none is
"parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# Number format
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode BF16 bit patterns to float64 exactly.

    BF16 keeps the sign, the 8-bit exponent and the top 7 fraction bits of an
    IEEE binary32 ("Building a high-performance LLM inference engine from
    scratch with Tiny-vLLM", section on the BF16 choice).  Its bits are
    therefore the upper half of a binary32 word, and widening binary32 to
    binary64 is exact.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Paged cache addressing
# ---------------------------------------------------------------------------
def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``h``: consecutive groups of Hq/Hkv heads."""
    group = num_q_heads // num_kv_heads
    return h // group


def gather_sequence(pool_bits, block_table_row, seq_len: int) -> np.ndarray:
    """Return the logical ``[L][Hkv][D]`` float64 cache rows of one sequence.

    The engine keeps K and V in one shared pool of fixed-size physical pages
    and maps each sequence's logical pages through its own block table ("6
    Hours of YouTube and 85 handtyped pages of notes on LLM Inference",
    features completed so far: shared BF16 KV page pool with per-sequence
    block tables, 16 tokens per page).  Logical page ``i`` covers tokens
    ``i*P .. i*P+P-1``; only the first ``L - i*P`` slots of the last page are
    part of the sequence.  This is the contiguous gather the GPU kernel never
    performs; the oracle does it because it is the plain definition.
    """
    pool = np.asarray(pool_bits)
    page_size = pool.shape[1]
    n_pages = (seq_len + page_size - 1) // page_size
    parts = []
    for i in range(n_pages):
        physical = int(block_table_row[i])
        valid = min(page_size, seq_len - i * page_size)
        parts.append(pool[physical, :valid])
    if not parts:
        return np.zeros((0,) + pool.shape[2:], dtype=np.float64)
    return bf16_bits_to_f64(np.concatenate(parts, axis=0))


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def attention_one_query(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Single-query attention with a two-pass, max-subtracted softmax.

    Follows "Building an LLM inference engine from scratch: KV cache, operator
    fusion and quantisation practice", section 3.2: scores are the dot products
    of the query with every cached key, scaled (here by ``scale``, which is
    1/sqrt(head_dim) for the model); the softmax over the sequence subtracts
    the maximum score first; the output is the softmax-weighted sum of the
    cached values.

    Pass 1 computes every score and their maximum; pass 2 exponentiates,
    normalises and accumulates.  Returns ``(o, w, lse)``: the output row, the
    normalised weights and ``log(sum_t exp(s_t))``.
    """
    s = scale * (K @ q)                     # pass 1: scores
    m = s.max()
    e = np.exp(s - m)                       # pass 2: exponentials
    z = e.sum()
    w = e / z
    o = (e @ V) / z
    return o, w, m + math.log(z)


def decode_attention(q_bits, k_pool_bits, v_pool_bits, block_tables, seq_lens,
                     scale: float, sequences=None, return_weights: bool = False,
                     return_lse: bool = False):
    """Paged GQA decode attention for a batch, in float64.

    Each active sequence's query heads attend that sequence's cached tokens
    only, through its own block table and attention length ("6 Hours of
    YouTube ...", features completed so far: batched decode with a page map and
    attention length per sequence; paged decode attention streaming each query
    head's pages).  The result is the same as the textbook computation on the
    gathered cache, which is what this function does.

    ``sequences`` restricts the work to the listed batch indices (other rows
    stay zero).  Returns ``out`` float64 ``[B][Hq][D]`` and, on request, the
    per-(b, h) weights (a dict) and log-sum-exp (float64 ``[B][Hq]``, ``-inf``
    for idle slots).
    """
    q_all = np.asarray(q_bits)
    B, Hq, D = q_all.shape
    Hkv = np.asarray(k_pool_bits).shape[2]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    weights = {}
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    todo = range(B) if sequences is None else sequences
    for b in todo:
        L = int(seq_lens[b])
        if L == 0:
            continue
        K = gather_sequence(k_pool_bits, block_tables[b], L)
        V = gather_sequence(v_pool_bits, block_tables[b], L)
        q = bf16_bits_to_f64(q_all[b])
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            o, w, l = attention_one_query(q[h], K[:, g, :], V[:, g, :], scale)
            out[b, h] = o
            lse[b, h] = l
            if return_weights:
                weights[(b, h)] = w
    extras = []
    if return_weights:
        extras.append(weights)
    if return_lse:
        extras.append(lse)
    return (out, *extras) if extras else out


# ---------------------------------------------------------------------------
# One-token append
# ---------------------------------------------------------------------------
def append_kv(k_pool_bits, v_pool_bits, k_new_bits, v_new_bits, block_tables, seq_lens):
    """Write each sequence's new K/V row into its page slot; return new pools.

    Decode appends the new token's K/V at its absolute position ("6 Hours of
    YouTube ...", features completed so far).  ``seq_lens[b]`` is the length
    after the append, so the new token is token ``L-1``; it lands in logical
    page ``(L-1) // P``, slot ``(L-1) % P``.  Idle slots (``L == 0``) write
    nothing.  Pure integer work: the bit patterns are copied unchanged.
    """
    k_out = np.array(k_pool_bits, copy=True)
    v_out = np.array(v_pool_bits, copy=True)
    page_size = k_out.shape[1]
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        if L == 0:
            continue
        pos = L - 1
        physical = int(block_tables[b][pos // page_size])
        slot = pos % page_size
        k_out[physical, slot] = k_new_bits[b]
        v_out[physical, slot] = v_new_bits[b]
    return k_out, v_out


def fill_kv(k_pool_bits, v_pool_bits, k_rows_bits, v_rows_bits, block_table_row, start: int):
    """Write tokens ``start .. start+T-1`` of one sequence into its pages; return new pools.

    The prefill fills the prompt's pages ("6 Hours of YouTube ...", features
    completed so far: prefill fills the prompt pages, decode appends one
    token); token t goes to page ``block_table_row[t // P]``, slot ``t % P``.
    ``k_rows_bits``/``v_rows_bits``: ``[T][Hkv][D]``.  Integer copy only.
    """
    k_out = np.array(k_pool_bits, copy=True)
    v_out = np.array(v_pool_bits, copy=True)
    page_size = k_out.shape[1]
    for j in range(len(k_rows_bits)):
        t = start + j
        physical = int(block_table_row[t // page_size])
        k_out[physical, t % page_size] = k_rows_bits[j]
        v_out[physical, t % page_size] = v_rows_bits[j]
    return k_out, v_out
