"""Seeded synthetic inputs for paged GQA decode attention.

This module is the only code the CPU oracle and the HIP path share: it draws
random numbers, rounds them to BF16 and lays them out in a page pool.  It holds
none of the attention arithmetic.

Shapes follow the Llama-3.2-1B layer the pages describe ("6 Hours of YouTube
and 85 handtyped pages of notes on LLM Inference", features completed so far
and current scope): 32 query heads sharing 8 KV heads of dimension 64, BF16
K/V in a shared pool of 16-token pages reached through per-sequence block
tables, a 2,048-token context and a 128 MiB default pool.

Pool layout handed to both sides: ``[num_pages][16 slots][8 kv heads][64]``
BF16 bits for K and, separately, for V.  Every pool byte that no sequence owns
(unused pages, slots past a sequence's length in its last page, the slot a
pending append will fill) holds the BF16 quiet NaN ``0x7FC0``, and every
unused block-table entry holds ``-1``, so that a kernel reading anything
outside the sequence shows it in the result.

Random numbers come from NumPy's PCG64 ``default_rng``: standard normals drawn
in float32, scaled, then rounded to BF16 with round-to-nearest-even.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 64
PAGE_SIZE = 16
MAX_CONTEXT = 2048
MAX_BLOCKS = MAX_CONTEXT // PAGE_SIZE          # block-table row length (128)
SCALE = 0.125                                   # 1/sqrt(64)
BF16_NAN = 0x7FC0
PAGE_BYTES_K = PAGE_SIZE * NUM_KV_HEADS * HEAD_DIM * 2   # 16 KiB of K per page


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to BF16 bit patterns, round-to-nearest-even.

    Adds ``0x7FFF`` plus the lowest kept bit to the binary32 word and keeps the
    upper 16 bits (the usual bias method).  Inputs here are finite normals.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


@dataclass
class DecodeBatch:
    """One layer's decode-step inputs, as BF16 bit arrays and int32 metadata."""

    name: str
    q: np.ndarray               # uint16 [B][32][64]
    k_pool: np.ndarray          # uint16 [num_pages][16][8][64]
    v_pool: np.ndarray          # uint16 [num_pages][16][8][64]
    block_tables: np.ndarray    # int32  [B][128]
    seq_lens: np.ndarray        # int32  [B]
    scale: float = SCALE
    k_new: Optional[np.ndarray] = None   # uint16 [B][8][64] when the step appends
    v_new: Optional[np.ndarray] = None
    recipe: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0


def pages_for(seq_len: int) -> int:
    return (int(seq_len) + PAGE_SIZE - 1) // PAGE_SIZE


def make_batch(seq_lens, num_pages: int, seed, *, q_sigma: float = 1.0,
               append: bool = False, placement: str = "random",
               name: str = "custom", recipe: Optional[dict] = None,
               max_blocks: int = MAX_BLOCKS) -> DecodeBatch:
    """Build a poisoned page pool holding random BF16 K/V for ``seq_lens``.

    ``placement`` is ``"random"`` (pages taken in the order of a seeded
    permutation of the pool) or ``"identity"`` (pages 0, 1, 2, ... in order).
    With ``append=True`` the pool holds tokens ``0 .. L-2`` of each sequence
    and the last token is returned separately in ``k_new``/``v_new``; its slot
    is poisoned until an append writes it.

    ``max_blocks`` is the block-table row length (sequences up to
    ``16 * max_blocks`` tokens; the model's context is 2,048, 128 blocks).

    Draw order (fixed, so a seed reproduces every byte): page permutation, q,
    then for each sequence in batch order its K block then its V block.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = int(seq_lens.shape[0])
    if np.any(seq_lens < 0) or np.any(seq_lens > max_blocks * PAGE_SIZE):
        raise ValueError("seq_lens must lie in [0, %d]" % (max_blocks * PAGE_SIZE))
    rng = np.random.default_rng(seed)
    n_pages = [pages_for(L) for L in seq_lens]
    need = sum(n_pages)
    if need > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {need} pages")
    # the permutation is always drawn, so the values that follow do not depend
    # on the placement: "identity" and "random" hold the same logical cache
    perm = rng.permutation(num_pages).astype(np.int32)
    if placement == "random":
        order = perm
    elif placement == "identity":
        order = np.arange(num_pages, dtype=np.int32)
    else:
        raise ValueError(placement)

    block_tables = np.full((B, max_blocks), -1, dtype=np.int32)
    shape_pool = (num_pages, PAGE_SIZE, NUM_KV_HEADS, HEAD_DIM)
    k_pool = np.full(shape_pool, BF16_NAN, dtype=np.uint16)
    v_pool = np.full(shape_pool, BF16_NAN, dtype=np.uint16)
    q = f32_to_bf16_bits(
        rng.standard_normal((B, NUM_Q_HEADS, HEAD_DIM), dtype=np.float32) * np.float32(q_sigma))
    k_new = np.full((B, NUM_KV_HEADS, HEAD_DIM), BF16_NAN, dtype=np.uint16) if append else None
    v_new = np.full((B, NUM_KV_HEADS, HEAD_DIM), BF16_NAN, dtype=np.uint16) if append else None

    cursor = 0
    for b in range(B):
        L, n = int(seq_lens[b]), n_pages[b]
        pages = order[cursor:cursor + n]
        cursor += n
        block_tables[b, :n] = pages
        if L == 0:
            continue
        tok_shape = (L, NUM_KV_HEADS, HEAD_DIM)
        K = f32_to_bf16_bits(rng.standard_normal(tok_shape, dtype=np.float32))
        V = f32_to_bf16_bits(rng.standard_normal(tok_shape, dtype=np.float32))
        stored = L
        if append:
            k_new[b], v_new[b] = K[L - 1], V[L - 1]
            stored = L - 1
        _place(k_pool, pages, K[:stored])
        _place(v_pool, pages, V[:stored])

    rec = dict(recipe or {})
    rec.update(num_pages=num_pages, placement=placement, q_sigma=q_sigma,
               append=append, seed=_seed_repr(seed))
    return DecodeBatch(name=name, q=q, k_pool=k_pool, v_pool=v_pool,
                       block_tables=block_tables, seq_lens=seq_lens, scale=SCALE,
                       k_new=k_new, v_new=v_new, recipe=rec)


def pack_logical(q, k_rows, v_rows, num_pages: int, seed, *, capacity=None,
                 placement: str = "random", name: str = "packed") -> DecodeBatch:
    """Place caller-given logical K/V rows into a poisoned page pool.

    ``k_rows[b]`` / ``v_rows[b]`` are uint16 ``[T_b][8][64]`` BF16 bits of
    tokens ``0 .. T_b-1``.  ``capacity[b]`` (default ``T_b``) is the sequence
    length to reserve pages for and to report in ``seq_lens``; it may exceed
    ``T_b`` by one to leave the slot of a pending append poisoned.  Pages are
    taken in the order of ``default_rng(seed).permutation(num_pages)`` (or
    0, 1, 2, ... for ``"identity"``), sequence by sequence.
    """
    B = len(k_rows)
    cap = [int(k.shape[0]) for k in k_rows] if capacity is None else [int(c) for c in capacity]
    rng = np.random.default_rng(seed)
    order = (rng.permutation(num_pages) if placement == "random"
             else np.arange(num_pages)).astype(np.int32)
    need = sum(pages_for(c) for c in cap)
    if need > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {need} pages")
    shape_pool = (num_pages, PAGE_SIZE, NUM_KV_HEADS, HEAD_DIM)
    k_pool = np.full(shape_pool, BF16_NAN, dtype=np.uint16)
    v_pool = np.full(shape_pool, BF16_NAN, dtype=np.uint16)
    block_tables = np.full((B, MAX_BLOCKS), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        if not 0 <= k_rows[b].shape[0] <= cap[b] <= MAX_CONTEXT:
            raise ValueError("rows must fit the reserved capacity")
        n = pages_for(cap[b])
        pages = order[cursor:cursor + n]
        cursor += n
        block_tables[b, :n] = pages
        _place(k_pool, pages, np.asarray(k_rows[b], dtype=np.uint16))
        _place(v_pool, pages, np.asarray(v_rows[b], dtype=np.uint16))
    return DecodeBatch(name=name, q=np.asarray(q, dtype=np.uint16), k_pool=k_pool,
                       v_pool=v_pool, block_tables=block_tables,
                       seq_lens=np.asarray(cap, dtype=np.int32), scale=SCALE,
                       recipe={"num_pages": num_pages, "placement": placement,
                               "seed": _seed_repr(seed)})


def random_rows(rng, T: int, sigma: float = 1.0) -> np.ndarray:
    """``[T][8][64]`` BF16 bits of N(0, sigma^2) values."""
    return f32_to_bf16_bits(
        rng.standard_normal((T, NUM_KV_HEADS, HEAD_DIM), dtype=np.float32) * np.float32(sigma))


def random_q(rng, B: int, sigma: float = 1.0) -> np.ndarray:
    """``[B][32][64]`` BF16 bits of N(0, sigma^2) values."""
    return f32_to_bf16_bits(
        rng.standard_normal((B, NUM_Q_HEADS, HEAD_DIM), dtype=np.float32) * np.float32(sigma))


def _place(pool: np.ndarray, pages: np.ndarray, rows: np.ndarray) -> None:
    """Store token rows ``[T][8][64]`` into consecutive logical pages."""
    T = rows.shape[0]
    full = T // PAGE_SIZE
    if full:
        pool[pages[:full]] = rows[:full * PAGE_SIZE].reshape(full, PAGE_SIZE, NUM_KV_HEADS, HEAD_DIM)
    tail = T - full * PAGE_SIZE
    if tail:
        pool[pages[full], :tail] = rows[full * PAGE_SIZE:]


def _seed_repr(seed):
    return list(seed) if isinstance(seed, (list, tuple)) else seed


# ---------------------------------------------------------------------------
# The workloads: Llama-3.2-1B decode-step shapes (synthetic stand-ins; the
# pages name no public benchmark or dataset)
# ---------------------------------------------------------------------------
WORKLOADS = {
    1: "single sequence, seq_len 37 (pages 16+16+5), 64-page pool",
    2: "batch 8, seq_len uniform in [1, 2048], 4096-page (128 MiB) pool",
    3: "16 layers, batch 64, seq_len uniform in [16, 2048], q sigma 0.5, append then attend per layer",
    4: "batch 256, every seq_len 2048 (1 GiB of K/V), pool of exactly 32768 pages",
    5: "batch 512, seq_len Zipf(1.1) clipped to [1, 2048], append then attend, 10% poison slack",
    6: "batch 512, seq_len Zipf(1.1) truncated to [1, 2048] (the law renormalised on 1..2048), "
       "append then attend, 10% poison slack",
}
NUM_LAYERS_W3 = 16
POOL_PAGES_W3 = 8192


def workload_seq_lens(index: int, seed: Optional[int] = None) -> np.ndarray:
    """Sequence lengths of workload ``index`` (drawn from their own stream)."""
    seed = index if seed is None else seed
    rng = np.random.default_rng([seed, 0])
    if index == 1:
        return np.array([37], dtype=np.int32)
    if index == 2:
        return rng.integers(1, MAX_CONTEXT + 1, size=8).astype(np.int32)
    if index == 3:
        return rng.integers(16, MAX_CONTEXT + 1, size=64).astype(np.int32)
    if index == 4:
        return np.full(256, MAX_CONTEXT, dtype=np.int32)
    if index == 5:
        return np.clip(rng.zipf(1.1, size=512), 1, MAX_CONTEXT).astype(np.int32)
    if index == 6:
        # the other reading of "Zipf (s=1.1, clipped to [1, 2048])": P(L = k) proportional
        # to k^-1.1 on 1..2048 only (mean about 179, against about 1000 for the clipped draw)
        k = np.arange(1, MAX_CONTEXT + 1, dtype=np.float64)
        p = k ** -1.1
        return rng.choice(MAX_CONTEXT, size=512, p=p / p.sum()).astype(np.int32) + 1
    raise ValueError(index)


def make_workload(index: int, seed: Optional[int] = None, layer: int = 0,
                  placement: str = "random", append: Optional[bool] = None) -> DecodeBatch:
    """Inputs of workload ``index`` (for workload 3: of layer ``layer``).

    ``append`` overrides whether the last token of every sequence is held
    back for an append (default: workloads 3, 5 and 6 append, the others not).
    """
    seed = index if seed is None else seed
    lens = workload_seq_lens(index, seed)
    name = f"w{index}"
    recipe = {"workload": WORKLOADS[index]}
    app = (index in (3, 5, 6)) if append is None else bool(append)
    if index == 1:
        return make_batch(lens, 64, [seed, 1], name=name, recipe=recipe, placement=placement,
                          append=app)
    if index == 2:
        return make_batch(lens, 4096, [seed, 1], name=name, recipe=recipe, placement=placement,
                          append=app)
    if index == 3:
        if not 0 <= layer < NUM_LAYERS_W3:
            raise ValueError(layer)
        return make_batch(lens, POOL_PAGES_W3, [seed, 1, layer], q_sigma=0.5, append=app,
                          name=f"{name}_layer{layer}", recipe=dict(recipe, layer=layer),
                          placement=placement)
    if index == 4:
        return make_batch(lens, 256 * MAX_BLOCKS, [seed, 1], name=name, recipe=recipe,
                          placement=placement, append=app)
    if index in (5, 6):
        need = int(sum(pages_for(L) for L in lens))
        pool = need + (need + 9) // 10
        return make_batch(lens, pool, [seed, 1], append=app, name=name, recipe=recipe,
                          placement=placement)
    raise ValueError(index)


@dataclass
class Q8Batch:
    """One layer's decode-step inputs over INT8 (or INT4) pages.

    Codes are int8 ``[num_pages][8][16][64]`` (per page, each KV head's 16
    token rows contiguous), or for ``nbits == 4`` uint8 ``[num_pages][8][16][32]``
    (two codes per byte, each stored as code + 8, dim 2j in the low nibble);
    scales float32 ``[num_pages][8][2][16]`` (per page and KV head: 16 K
    scales, 16 V scales).
    """

    name: str
    q: np.ndarray               # uint16 [B][32][64]
    k_codes: np.ndarray         # int8   [num_pages][8][16][64]
    v_codes: np.ndarray
    kv_scales: np.ndarray       # float32 [num_pages][8][2][16]
    block_tables: np.ndarray    # int32  [B][128]
    seq_lens: np.ndarray        # int32  [B]
    scale: float = SCALE
    k_new: Optional[np.ndarray] = None   # uint16 [B][8][64] BF16 rows when the step appends
    v_new: Optional[np.ndarray] = None
    recipe: dict = field(default_factory=dict)
    nbits: int = 8              # 4: codes are uint8 [num_pages][8][16][32], two per byte

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_codes.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0


Q8_CODE_SIGMA = 45.0            # codes of N(0, 1) rows of 64 values: amax ~ 2.8 -> 127
Q8_SCALE_RANGE = (0.018, 0.028)
Q4_CODE_SIGMA = 2.5             # the same rows at 4 bits: amax ~ 2.8 -> 7
Q4_SCALE_RANGE = (0.32, 0.5)


def make_q8_batch(seq_lens, num_pages: int, seed, *, append: bool = False,
                  placement: str = "random", name: str = "q8",
                  max_blocks: int = MAX_BLOCKS, nbits: int = 8) -> Q8Batch:
    """Random INT8 pages for ``seq_lens``, shaped like quantised N(0, 1) rows.

    Every stored (token, head) row gets codes round(N(0, 45)) clipped to
    [-127, 127] with one code set to +-127 (its largest magnitude), and a
    scale uniform in [0.018, 0.028].  Slots that hold no token have random
    codes and a NaN scale (poison).  With ``append=True`` the slot of token
    L-1 stays poisoned and BF16 N(0, 1) rows for it come in ``k_new``/``v_new``.

    ``max_blocks`` is the block-table row length, as in ``make_batch``.

    ``nbits=4`` draws INT4 pages instead: codes ``round(N(0, 2.5))`` clipped to
    [-7, 7] with one +-7 per row, scales uniform in [0.32, 0.5], stored two
    per byte as code + 8 (dim 2j in the low nibble of byte j); unused slots
    hold random bytes and NaN scales.

    Draw order: page permutation, q, poison codes, then per sequence its K
    codes, V codes, K scales, V scales (and, appending, its new K and V rows).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = int(seq_lens.shape[0])
    if np.any(seq_lens < 0) or np.any(seq_lens > max_blocks * PAGE_SIZE):
        raise ValueError("seq_lens must lie in [0, %d]" % (max_blocks * PAGE_SIZE))
    rng = np.random.default_rng(seed)
    n_pages = [pages_for(L) for L in seq_lens]
    if sum(n_pages) > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {sum(n_pages)} pages")
    perm = rng.permutation(num_pages).astype(np.int32)
    order = perm if placement == "random" else np.arange(num_pages, dtype=np.int32)
    if placement not in ("random", "identity"):
        raise ValueError(placement)
    if nbits not in (8, 4):
        raise ValueError("nbits must be 8 or 4")
    q = f32_to_bf16_bits(rng.standard_normal((B, NUM_Q_HEADS, HEAD_DIM), dtype=np.float32))
    if nbits == 8:
        shape = (num_pages, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM)
        k_codes = rng.integers(-128, 128, size=shape, dtype=np.int8)
        v_codes = rng.integers(-128, 128, size=shape, dtype=np.int8)
        sigma, qmax, scale_range = Q8_CODE_SIGMA, 127, Q8_SCALE_RANGE
    else:
        shape = (num_pages, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM // 2)
        k_codes = rng.integers(0, 256, size=shape, dtype=np.uint8)
        v_codes = rng.integers(0, 256, size=shape, dtype=np.uint8)
        sigma, qmax, scale_range = Q4_CODE_SIGMA, 7, Q4_SCALE_RANGE
    kv_scales = np.full((num_pages, NUM_KV_HEADS, 2, PAGE_SIZE), np.nan, dtype=np.float32)
    k_new = np.zeros((B, NUM_KV_HEADS, HEAD_DIM), np.uint16) if append else None
    v_new = np.zeros((B, NUM_KV_HEADS, HEAD_DIM), np.uint16) if append else None
    block_tables = np.full((B, max_blocks), -1, dtype=np.int32)

    def codes(T):
        c = np.clip(np.rint(rng.standard_normal((T, NUM_KV_HEADS, HEAD_DIM), dtype=np.float32)
                            * np.float32(sigma)), -qmax, qmax).astype(np.int8)
        pick = rng.integers(0, HEAD_DIM, size=(T, NUM_KV_HEADS))
        sign = rng.choice(np.array([-qmax, qmax], np.int8), size=(T, NUM_KV_HEADS))
        np.put_along_axis(c, pick[..., None], sign[..., None], axis=-1)
        if nbits == 4:                 # two per byte, offset by 8
            u = (c.astype(np.int16) + 8).astype(np.uint8)
            c = (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)
        return c

    cursor = 0
    for b in range(B):
        L, n = int(seq_lens[b]), n_pages[b]
        pages = order[cursor:cursor + n]
        cursor += n
        block_tables[b, :n] = pages
        if L == 0:
            continue
        kc, vc = codes(L), codes(L)
        ks = rng.uniform(*scale_range, size=(L, NUM_KV_HEADS)).astype(np.float32)
        vs = rng.uniform(*scale_range, size=(L, NUM_KV_HEADS)).astype(np.float32)
        stored = L - 1 if append else L
        for t in range(stored):
            page, slot = pages[t // PAGE_SIZE], t % PAGE_SIZE
            k_codes[page, :, slot] = kc[t]
            v_codes[page, :, slot] = vc[t]
            kv_scales[page, :, 0, slot] = ks[t]
            kv_scales[page, :, 1, slot] = vs[t]
        if append:
            k_new[b] = f32_to_bf16_bits(rng.standard_normal((NUM_KV_HEADS, HEAD_DIM), dtype=np.float32))
            v_new[b] = f32_to_bf16_bits(rng.standard_normal((NUM_KV_HEADS, HEAD_DIM), dtype=np.float32))
    recipe = dict(num_pages=num_pages, placement=placement, append=append, seed=_seed_repr(seed),
                  code_sigma=sigma, scale_range=scale_range, nbits=nbits)
    return Q8Batch(name=name, q=q, k_codes=k_codes, v_codes=v_codes, kv_scales=kv_scales,
                   block_tables=block_tables, seq_lens=seq_lens, k_new=k_new, v_new=v_new,
                   recipe=recipe, nbits=nbits)


# ---------------------------------------------------------------------------
# Sharp-score inputs: later keys score far above earlier ones, so a running
# maximum taken page by page must be raised (and what was summed under the old
# one rescaled) long after the first page, and split maxima lie far apart.
# Each mode only shapes the key rows (or the scale); the values stay N(0, 1).
# ---------------------------------------------------------------------------
SHARP_MODES = ("ramp_up", "ramp_down", "tail_max", "mid_max", "scale2")
SHARP_SCALE2 = 2.0              # the scale of mode "scale2" (scores of sigma 16)
SPIKE_GAIN = 1.5                # a spike key is 1.5 x the sum of its group's query rows


def bf16_bits_to_f32(bits) -> np.ndarray:
    """BF16 bit patterns -> float32 values (the upper half of a binary32 word)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_sharp_batch(seq_lens, num_pages: int, seed, mode: str, *, append: bool = False,
                     placement: str = "random", max_blocks: int = MAX_BLOCKS) -> DecodeBatch:
    """Inputs whose scores rise far past the running maximum after the first page.

    Modes (K of token ``t`` of a sequence of length ``L``; q, V and the other
    keys N(0, 1); scale 1/8 unless stated):

    * ``ramp_up``: ``K[t]`` scaled by ``0.25 + 5.75 t / (L - 1)``: every later
      page's scores spread wider than the earlier ones' (standard deviation
      0.25 on the first page, 6 at the end);
    * ``ramp_down``: the reverse ramp (the largest scores on the first pages);
    * ``tail_max``: the last token's key of each KV head ``g`` is 1.5 x the sum
      of the query rows of heads ``4g .. 4g+3``, its score about 12 above the
      others.  It sits in the last page, which ends mid-page for most
      lengths; with ``append=True`` it is the appended token;
    * ``mid_max``: the same spike on token ``L // 2``;
    * ``scale2``: no shaping; the batch's scale is 2.0 (score sigma 16).

    Draw order: as ``make_batch`` (page permutation, q, then per sequence its
    K block then its V block).
    """
    if mode not in SHARP_MODES:
        raise ValueError(mode)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = int(seq_lens.shape[0])
    if np.any(seq_lens < 0) or np.any(seq_lens > max_blocks * PAGE_SIZE):
        raise ValueError("seq_lens must lie in [0, %d]" % (max_blocks * PAGE_SIZE))
    rng = np.random.default_rng(seed)
    n_pages = [pages_for(L) for L in seq_lens]
    if sum(n_pages) > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {sum(n_pages)} pages")
    perm = rng.permutation(num_pages).astype(np.int32)
    if placement not in ("random", "identity"):
        raise ValueError(placement)
    order = perm if placement == "random" else np.arange(num_pages, dtype=np.int32)
    q = f32_to_bf16_bits(rng.standard_normal((B, NUM_Q_HEADS, HEAD_DIM), dtype=np.float32))
    qf = bf16_bits_to_f32(q)
    group = NUM_Q_HEADS // NUM_KV_HEADS
    shape_pool = (num_pages, PAGE_SIZE, NUM_KV_HEADS, HEAD_DIM)
    k_pool = np.full(shape_pool, BF16_NAN, dtype=np.uint16)
    v_pool = np.full(shape_pool, BF16_NAN, dtype=np.uint16)
    block_tables = np.full((B, max_blocks), -1, dtype=np.int32)
    k_new = np.full((B, NUM_KV_HEADS, HEAD_DIM), BF16_NAN, dtype=np.uint16) if append else None
    v_new = np.full((B, NUM_KV_HEADS, HEAD_DIM), BF16_NAN, dtype=np.uint16) if append else None
    cursor = 0
    for b in range(B):
        L, n = int(seq_lens[b]), n_pages[b]
        pages = order[cursor:cursor + n]
        cursor += n
        block_tables[b, :n] = pages
        if L == 0:
            continue
        K = rng.standard_normal((L, NUM_KV_HEADS, HEAD_DIM), dtype=np.float32)
        V = f32_to_bf16_bits(rng.standard_normal((L, NUM_KV_HEADS, HEAD_DIM), dtype=np.float32))
        pos = np.arange(L, dtype=np.float32) / np.float32(max(L - 1, 1))
        if mode == "ramp_up":
            K *= (np.float32(0.25) + np.float32(5.75) * pos)[:, None, None]
        elif mode == "ramp_down":
            K *= (np.float32(6.0) - np.float32(5.75) * pos)[:, None, None]
        elif mode in ("tail_max", "mid_max"):
            t = L - 1 if mode == "tail_max" else L // 2
            spike = qf[b].reshape(NUM_KV_HEADS, group, HEAD_DIM).sum(axis=1)
            K[t] = np.float32(SPIKE_GAIN) * spike
        K = f32_to_bf16_bits(K)
        stored = L
        if append:
            k_new[b], v_new[b] = K[L - 1], V[L - 1]
            stored = L - 1
        _place(k_pool, pages, K[:stored])
        _place(v_pool, pages, V[:stored])
    recipe = dict(num_pages=num_pages, placement=placement, append=append,
                  seed=_seed_repr(seed), sharp_mode=mode)
    return DecodeBatch(name=f"sharp_{mode}", q=q, k_pool=k_pool, v_pool=v_pool,
                       block_tables=block_tables, seq_lens=seq_lens,
                       scale=SHARP_SCALE2 if mode == "scale2" else SCALE,
                       k_new=k_new, v_new=v_new, recipe=recipe)


def logical_rows(pool: np.ndarray, block_table_row, count: int) -> np.ndarray:
    """Tokens ``0 .. count-1`` of one sequence as ``[count][8][64]`` BF16 bits
    (the page pool read back through the block table; layout only)."""
    n = pages_for(count)
    return np.ascontiguousarray(pool[np.asarray(block_table_row[:n])]
                                .reshape(-1, NUM_KV_HEADS, HEAD_DIM)[:count])


def poison_summary(batch: DecodeBatch) -> dict:
    """Counts of poisoned pool rows and block-table entries (for reports)."""
    nan_rows = int(np.count_nonzero(batch.k_pool[..., 0, 0] == BF16_NAN))
    return {"nan_slots": nan_rows, "unused_bt": int(np.count_nonzero(batch.block_tables < 0))}


def rope_table(max_pos: int = MAX_CONTEXT, head_dim: int = HEAD_DIM, base: float = 500000.0):
    """Float32 cos and sin ``[max_pos][head_dim/2]`` for rotary embeddings.

    Frequency ``i`` is ``base ** (-2 i / head_dim)`` (500000 is the Llama-3
    base); angles are formed and evaluated in float64, then rounded to float32.
    Callers that use another frequency schedule pass their own table.
    """
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
