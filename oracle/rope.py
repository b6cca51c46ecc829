"""Reference rotary position embedding (RoPE) of the new token, fused with the append.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name RoPE as a step of the model ("6 Hours of YouTube and 85
handtyped pages of notes on LLM Inference", build series part 4 and
features completed so far: RoPE in the prefill path; decode appends the new
token's K/V at its absolute RoPE position) but print no formula.  Reading
taken, the one of the checkpoint the engine loads (Hugging Face Llama 3.2):
rotate-half pairing, i.e. dims i and i + D/2 form one rotation pair with
angle ``pos * inv_freq[i]``:

    out[i]       = x[i] * cos - x[i + D/2] * sin
    out[i + D/2] = x[i + D/2] * cos + x[i] * sin

The angles enter as a caller-given table of float32 cos and sin values per
position and frequency, so the frequency schedule (base, scaling) is the
caller's choice.  Every product and sum is rounded to float32 separately
(no fused multiply-add) and the result is rounded to BF16 to nearest-even:
the rounding of the BF16 code is a decision both sides must take the same
way, in float32.
"""

from __future__ import annotations

import numpy as np

from .paged_decode import bf16_bits_to_f64


def f32_to_bf16_bits_rne(x) -> np.ndarray:
    """Round float32 values to BF16 bits, nearest with ties to even.

    Written from the definition: the two BF16 neighbours of x are x with its
    low 16 bits cleared (towards zero) and the next BF16 code away from zero;
    pick the nearer, and on a tie the one whose last kept bit is 0.
    Finite inputs only.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    down = (u >> 16).astype(np.uint64)                 # truncated code
    half = 0x8000
    up = (low > half) | ((low == half) & ((down & 1) == 1))
    return (down + up.astype(np.uint64)).astype(np.uint16)


def rope_rotate_f32(x_bits, cos_row, sin_row) -> np.ndarray:
    """Rotate one or more head vectors (BF16 bits ``[..., D]``); float32 result."""
    x = bf16_bits_to_f64(x_bits).astype(np.float32)
    c = np.asarray(cos_row, dtype=np.float32)
    s = np.asarray(sin_row, dtype=np.float32)
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    with np.errstate(over="ignore"):
        a = (x1 * c).astype(np.float32) - (x2 * s).astype(np.float32)
        b = (x2 * c).astype(np.float32) + (x1 * s).astype(np.float32)
    return np.concatenate([a.astype(np.float32), b.astype(np.float32)], axis=-1)


def rope_new_token(q_bits, k_new_bits, seq_lens, rope_cos, rope_sin):
    """RoPE of each sequence's new query and key at position ``seq_lens[b] - 1``.

    ``rope_cos``/``rope_sin``: float32 ``[max_pos][D/2]``.  Returns BF16 bits
    ``(q_rot [B][Hq][D], k_rot [B][Hkv][D])``; idle slots (L == 0) keep their
    inputs unchanged.
    """
    q_out = np.array(q_bits, dtype=np.uint16, copy=True)
    k_out = np.array(k_new_bits, dtype=np.uint16, copy=True)
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        if L == 0:
            continue
        pos = L - 1
        q_out[b] = f32_to_bf16_bits_rne(rope_rotate_f32(q_bits[b], rope_cos[pos], rope_sin[pos]))
        k_out[b] = f32_to_bf16_bits_rne(rope_rotate_f32(k_new_bits[b], rope_cos[pos], rope_sin[pos]))
    return q_out, k_out
