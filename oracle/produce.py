"""Float oracle of the synthetic draft producer of the two-batch schedule.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the page "MineDraft: A Framework for Batch Parallel Speculative
Decoding", section 2 (the core mechanism, alternation between batches): two
batches are kept; while the target model verifies the drafts of one, the
draft model drafts the other, and the roles swap at the end of every step.
On one GPU the verify step of one batch runs on one stream while a producer
of the other batch's drafts runs on a second stream.

The pages give no drafter, so the producer is defined here.  For every
batch row b and draft position j < K:

  * delta(b, j, v) = ((h >> 5) - 1024) * 2^-9, where h is the 16-bit half
    (v & 1: 0 = low, 1 = high) of word (v & 7) >> 1 of Philox4x32-10 at
    counter (v >> 3, b, j, 3) with key (seed low, seed high).  delta is
    uniform on the 2048 points of a 1/512 grid in [-2, 2) and exact in
    float32.
  * draft[b, j, v] = round(float32(target[b, j, v]) + delta): one float32
    addition (round to nearest even), then for bf16 logits the float32 ->
    bf16 conversion with round to nearest even (NaN stays NaN).
  * token[b, j] = the lowest id holding the largest draft logit of the row (a
    greedy drafter); -1 when the draft row holds a NaN.
"""

import numpy as np

from .philox import philox4x32_10, seed_key


def deltas(seed, b, j, V):
    """delta(b, j, v) for v = 0..V-1 as float32."""
    v = np.arange(V, dtype=np.uint64)
    ctr = np.stack([v >> np.uint64(3), np.full(V, b, np.uint64), np.full(V, j, np.uint64),
                    np.full(V, 3, np.uint64)], axis=-1)
    words = philox4x32_10(ctr, seed_key(seed))  # [V, 4]
    w = words[np.arange(V), ((v & np.uint64(7)) >> np.uint64(1)).astype(np.int64)].astype(np.uint64)
    h = np.where((v & np.uint64(1)) == 0, w & np.uint64(0xFFFF), w >> np.uint64(16))
    return ((h >> np.uint64(5)).astype(np.int64) - 1024).astype(np.float32) * np.float32(2.0 ** -9)


def f32_to_bf16_rne(x):
    """float32 -> bf16 bit patterns, round to nearest even; NaN -> 0x7FC0."""
    x = np.asarray(x, dtype=np.float32)
    shape = x.shape
    x = x.reshape(-1)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = r.astype(np.uint16)
    out[np.isnan(x)] = np.uint16(0x7FC0)
    return out.reshape(shape)


def bf16_to_f32(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def produce_drafts(target, K, seed):
    """target [B, P >= K, V]: float32 logits, or uint16 bf16 bit patterns.
    Returns (draft [B, K, V] of the same kind, tokens [B, K] int64)."""
    target = np.asarray(target)
    bf16 = target.dtype == np.uint16
    B, _, V = target.shape
    draft = np.empty((B, K, V), dtype=target.dtype)
    tokens = np.empty((B, K), dtype=np.int64)
    for b in range(B):
        for j in range(K):
            t = bf16_to_f32(target[b, j]) if bf16 else target[b, j].astype(np.float32)
            s = t + deltas(seed, b, j, V)  # one float32 addition per element
            if bf16:
                draft[b, j] = f32_to_bf16_rne(s)
                d = bf16_to_f32(draft[b, j])
            else:
                draft[b, j] = s
                d = s
            tokens[b, j] = -1 if np.isnan(d).any() else int(np.argmax(d))
    return draft, tokens
