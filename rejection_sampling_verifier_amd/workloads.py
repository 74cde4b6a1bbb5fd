"""Seeded synthetic inputs for the verify step.

This module is shared by the tests, the benchmark and the smoke check.  It
holds input generation only -- none of the verify method's arithmetic -- and
imports neither the oracle nor the HIP library.

The five workloads stand in for the setup on the page "Speculative Decoding
للمحترف: ضاعف سرعة Llama 70B لـ 2.4x بدون فقد token واحد" (section "كود شغّال
على vLLM": K = 5 drafted tokens, temperature 0.7, top_p 0.9; section
"الأرقام": batch 1) with the Llama-3 vocabulary size V = 128256, plus a
batched, a ragged-batch (page "HiSpec", section 2: per-sequence accepted
lengths in one batch) and a filtered variant.  No model, dataset or checkpoint
is involved: logits are random with the stated distributions.

Recipe (all draws from numpy PCG64 seeded by SeedSequence([0x5EED0000 + cfg,
step])):
  * target logits i.i.d. N(0, 3^2) over [B, K+1, V];
  * draft logits = target[:, :K] + N(0, sigma^2), sigma per workload;
  * bfloat16 workloads round float32 values to bfloat16 by
    round-to-nearest-even on the bit pattern (checked against torch's cast);
  * drafted tokens are exact samples of softmax(draft / T) by the Gumbel-max
    construction: argmax(draft/T + G) with G standard Gumbel noise.  For the
    filtered workload the Gumbel-max runs over the draft's 64 largest logits
    only, which at these logit scales lie inside the draft's 0.9-nucleus, so
    every drafted token has non-zero filtered draft probability;
  * ragged workload: per-row draft length uniform in 1..K; 4 distinct ids per
    (row, position) get +8; padded positions (target position > L, draft
    position >= L) are filled with NaN and padded drafted ids with -1, so that
    reading them would be detected;
  * the verify seed for step s of workload c is (c << 32) | s.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

V_LLAMA3 = 128256


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    B: int
    K: int
    V: int
    dtype: str            # "f32" or "bf16"
    temperature: float
    top_p: float
    sigma: tuple          # draft noise: (lo, hi) uniform per row, or (s, s)
    ragged: bool = False
    spikes: int = 0
    steps: int = 1        # verify steps the workload is defined over


CONFIGS = {
    0: Workload(0, "tiny B=1 K=5 V=1000 fp32 T=1", 1, 5, 1000, "f32", 1.0, 1.0, (1.0, 1.0), steps=1000),
    1: Workload(1, "single-stream B=1 K=5 V=128256 fp32 T=0.7", 1, 5, V_LLAMA3, "f32", 0.7, 1.0,
                (1.0, 1.0), steps=10000),
    2: Workload(2, "batched B=64 K=5 V=128256 bf16 T=0.7", 64, 5, V_LLAMA3, "bf16", 0.7, 1.0,
                (0.25, 2.0), steps=250),
    3: Workload(3, "ragged B=256 K=8 V=128256 bf16 T=1", 256, 8, V_LLAMA3, "bf16", 1.0, 1.0,
                (1.0, 1.0), ragged=True, spikes=4, steps=120),
    4: Workload(4, "filtered B=64 K=5 V=128256 bf16 T=0.7 top_p=0.9", 64, 5, V_LLAMA3, "bf16", 0.7,
                0.9, (0.25, 2.0), steps=250),
}

NAN_BF16 = np.uint16(0x7FC0)


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns, round to nearest even; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = rounded.astype(np.uint16)
    out[np.isnan(x)] = NAN_BF16
    return out


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    workload: Workload
    step: int
    target: np.ndarray          # [B, K+1, V] float32, or uint16 bfloat16 bits
    draft: np.ndarray           # [B, K, V]   same dtype as target
    draft_tokens: np.ndarray    # [B, K] int32
    draft_len: Optional[np.ndarray]  # [B] int32, or None for "all K"
    temperature: np.float32
    top_p: np.float32
    seed: int

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def K(self):
        return self.target.shape[1] - 1

    @property
    def V(self):
        return self.target.shape[2]

    @property
    def elem_bytes(self):
        return 2 if self.target.dtype == np.uint16 else 4

    def lengths(self):
        return np.full(self.B, self.K, np.int64) if self.draft_len is None else self.draft_len.astype(np.int64)

    def logical_bytes(self):
        """Bytes of every needed logit row read once: sum_b (2 L_b + 1) V e."""
        return int(np.sum(2 * self.lengths() + 1)) * self.V * self.elem_bytes

    def positions(self):
        """Verified draft positions: sum_b L_b."""
        return int(np.sum(self.lengths()))


def _rng(cfg, step):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x5EED0000 + cfg, step])))


def _nucleus_gumbel(rng, logits, temperature, top_p, cand=4096):
    """Sample of the top-p-filtered softmax(logits / T) per row: tokens sorted
    by probability (descending, ties by the lower id), the shortest prefix
    whose running mass reaches top_p kept, then Gumbel-max over the kept ids
    (an exact sample of the renormalised prefix).  The prefix is looked for
    among the `cand` largest logits first, the whole row when it lies deeper.
    logits: [..., V] float32."""
    flat = logits.reshape(-1, logits.shape[-1])
    out = np.empty(flat.shape[0], np.int64)
    for i, row in enumerate(flat):
        z = row.astype(np.float64) / temperature
        e = np.exp(z - np.max(z))
        S = float(np.sum(e))
        V = row.size
        ids = np.arange(V) if V <= cand else np.sort(np.argpartition(-z, cand - 1)[:cand])
        order = ids[np.argsort(-e[ids], kind="stable")]
        run = np.cumsum(e[order]) / S
        hit = np.nonzero(run >= top_p)[0]
        if hit.size == 0 and ids.size < V:
            order = np.argsort(-e, kind="stable")
            run = np.cumsum(e[order]) / S
            hit = np.nonzero(run >= top_p)[0]
        kept = order[: int(hit[0]) + 1] if hit.size else order
        g = -np.log(-np.log(rng.random(kept.size)))
        out[i] = kept[int(np.argmax(z[kept] + g))]
    return out.reshape(logits.shape[:-1])


def _gumbel_argmax(rng, logits, temperature):
    """Exact sample of softmax(logits / T) by Gumbel-max.  logits: [..., V]
    float32."""
    flat = logits.reshape(-1, logits.shape[-1])
    out = np.empty(flat.shape[0], np.int64)
    for i, row in enumerate(flat):
        g = -np.log(-np.log(rng.random(row.size)))
        out[i] = int(np.argmax(row.astype(np.float64) / temperature + g))
    return out.reshape(logits.shape[:-1])


def make_inputs(cfg, step=0, *, B=None, K=None, V=None, dtype=None, temperature=None,
                top_p=None):
    """Generate step `step` of workload `cfg`.  Keyword overrides shrink or
    reshape the workload for tests while keeping its value distribution."""
    w = CONFIGS[cfg]
    B = w.B if B is None else B
    K = w.K if K is None else K
    V = w.V if V is None else V
    dtype = w.dtype if dtype is None else dtype
    T = np.float32(w.temperature if temperature is None else temperature)
    tp = np.float32(w.top_p if top_p is None else top_p)
    rng = _rng(cfg, step)

    target = rng.standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(3.0)
    if w.spikes:
        for b in range(B):
            for j in range(K + 1):
                target[b, j, rng.choice(V, w.spikes, replace=False)] += np.float32(8.0)
    lo, hi = w.sigma
    sig = rng.uniform(lo, hi, size=B).astype(np.float32) if hi > lo else np.full(B, lo, np.float32)
    draft = target[:, :K] + rng.standard_normal((B, K, V), dtype=np.float32) * sig[:, None, None]

    if dtype == "bf16":
        target_s = f32_to_bf16_bits(target)
        draft_s = f32_to_bf16_bits(draft)
        draft_vals = bf16_bits_to_f32(draft_s)
    else:
        target_s, draft_s, draft_vals = target, draft.astype(np.float32), draft.astype(np.float32)

    if tp < 1.0:
        tokens = _nucleus_gumbel(rng, draft_vals, float(T), float(tp)).astype(np.int32)
    else:
        tokens = _gumbel_argmax(rng, draft_vals, float(T)).astype(np.int32)

    draft_len = None
    if w.ragged:
        draft_len = rng.integers(1, K + 1, size=B).astype(np.int32)
        for b in range(B):
            L = int(draft_len[b])
            if dtype == "bf16":
                target_s[b, L + 1:] = NAN_BF16
                draft_s[b, L:] = NAN_BF16
            else:
                target_s[b, L + 1:] = np.nan
                draft_s[b, L:] = np.nan
            tokens[b, L:] = -1
    seed = (cfg << 32) | step
    return Inputs(w, step, np.ascontiguousarray(target_s), np.ascontiguousarray(draft_s),
                  tokens, draft_len, T, tp, seed)


def synthetic(B, K, V, *, dtype="f32", temperature=1.0, top_p=1.0, sigma=1.0, scale=3.0,
              draft_len=None, seed=0, gen_seed=0):
    """Free-form inputs of the same recipe, for edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x5EED1000, gen_seed])))
    target = rng.standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(scale)
    draft = target[:, :K] + rng.standard_normal((B, K, V), dtype=np.float32) * np.float32(sigma)
    if dtype == "bf16":
        ts, ds = f32_to_bf16_bits(target), f32_to_bf16_bits(draft)
        dv = bf16_bits_to_f32(ds)
    else:
        ts, ds, dv = target, draft.astype(np.float32), draft.astype(np.float32)
    T = np.float32(temperature)
    tokens = _gumbel_argmax(rng, dv, float(T)).astype(np.int32) if K > 0 else np.zeros((B, 0), np.int32)
    dl = None if draft_len is None else np.asarray(draft_len, np.int32)
    return Inputs(CONFIGS[0], 0, np.ascontiguousarray(ts), np.ascontiguousarray(ds), tokens, dl, T,
                  np.float32(top_p), int(seed))


@dataclass
class HispecInputs:
    final: np.ndarray        # [B, K+2, V] float32 or bfloat16 bits
    inter: np.ndarray        # [B, K+1, V]
    draft: np.ndarray        # [B, K, V]
    draft_tokens: np.ndarray # [B, K] int32
    draft_len: Optional[np.ndarray]
    temperature: np.float32
    top_p: np.float32
    seed: int


def make_hispec_inputs(B, K, V, *, dtype="bf16", step=0, temperature=0.7, top_p=1.0, sig_inter=0.7,
                       sig_draft=1.0, ragged=False):
    """Three exit layers of one early-exit model (page "HiSpec", section 2):
    final-layer logits N(0, 3^2) over [B, K+2, V]; intermediate layer = final
    + N(0, sig_inter^2) at positions 0..K; draft layer = intermediate +
    N(0, sig_draft^2) at positions 0..K-1; drafted tokens sampled from the
    draft layer's softmax at the temperature (Gumbel-max); with `ragged`,
    per-row draft lengths uniform in 0..K.  Seeded by SeedSequence([0x5EED2000,
    step])."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x5EED2000, step])))
    f = rng.standard_normal((B, K + 2, V), dtype=np.float32) * np.float32(3.0)
    i = f[:, : K + 1] + rng.standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(sig_inter)
    d = i[:, :K] + rng.standard_normal((B, K, V), dtype=np.float32) * np.float32(sig_draft)
    if dtype == "bf16":
        f, i, d = f32_to_bf16_bits(f), f32_to_bf16_bits(i), f32_to_bf16_bits(d)
        dv = bf16_bits_to_f32(d)
    else:
        dv = d
    T = np.float32(temperature)
    tokens = _gumbel_argmax(rng, dv, float(T)).astype(np.int32)
    dl = rng.integers(0, K + 1, size=B).astype(np.int32) if ragged else None
    return HispecInputs(np.ascontiguousarray(f), np.ascontiguousarray(i), np.ascontiguousarray(d), tokens, dl, T,
                        np.float32(top_p), (0x5EED2 << 32) | step)
