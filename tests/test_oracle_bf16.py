"""Pins of the oracle's bfloat16 ingest (`oracle.widen_bf16` and the uint16
branch of the oracle's input widening) to facts fixed outside the oracle.

Every bfloat16 call of the verify, SMC, two-stage and greedy oracles widens
its logits through this one function, so it is pinned on all 65,536 bit
patterns against two independent definitions: torch's bfloat16 -> float32
cast, and the IEEE-754 binary16-brain field formula (sign, 8-bit biased
exponent, 7-bit fraction) evaluated with Python integers.  Then the whole
verify oracle is run on bfloat16 bit patterns: a worked example whose
probabilities are written out by hand from the decoded values, and the law of
the emitted token (the exactness claim of the page "Speculative Decoding
للمحترف: ضاعف سرعة Llama 70B لـ 2.4x بدون فقد token واحد", section "التعريف
الرياضي من Leviathan et al.") over many independent rows.
"""

import math

import numpy as np
import scipy.stats
import torch

import oracle
from oracle.verify import _widen, widen_bf16

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _field_value(bits):
    """bfloat16 value from its fields, with Python integers and floats."""
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    sign = -1.0 if s else 1.0
    if e == 0xFF:
        return math.nan if f else sign * math.inf
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)      # subnormal: 0.f * 2^-126
    return sign * math.ldexp(128 + f, e - 127 - 7)  # normal: 1.f * 2^(e-127)


def test_widen_all_patterns_match_torch_cast():
    ours = widen_bf16(ALL)
    ref = torch.from_numpy(ALL.view(np.int16)).view(torch.bfloat16).to(torch.float32).double().numpy()
    assert ours.dtype == np.float64 and ours.shape == (1 << 16,)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0x0000])


def test_widen_all_patterns_match_field_formula():
    ours = widen_bf16(ALL)
    ref = np.array([_field_value(int(b)) for b in ALL])
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    # 254 binades of 128 normal values and 127 subnormals per sign, +-0, +-inf
    finite = ref[np.isfinite(ref)]
    assert np.unique(finite).size == 2 * (254 * 128 + 127) + 1


def test_input_widening_takes_the_bf16_branch():
    # the verify oracle's ingest: uint16 arrays are bit patterns, anything
    # else is a numeric value
    bits = np.array([[0x3F80, 0xC000, 0x0001]], dtype=np.uint16)  # 1, -2, 2^-133
    np.testing.assert_array_equal(_widen(bits), [[1.0, -2.0, math.ldexp(1.0, -133)]])
    np.testing.assert_array_equal(_widen(np.array([1.0, -2.0], np.float32)), [1.0, -2.0])


def _bits(values):
    """Exact bfloat16 patterns of values that bfloat16 represents exactly."""
    v = np.asarray(values, dtype=np.float32)
    u = v.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "not a bfloat16 value"
    return (u >> 16).astype(np.uint16)


def test_bf16_worked_example():
    """V = 3, T = 0.5, one drafted token, logits chosen exactly representable
    in bfloat16.  Probabilities written out from the decoded values with
    math.exp: p = softmax(l/T) for the target, q for the draft; alpha(x) =
    min(1, p(x)/q(x)); residual max(0, p - q)/Z."""
    lt = [[1.5, 0.25, -0.75], [0.0, 0.5, 1.0]]   # target positions 0, 1
    ld = [[0.5, 1.25, -0.25]]                    # draft position 0
    T = 0.5
    t_bits = _bits(lt)[None]
    d_bits = _bits(ld)[None]

    def sm(row):
        e = [math.exp(v / T) for v in row]
        s = sum(e)
        return [x / s for x in e], s

    p0, s0 = sm(lt[0])
    q0, sd = sm(ld[0])
    p1, _ = sm(lt[1])
    for x in range(3):
        # draw every drafted id; over seeds the decision must follow alpha
        r = oracle.verify(t_bits, d_bits, np.array([[x]]), None, T, 1.0, 0)
        pp = r.probe_pos[0]
        assert abs(pp[0, 4] - p0[x]) < 1e-15 and abs(pp[0, 5] - q0[x]) < 1e-15
        # probe fields 1 and 3 hold sum exp((l - max)/T)
        assert abs(pp[0, 1] - s0 / math.exp(max(lt[0]) / T)) < 1e-14
        assert abs(pp[0, 3] - sd / math.exp(max(ld[0]) / T)) < 1e-14
    # decisions against hand thresholds: token 1 has alpha = p0[1]/q0[1] < 1
    alpha1 = p0[1] / q0[1]
    assert alpha1 < 1.0
    z = sum(max(0.0, a - b) for a, b in zip(p0, q0))
    w = [max(0.0, a - b) / z for a, b in zip(p0, q0)]
    for seed in range(200):
        r = oracle.verify(t_bits, d_bits, np.array([[1]]), None, T, 1.0, seed)
        ua, ur = oracle.uniforms(seed, 0, 0)
        if ua < alpha1:
            # accepted: the bonus is drawn from p1 by inverse CDF with word 1
            # of position 1
            u1 = oracle.uniforms(seed, 0, 1)[1]
            c, y = 0.0, 0
            while True:
                c += p1[y]
                if c > u1 or y == 2:
                    break
                y += 1
            assert r.n_accepted[0] == 1 and list(r.tokens[0]) == [1, y]
        else:
            c, y = 0.0, 0
            while True:
                c += w[y]
                if c > ur or y == 2:
                    break
                y += 1
            assert r.n_accepted[0] == 0 and r.tokens[0, 0] == y
            assert abs(r.probe_row[0, 0] - z) < 1e-15


def test_bf16_emitted_token_law():
    """Many independent rows of the same bfloat16 logits (each row draws its
    own Philox uniforms): the first emitted token follows softmax(l/T) of the
    decoded target values, and position 0 accepts with probability
    sum_x min(p, q) -- both computed here from the field formula, not from
    the oracle.  A wrong widening (a shift, a dropped sign, a lost bit)
    changes the values and fails the chi-square tests."""
    rng = np.random.default_rng(2024)
    V, B, T = 6, 6000, 0.8
    t_vals = np.round(rng.normal(0, 1.5, size=(2, V)) * 8) / 8   # 1/8 grid: exact in bfloat16
    d_vals = np.round((t_vals[:1] + rng.normal(0, 0.8, size=(1, V))) * 8) / 8
    t_bits = np.broadcast_to(_bits(t_vals), (B, 2, V)).copy()
    d_bits = np.broadcast_to(_bits(d_vals), (B, 1, V)).copy()
    dv = np.array([_field_value(int(b)) for b in _bits(d_vals)[0]])
    tv = np.array([_field_value(int(b)) for b in _bits(t_vals)[0]])
    q = np.exp(dv / T) / np.exp(dv / T).sum()
    p = np.exp(tv / T) / np.exp(tv / T).sum()
    x = rng.choice(V, size=B, p=q)[:, None]
    r = oracle.verify(t_bits, d_bits, x, None, T, 1.0, 77)
    first = r.tokens[:, 0]
    counts = np.bincount(first, minlength=V)
    assert scipy.stats.chisquare(counts, B * p).pvalue > 1e-4
    beta = np.minimum(p, q).sum()
    acc = int(np.sum(r.n_accepted == 1))
    assert abs(acc - B * beta) < 4.5 * math.sqrt(B * beta * (1 - beta))
