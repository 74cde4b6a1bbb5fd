"""GPU parity of the SMC-SD step: the HIP library's spec_smc_step against
the float64 oracle (oracle.smc_step) on the same seeded inputs, through the
C ABI.

Bar: identical bonus tokens except draws within the library's band (the
verify step's draw: 1e-10 of the target mass plus float64 rounding, the
bonus mass being the whole kept mass); log-weights to 1e-5 per drafted position (log-probabilities to the
1e-5 relative bar of probabilities); ESS to 1e-5 relative; the same
resampling decision and identical ancestors unless the oracle flags the ESS
threshold or a resampling point; flagged ancestors must still be a valid
systematic draw (non-decreasing, positive-weight particles).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BAND_SAMPLE, SAMPLE_REL_EPS, dev_array, say
from rejection_sampling_verifier_amd import binding
from rejection_sampling_verifier_amd import workloads as W

pytestmark = pytest.mark.gpu

FLAG = oracle.FLAG_BAND
DRAW_BAND = BAND_SAMPLE + SAMPLE_REL_EPS  # a bonus draw: Z is the whole target mass


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.load()
    yield
    torch.cuda.synchronize()


def _inputs(N, K, V, dtype, s, sigma=1.0, T=0.8):
    inp = W.synthetic(N, K, V, dtype=dtype, temperature=T, sigma=sigma, seed=s, gen_seed=5000 + s)
    lw = np.random.default_rng(s).normal(0, 0.7, size=N)
    return inp.target, inp.draft, inp.draft_tokens, lw


def _check(t, d, x, lw, T, frac, seed, label, in_place=False):
    N, K1 = t.shape[0], t.shape[1]
    K = K1 - 1
    say(f"[smc] {label} N={N} K={K} V={t.shape[2]} {t.dtype} T={T} ess_fraction={frac} seed={seed:#x}")
    tt, dd = dev_array(t), dev_array(d)
    xx = torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    lwt = torch.from_numpy(np.ascontiguousarray(lw, dtype=np.float64)).cuda()
    out = binding.smc_step(tt, dd, xx, lwt, T, frac, seed, out_logw=lwt if in_place else None)
    torch.cuda.synchronize()
    bonus, lwo, anc, e, rs = (o.cpu().numpy() for o in out)
    e, rs = float(e[0]), bool(rs[0])
    r = oracle.smc_step(t, d, x, lw, T, frac, seed)
    valid = r.bonus >= 0
    # bonus draws
    for i in range(N):
        if r.bonus[i] < 0:
            assert bonus[i] == -1, (label, i)
        elif r.bonus_margin[i] >= DRAW_BAND:
            assert bonus[i] == r.bonus[i], (label, i, bonus[i], r.bonus[i])
    # effective sample size and the decision to resample
    if r.ess == 0.0:
        assert e == 0.0 and not rs
    else:
        assert abs(e - r.ess) <= 1e-5 * r.ess, (label, e, r.ess)
    if r.ess_margin >= FLAG:
        assert rs == r.resampled, (label, e, r.ess)
    if rs:
        assert np.all(lwo == 0.0)
        if r.resampled and r.resample_margin >= FLAG:
            assert np.array_equal(anc, r.ancestors), (label, anc, r.ancestors)
        else:
            assert np.all(np.diff(anc) >= 0) and np.all(valid[anc])
    else:
        assert np.array_equal(anc, np.arange(N))
        ok = r.bonus >= 0
        np.testing.assert_allclose(lwo[ok], r.logw[ok], rtol=0, atol=1e-5 * K)
        assert np.all(lwo[~ok] == -np.inf)
    flagged = int(np.sum(r.bonus_margin < DRAW_BAND)) + int(r.ess_margin < FLAG) + int(r.resample_margin < FLAG)
    say(f"    resampled={rs} ess={e:.4f} (oracle {r.ess:.4f}) flagged decisions={flagged}/{r.n_decisions}")
    return r


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_smc_small(dtype):
    for s in range(4):
        t, d, x, lw = _inputs(8, 3, 1000, dtype, s)
        _check(t, d, x, lw, 0.8, 0.5, 0x5A000 + s, f"small s={s}")


def test_smc_several_chunks_bf16():
    for s in range(3):
        t, d, x, lw = _inputs(16, 5, 20011, "bf16", 10 + s, sigma=1.5, T=0.7)
        _check(t, d, x, lw, 0.7, 0.5, 0x5B000 + s, f"V=20011 s={s}")


def test_smc_always_and_never_resample():
    t, d, x, lw = _inputs(12, 4, 3001, "bf16", 20, sigma=2.0)
    r = _check(t, d, x, lw, 0.8, 2.0, 0x5C001, "always")
    assert r.resampled
    r = _check(t, d, x, lw, 0.8, 0.0, 0x5C001, "never")
    assert not r.resampled


def test_smc_invalid_particles_and_dead_weights():
    t, d, x, lw = _inputs(10, 3, 700, "f32", 30)
    x = x.copy()
    x[1, 2] = 700               # drafted id out of range
    t[2, 3, 11] = np.nan        # NaN in the bonus row
    d[3, 0, :] = -np.inf        # all -inf draft row
    lw[4] = np.nan              # unusable input weight
    lw[5] = np.inf
    lw[6] = -np.inf             # a dead particle stays dead
    r = _check(t, d, x, lw, 0.9, 1.5, 0x5D001, "invalid, resampling")
    assert np.sum(r.bonus < 0) == 5
    _check(t, d, x, lw, 0.9, 0.0, 0x5D002, "invalid, keeping weights")
    x2 = np.full_like(x, 700)
    r = _check(t, d, x2, lw, 0.9, 1.0, 0x5D003, "no valid particle")
    assert r.ess == 0.0


def test_smc_many_particles():
    # the resampling kernel's loops over N and its binary searches
    t, d, x, lw = _inputs(1024, 1, 64, "f32", 40, sigma=2.0, T=1.0)
    _check(t, d, x, lw, 1.0, 0.9, 0x5E001, "N=1024")
    _check(t, d, x, lw, 1.0, 0.0, 0x5E002, "N=1024 keep")


def test_smc_in_place_log_weights():
    t, d, x, lw = _inputs(8, 2, 513, "bf16", 50)
    _check(t, d, x, lw, 0.8, 0.0, 0x5F001, "in place", in_place=True)
    _check(t, d, x, lw, 0.8, 1.5, 0x5F002, "in place, resampling", in_place=True)


def test_smc_full_size_batched_workload():
    # the batched workload's inputs as 64 particles, K = 5, V = 128256 bf16
    inp = W.make_inputs(2, 7)
    lw = np.random.default_rng(7).normal(0, 0.5, size=inp.B)
    _check(inp.target, inp.draft, inp.draft_tokens, lw, float(inp.temperature), 0.5, 0x60001, "full size")
