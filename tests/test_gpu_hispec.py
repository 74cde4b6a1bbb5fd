"""GPU parity of the two-stage (hierarchical) verify: spec_hispec_verify
against the float64 oracle (oracle.hispec_verify) on the same seeded inputs,
through the C ABI.

Bar: identical stage-1 counts, final counts and emitted tokens on every row
with no decision inside the library's band for its kind (tests/gpu_helpers.py:
acceptance tests 2.5e-6 on the u scale, 3.5e-6 with top-p; draws 1e-10 of
the residual mass plus float64 rounding; nucleus cuts 3e-6), each stage
judged by its own decisions; at most one such row per call.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import dev_array, near_boundary, say
from rejection_sampling_verifier_amd import binding
from rejection_sampling_verifier_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.load()
    yield
    torch.cuda.synchronize()


def _layers(B, K, V, dtype, s, T=0.8, ragged=False):
    h = W.make_hispec_inputs(B, K, V, dtype=dtype, step=s, temperature=T, ragged=ragged)
    return h.final, h.inter, h.draft, h.draft_tokens, h.draft_len


def _check(f, i, d, x, dl, T, top_p, seed, label):
    B, K = d.shape[0], d.shape[1]
    say(f"[hispec] {label} B={B} K={K} V={d.shape[2]} {d.dtype} T={T} top_p={top_p} seed={seed:#x}")
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    dlt = None if dl is None else torch.from_numpy(dl).cuda()
    tok, n, n1 = binding.hispec_verify(dev_array(f), dev_array(i), dev_array(d), xt, dlt, T, top_p, seed)
    torch.cuda.synchronize()
    tok, n, n1 = tok.cpu().numpy(), n.cpu().numpy(), n1.cpu().numpy()
    r = oracle.hispec_verify(f, i, d, x, dl, T, top_p, seed)
    checked = near = 0
    for b in range(B):
        if near_boundary(r.stage1, b, top_p):
            near += 1
            continue
        assert n1[b] == r.n_stage1[b], (label, b, n1[b], r.n_stage1[b])
        if near_boundary(r.stage2, b, top_p):
            near += 1
            continue
        checked += 1
        assert n[b] == r.n_accepted[b], (label, b, n[b], r.n_accepted[b])
        assert np.array_equal(tok[b], r.tokens[b]), (label, b, tok[b], r.tokens[b])
    say(f"    rows checked={checked} within a band={near} (oracle rows within 1e-6: {int(np.sum(r.flagged))}); "
        f"mean n1={np.mean(r.n_stage1):.2f} n={np.mean(r.n_accepted):.2f}")
    assert near <= 1, (label, near)
    return r


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hispec_small(dtype):
    for s in range(4):
        f, i, d, x, dl = _layers(8, 3, 1000, dtype, s)
        _check(f, i, d, x, dl, 0.8, 1.0, 0x4A000 + s, f"small s={s}")


def test_hispec_several_chunks_ragged():
    for s in range(3):
        f, i, d, x, dl = _layers(16, 5, 20011, "bf16", 10 + s, T=0.7, ragged=True)
        _check(f, i, d, x, dl, 0.7, 1.0, 0x4B000 + s, f"V=20011 ragged s={s}")


def test_hispec_top_p():
    f, i, d, x, dl = _layers(12, 4, 6007, "bf16", 20, T=0.9)
    _check(f, i, d, x, dl, 0.9, 0.8, 0x4C001, "top_p=0.8")


def test_hispec_identical_layers():
    # intermediate == final: stage 2 passes all n1 + 1 tokens
    f, i, d, x, dl = _layers(8, 3, 900, "f32", 30)
    f[:, :4] = i
    r = _check(f, i, d, x, dl, 0.8, 1.0, 0x4D001, "identical inter/final")
    assert np.all(r.n_accepted == r.n_stage1 + 1)


def test_hispec_invalid_rows():
    f, i, d, x, dl = _layers(6, 3, 500, "f32", 40)
    x = x.copy()
    x[1, 0] = 500            # drafted id out of range
    i[2, 1, 7] = np.nan      # NaN in an intermediate row stage 1 reads
    dl = np.array([3, 3, 3, 3, 4, -1], np.int32)  # bad lengths on rows 4 and 5
    r = _check(f, i, d, x, dl, 0.8, 1.0, 0x4E001, "invalid rows")
    assert list(r.n_accepted[[1, 2, 4, 5]]) == [-1, -1, -1, -1]


def test_hispec_full_size():
    f, i, d, x, dl = _layers(64, 5, W.V_LLAMA3, "bf16", 50, T=0.7)
    _check(f, i, d, x, dl, 0.7, 1.0, 0x4F001, "full size")
