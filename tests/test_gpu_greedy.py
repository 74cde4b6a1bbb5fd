"""GPU parity of greedy verify with the next-next-token top-k:
spec_greedy_verify against the float64 oracle (oracle.greedy_verify) on the
same seeded inputs, through the C ABI.  Greedy decisions are exact
comparisons, so every row must match exactly: accepted counts, emitted
tokens and the top-k ids."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import dev_array, say
from rejection_sampling_verifier_amd import binding
from rejection_sampling_verifier_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.load()
    yield
    torch.cuda.synchronize()


def _drafts(target_f32, s, agree=0.7):
    """Drafts that agree with the target's argmax with probability `agree`."""
    rng = np.random.default_rng(4000 + s)
    B, K1, V = target_f32.shape
    am = np.argmax(target_f32[:, : K1 - 1], axis=-1)
    rnd = rng.integers(0, V, size=am.shape)
    return np.where(rng.random(am.shape) < agree, am, rnd).astype(np.int32)


def _check(t, x, dl, k, label):
    B, K1 = t.shape[0], t.shape[1]
    say(f"[greedy] {label} B={B} K={K1 - 1} V={t.shape[2]} {t.dtype} k={k}")
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    dlt = None if dl is None else torch.from_numpy(np.ascontiguousarray(dl, dtype=np.int32)).cuda()
    tok, n, tk = binding.greedy_verify(dev_array(t), xt, dlt, k)
    torch.cuda.synchronize()
    tok, n, tk = tok.cpu().numpy(), n.cpu().numpy(), tk.cpu().numpy()
    r = oracle.greedy_verify(t, x, dl, k)
    assert np.array_equal(n, r.n_accepted), (label, n, r.n_accepted)
    assert np.array_equal(tok, r.tokens), label
    if k:
        bad = np.nonzero(np.any(tk != r.topk, axis=1))[0]
        assert bad.size == 0, (label, bad[:4], tk[bad[:1]], r.topk[bad[:1]])
    say(f"    mean n={np.mean(r.n_accepted):.2f}")
    return r


def _f32(t):
    return W.bf16_bits_to_f32(t) if t.dtype == np.uint16 else t


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [10, 60])
def test_greedy_small(dtype, k):
    for s in range(3):
        inp = W.synthetic(16, 4, 1000, dtype=dtype, seed=s, gen_seed=6000 + s)
        x = _drafts(_f32(inp.target), s)
        _check(inp.target, x, None, k, f"small s={s}")


def test_greedy_several_chunks_ragged():
    for s in range(2):
        # padded positions hold NaN and are never read; their drafted ids are -1
        inp = W.make_inputs(3, 20 + s, B=24, V=40009)
        x = _drafts(np.nan_to_num(W.bf16_bits_to_f32(inp.target), nan=-1e30), s)
        x = np.where(inp.draft_tokens >= 0, x, -1)
        _check(inp.target, x, inp.draft_len, 60, f"ragged V=40009 s={s}")


def test_greedy_ties_and_flat_rows():
    rng = np.random.default_rng(9)
    B, K, V = 6, 3, 3000
    t = (np.round(rng.normal(0, 1.5, size=(B, K + 1, V)) * 2) / 2).astype(np.float32)  # heavy ties
    t[4] = 0.0                      # flat rows: every list overflows
    t[5, :, :] = -1.0
    t[5, :, 2500:2600] = 2.0        # a 100-way tie at the top of one wave
    x = _drafts(t, 9, agree=0.8)
    _check(W.f32_to_bf16_bits(t), x, None, 60, "ties and flat rows, bf16")
    _check(t, x, None, 17, "ties and flat rows, fp32")


def test_greedy_small_vocabulary_and_k0():
    inp = W.synthetic(5, 2, 40, dtype="f32", seed=3, gen_seed=6100)
    x = _drafts(inp.target, 3)
    _check(inp.target, x, None, 60, "V=40 < k+1")
    _check(inp.target, x, None, 0, "k=0")


def test_greedy_invalid_rows():
    inp = W.synthetic(6, 3, 700, dtype="f32", seed=4, gen_seed=6200)
    t = inp.target.copy()
    x = _drafts(t, 4)
    x[1, 0] = 700
    t[2, 1, 5] = np.nan
    t[3, 0, :] = -np.inf
    dl = np.array([3, 3, 3, 3, 4, -1], np.int32)
    r = _check(t, x, dl, 8, "invalid rows")
    assert list(r.n_accepted[[1, 2, 3, 4, 5]]) == [-1] * 5


def test_greedy_full_size():
    inp = W.make_inputs(2, 11)
    x = _drafts(W.bf16_bits_to_f32(inp.target), 11)
    _check(inp.target, x, None, 60, "full size")


def _wave0_ids(V, n_per_lane, lanes):
    """Ids that a 256-thread statistics workgroup with 16-byte loads of
    8 bf16 values gives to the given lanes of its first wave in the first
    chunk: vector u * 256 + lane, element i.  (A different split only moves
    the pattern between lists; the parity check holds either way.)"""
    ids = []
    for lane in lanes:
        for u in range(n_per_lane):
            ids.append((u * 256 + lane) * 8)
    return np.array(ids)


def test_greedy_list_cut_back_and_overflow():
    rng = np.random.default_rng(21)
    B, K, V = 4, 2, 40000
    t = (rng.standard_normal((B, K + 1, V)) - 10.0).astype(np.float32)
    # row 0: group g (lanes 8g..8g+7) of the first wave holds a few tokens at
    # 1 + g, group 0 thirty of them: more than one list's worth at the
    # smallest group max, few enough at the second smallest
    for j in range(K + 1):
        for g in range(8):
            lanes = range(8 * g, 8 * g + 8)
            ids = _wave0_ids(V, 8, lanes)
            take = ids[: (30 if g == 0 else 6)]
            t[0, j, take] = 1.0 + g
    # row 1: too many takers even at the second smallest group max
    for j in range(K + 1):
        ids = _wave0_ids(V, 8, range(64))
        t[1, j, ids[:200]] = 3.0
    # row 2: whole chunks of -inf (a masked vocabulary tail)
    t[2, :, 9000:] = -np.inf
    # row 3: logits rising with the id (one wave holds every top token)
    t[3] = np.linspace(-5.0, 5.0, V, dtype=np.float32)[None, :] + 0.01 * t[3]
    x = _drafts(t, 21, agree=0.8)
    _check(W.f32_to_bf16_bits(t), x, None, 60, "cut-back, overflow, masked tail, sorted, bf16")
    _check(t, x, None, 33, "cut-back, overflow, masked tail, sorted, fp32")


def test_greedy_nan_and_inf_in_a_full_chunk():
    inp = W.make_inputs(2, 12, B=6)
    t = inp.target.copy()
    x = _drafts(W.bf16_bits_to_f32(t), 12)
    t[1, 3, 70000] = W.NAN_BF16                     # NaN inside a full chunk
    t[2, 0, 5] = W.f32_to_bf16_bits(np.float32(np.inf)).item()  # +inf: invalid too
    t[3, 5, 128255] = W.f32_to_bf16_bits(np.float32(-np.inf)).item()
    r = _check(t, x, None, 60, "NaN / +inf / -inf in full rows")
    assert r.n_accepted[1] == -1 and r.n_accepted[2] == -1 and r.n_accepted[3] >= 0


def test_greedy_large_ragged_full_size():
    """The large ragged batch's shape (B=256, K=8, V=128256 bf16, ragged
    lengths, padded positions NaN and never read): every row's decision
    against the oracle, the top-60 on a sample of rows."""
    inp = W.make_inputs(3, 5)
    t = inp.target
    tf = np.nan_to_num(W.bf16_bits_to_f32(t), nan=-1e30)
    x = _drafts(tf, 5)
    x = np.where(inp.draft_tokens >= 0, x, -1).astype(np.int32)
    say(f"[greedy] large ragged B={t.shape[0]} K={t.shape[1] - 1} V={t.shape[2]}")
    xt = torch.from_numpy(x).cuda()
    dlt = torch.from_numpy(inp.draft_len.astype(np.int32)).cuda()
    tok, n, tk = binding.greedy_verify(dev_array(t), xt, dlt, 60)
    torch.cuda.synchronize()
    tok, n, tk = tok.cpu().numpy(), n.cpu().numpy(), tk.cpu().numpy()
    rows = list(range(0, t.shape[0], 16)) + [t.shape[0] - 1]
    for b in range(t.shape[0]):
        L = int(inp.draft_len[b])
        am = [oracle.argmax_lowest(W.bf16_bits_to_f32(t[b, j])) for j in range(L + 1)]
        nb = next((j for j in range(L) if x[b, j] != am[j]), L)
        assert n[b] == nb, (b, n[b], nb)
        assert np.array_equal(tok[b, :nb], x[b, :nb]) and tok[b, nb] == am[nb] and np.all(tok[b, nb + 1:] == -1), b
        if b in rows:
            assert np.array_equal(tk[b], oracle.top_k_after_first(W.bf16_bits_to_f32(t[b, nb]), 60)), b


@pytest.mark.parametrize("unroll", [4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_greedy_statistics_variants(unroll, dtype, monkeypatch):
    """Both compiled statistics variants (4 or 8 vectors per lane; with 4, a
    V = 128256 bf16 row has 16 chunks, so the row kernel reads the lists in
    two batches of eight chunks)."""
    monkeypatch.setenv("SPECVERIFY_STATS_UNROLL", str(unroll))
    inp = W.make_inputs(2, 13, B=6, dtype=dtype)
    x = _drafts(_f32(inp.target), 13)
    _check(inp.target, x, None, 60, f"unroll={unroll} {dtype}")


def test_greedy_large_vocabulary():
    inp = W.make_inputs(2, 14, B=6, V=262147)
    x = _drafts(_f32(inp.target), 14)
    _check(inp.target, x, None, 64, "V=262147 k=64")


def test_greedy_largest_vocabulary():
    """V = 2^24, the largest vocabulary greedy verify accepts: 1024
    statistics chunks and 4096 wave lists per logit row."""
    V = 1 << 24
    inp = W.synthetic(2, 2, V, dtype="bf16", seed=5, gen_seed=V)
    x = _drafts(_f32(inp.target), 15)
    _check(inp.target, x, None, 64, "V=2^24 k=64")
