"""GPU parity of the synthetic draft producer (spec_draft_produce) against its
float oracle (oracle.produce_drafts), bit for bit, and of the two-batch
schedule: the producer of one batch on a second stream while the verify step
of the other runs on the first, the roles swapping every step; every verify
must return exactly what the same call returns alone."""

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


def _bits(t):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _check(target, K, seed, label, rows=None, out=None):
    say(f"[produce] {label} shape={tuple(target.shape)} K={K}")
    tt = dev_array(target)
    d, tok = binding.draft_produce(tt, K, seed, out=None if out is None else out(tt))
    torch.cuda.synchronize()
    d, tok = _bits(d), tok.cpu().numpy()
    if rows is None:
        rd, rt = oracle.produce_drafts(target, K, seed)
        assert np.array_equal(d.view(np.uint32 if d.dtype == np.float32 else np.uint16),
                              rd.view(np.uint32 if rd.dtype == np.float32 else np.uint16)), label
        assert np.array_equal(tok, rt), (label, np.nonzero(tok != rt))
    else:
        for b, j in rows:
            rd, rt = _oracle_row(target, b, j, seed)
            assert np.array_equal(d[b, j].view(np.uint16), rd.view(np.uint16)), (label, b, j)
            assert tok[b, j] == rt, (label, b, j)
    return d, tok


def _oracle_row(target, b, j, seed):
    """Oracle draft row (b, j) without producing the whole batch."""
    from oracle import produce as P
    V = target.shape[2]
    t = P.bf16_to_f32(target[b, j]) if target.dtype == np.uint16 else target[b, j].astype(np.float32)
    s = t + P.deltas(seed, b, j, V)
    if target.dtype == np.uint16:
        d = P.f32_to_bf16_rne(s)
        dv = P.bf16_to_f32(d)
    else:
        d, dv = s, s
    return d, (-1 if np.isnan(dv).any() else int(np.argmax(dv)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 7, 1000, 8193, 40009])
def test_produce_small(dtype, V):
    inp = W.synthetic(3, 3, V, dtype=dtype, seed=1, gen_seed=7000 + V)
    _check(inp.target, 3, 0x1234_5678_9ABC_DEF0, f"{dtype} V={V}")


def test_produce_unaligned_strided_and_special_rows():
    rng = np.random.default_rng(8)
    B, P, V = 3, 4, 5001
    base = (rng.standard_normal((B, P, V + 3)) * 3).astype(np.float32)
    base[1, 0, 100] = np.nan
    base[2, 1, :] = -np.inf
    base[2, 2, 17] = np.inf
    bits = W.f32_to_bf16_bits(base)
    # a view whose rows start one element past 16-byte alignment, written into
    # a strided output view
    full = dev_array(bits)
    tt = full[:, :, 1: V + 1]
    outbuf = torch.zeros((B, 3, V + 8), dtype=torch.bfloat16, device="cuda")
    d, tok = binding.draft_produce(tt, 3, 77, out=outbuf[:, :, 3: V + 3])
    torch.cuda.synchronize()
    d, tok = _bits(d), tok.cpu().numpy()
    tgt = np.ascontiguousarray(bits[:, :, 1: V + 1])
    rd, rt = oracle.produce_drafts(tgt, 3, 77)
    assert np.array_equal(d, rd)
    assert np.array_equal(tok, rt)
    # the view starts one element into the row: base id 17 is view id 16
    assert tok[1, 0] == -1 and tok[2, 1] == 0 and tok[2, 2] == 16
    # the elements around the written view are untouched
    ob = _bits(outbuf)
    assert not ob[:, :, :3].any() and not ob[:, :, V + 3:].any()


def test_produce_full_size_sampled_rows():
    inp = W.make_inputs(2, 30)
    rows = [(0, 0), (5, 4), (17, 2), (33, 1), (63, 4), (40, 3)]
    _check(inp.target, 5, inp.seed, "full size B=64 K=5 V=128256 bf16", rows=rows)


def test_two_stream_schedule_matches_standalone_calls():
    """Two batches alternate: while batch X is verified on stream 0, the
    producer drafts batch Y on stream 1; then the roles swap.  Every verify
    output must equal a standalone call on the same inputs."""
    B, K, V = 16, 5, 32768
    sets = [W.make_inputs(2, 40 + i, B=B, V=V) for i in range(2)]
    tgt = [dev_array(s.target) for s in sets]
    drafts = [torch.empty((B, K, V), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    toks = [torch.empty((B, K), dtype=torch.int32, device="cuda") for _ in range(2)]
    s0 = torch.cuda.Stream()
    s1 = torch.cuda.Stream()
    produced = [torch.cuda.Event() for _ in range(2)]
    verified = [torch.cuda.Event() for _ in range(2)]
    # step 0: draft batch 0 alone
    with torch.cuda.stream(s1):
        binding.draft_produce(tgt[0], K, 1000, stream=s1, out=drafts[0], out_tokens=toks[0])
        produced[0].record(s1)
    outs = []
    for step in range(6):
        x, y = step % 2, (step + 1) % 2
        seed_v, seed_p = 5000 + step, 1001 + step
        # verify x on stream 0 once its drafts exist; keep what it saw (on
        # the same stream, before the drafts may be overwritten)
        s0.wait_event(produced[x])
        with torch.cuda.stream(s0):
            tok_v, n_v = binding.verify(tgt[x], drafts[x], toks[x], None, 0.7, 1.0, seed_v, stream=s0)
            outs.append((x, seed_v, drafts[x].clone(), toks[x].clone(), tok_v, n_v))
            verified[x].record(s0)
        # draft y on stream 1 once its previous verify has read the drafts
        if step > 0:
            s1.wait_event(verified[y])
        with torch.cuda.stream(s1):
            binding.draft_produce(tgt[y], K, seed_p, stream=s1, out=drafts[y], out_tokens=toks[y])
            produced[y].record(s1)
    torch.cuda.synchronize()
    say(f"[produce] two-stream schedule: {len(outs)} verify steps")
    for x, seed_v, d, t, tok_v, n_v in outs:
        tok_r, n_r = binding.verify(tgt[x], d, t, None, 0.7, 1.0, seed_v)
        torch.cuda.synchronize()
        assert torch.equal(tok_v, tok_r) and torch.equal(n_v, n_r)
    # the drafts each verify consumed are the producer's, bit for bit
    x, _, d, t, _, _ = outs[-1]
    rd, rt = oracle.produce_drafts(sets[x].target, K, 1001 + len(outs) - 2)
    assert np.array_equal(_bits(d), rd) and np.array_equal(t.cpu().numpy(), rt)


def test_produce_largest_vocabulary_sampled_rows():
    """V = 2^24, the largest vocabulary the producer accepts (2048 chunk
    records per row for the token kernel); two rows checked."""
    inp = W.synthetic(2, 2, 1 << 24, dtype="bf16", seed=3, gen_seed=1 << 24)
    _check(inp.target, 2, 0x5EED, "V=2^24 bf16", rows=[(0, 0), (1, 1)])
