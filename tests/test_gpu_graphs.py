"""Greedy verify, the SMC-SD step, the two-stage verify and the draft
producer captured into HIP graphs: each is called once eagerly on a fresh
stream (the call that sizes the stream's scratch), captured, then replayed
on new inputs copied into the captured buffers, with eager calls of the same
entry point between the replays.  Every replay must give exactly the eager
outputs (the replays reuse the captured record tags, so this also checks
that each call rewrites every record it reads)."""

import numpy as np
import pytest
import torch

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


def _replay_check(call, inputs_for, bufs, label, reps=5):
    """call(stream, fixed, *bufs) issues the entry point and returns its
    output tensors (the captured call writes fixed output buffers, the eager
    reference calls fresh ones); inputs_for(rep) returns new device inputs
    for bufs."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call(stream, True, *bufs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        outs = call(stream, True, *bufs)
    torch.cuda.synchronize()
    for rep in range(reps):
        new = inputs_for(rep)
        for b, n in zip(bufs, new):
            b.copy_(n)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        ref = call(torch.cuda.current_stream(), False, *new)
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            assert torch.equal(g, r), (label, rep)
        say(f"[graph] {label} replay {rep} matches the eager call")


def test_greedy_graph_replays():
    sets = [W.make_inputs(3, 50 + s, B=10, V=20011) for s in range(3)]
    tgts = [dev_array(np.nan_to_num(W.bf16_bits_to_f32(s.target), nan=-3.0).astype(np.float32)) for s in sets]
    xs = []
    for s, t in zip(sets, tgts):
        am = torch.argmax(t[:, : s.K], dim=-1).to(torch.int32)
        rnd = torch.randint(0, s.V, am.shape, device="cuda", dtype=torch.int32)
        keep = torch.rand(am.shape, device="cuda") < 0.7
        xs.append(torch.where(keep, am, rnd).contiguous())
    lens = [torch.from_numpy(s.draft_len.astype(np.int32)).cuda() for s in sets]
    bufs = [tgts[0].clone(), xs[0].clone(), lens[0].clone()]
    B, K1 = bufs[0].shape[0], bufs[0].shape[1]
    o = [torch.empty((B, K1), dtype=torch.int32, device="cuda"), torch.empty((B,), dtype=torch.int32, device="cuda"),
         torch.empty((B, 40), dtype=torch.int32, device="cuda")]

    def call(st, fixed, t, x, dl):
        outs = o if fixed else [torch.empty_like(a) for a in o]
        return binding.greedy_verify(t, x, dl, 40, stream=st, out_tokens=outs[0], out_n_accepted=outs[1],
                                     out_topk=outs[2])

    _replay_check(call, lambda r: [tgts[r % 3], xs[r % 3], lens[r % 3]], bufs, "greedy")


def test_producer_graph_replays():
    sets = [W.make_inputs(2, 60 + s, B=6, V=30000) for s in range(3)]
    tgts = [dev_array(s.target) for s in sets]
    bufs = [tgts[0].clone()]
    B, K, V = 6, 5, 30000
    o = [torch.empty((B, K, V), dtype=torch.bfloat16, device="cuda"), torch.empty((B, K), dtype=torch.int32,
                                                                                   device="cuda")]

    def call(st, fixed, t):
        outs = o if fixed else [torch.empty_like(a) for a in o]
        return binding.draft_produce(t, K, 4242, stream=st, out=outs[0], out_tokens=outs[1])

    _replay_check(call, lambda r: [tgts[r % 3]], bufs, "producer")


def test_smc_graph_replays():
    sets = [W.make_inputs(2, 70 + s, B=8, V=20000) for s in range(3)]
    dev = [(dev_array(s.target), dev_array(s.draft), torch.from_numpy(s.draft_tokens).cuda()) for s in sets]
    lw = torch.linspace(-2.0, 0.0, 8, dtype=torch.float64, device="cuda")
    bufs = [dev[0][0].clone(), dev[0][1].clone(), dev[0][2].clone(), lw.clone()]

    def call(st, fixed, t, d, x, logw):
        return binding.smc_step(t, d, x, logw, 0.7, 0.5, 99, stream=st)

    _replay_check(call, lambda r: [dev[r % 3][0], dev[r % 3][1], dev[r % 3][2], lw * (r + 1)], bufs, "smc")


def test_hispec_graph_replays():
    hs = [W.make_hispec_inputs(6, 3, 12000, dtype="bf16", step=s, temperature=0.7) for s in range(3)]
    dev = [(dev_array(h.final), dev_array(h.inter), dev_array(h.draft), torch.from_numpy(h.draft_tokens).cuda())
           for h in hs]
    bufs = [a.clone() for a in dev[0]]

    def call(st, fixed, f, i, d, x):
        return binding.hispec_verify(f, i, d, x, None, 0.7, 1.0, 7, stream=st)

    _replay_check(call, lambda r: list(dev[r % 3]), bufs, "hispec")
