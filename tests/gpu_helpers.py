"""Shared helpers of the GPU tests: move seeded inputs to the device, run the
library through its binding, run the oracle on the same inputs, compare."""

import sys

import numpy as np
import torch

import oracle
from rejection_sampling_verifier_amd import binding

PROBE_RTOL = 1e-5  # probabilities and residual masses (spec tolerance)


def dev_array(a, device="cuda"):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(inp, device="cuda"):
    t = dev_array(inp.target, device)
    d = dev_array(inp.draft, device)
    x = torch.from_numpy(np.ascontiguousarray(inp.draft_tokens, dtype=np.int32)).to(device)
    dl = None if inp.draft_len is None else torch.from_numpy(np.ascontiguousarray(inp.draft_len, np.int32)).to(device)
    return t, d, x, dl


def run_gpu(inp, probe=True, tensors=None):
    t, d, x, dl = to_device(inp) if tensors is None else tensors
    out = binding.verify(t, d, x, dl, float(inp.temperature), float(inp.top_p), inp.seed, probe=probe)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def run_oracle(inp, rows=None):
    return oracle.verify(inp.target, inp.draft, inp.draft_tokens, inp.draft_len, inp.temperature, inp.top_p,
                         inp.seed, rows=rows)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_parity(inp, res, gpu, rows=None, check_probes=True):
    """Element-by-element comparison on the rows the oracle computed.

    Tokens and accepted counts must be identical on every row without a
    flagged decision.  Probe values (max logit, softmax normalisers, p'(x_j),
    q'(x_j), kept masses, Z, t) must agree to PROBE_RTOL relative.
    Returns (rows compared, rows flagged, decisions, flagged decisions)."""
    tokens, n_acc = gpu[0], gpu[1]
    rows = res.rows if rows is None else rows
    checked = flagged = 0
    for b in rows:
        if res.flagged[b]:
            flagged += 1
            continue
        checked += 1
        assert n_acc[b] == res.n_accepted[b], (b, int(n_acc[b]), int(res.n_accepted[b]))
        np.testing.assert_array_equal(tokens[b], res.tokens[b], err_msg=f"row {b}")
        if check_probes and len(gpu) > 2 and res.n_accepted[b] >= 0:
            pp, pr = gpu[2], gpu[3]
            ok = ~np.isnan(res.probe_pos[b])
            np.testing.assert_array_equal(np.isnan(pp[b]), ~ok, err_msg=f"probe NaN pattern, row {b}")
            np.testing.assert_allclose(pp[b][ok], res.probe_pos[b][ok], rtol=PROBE_RTOL, atol=0,
                                       err_msg=f"probe_pos row {b}")
            np.testing.assert_allclose(pr[b][:3], res.probe_row[b][:3], rtol=PROBE_RTOL, atol=0,
                                       err_msg=f"probe_row row {b}")
            assert pr[b][3] == res.n_accepted[b]
    dec = int(np.sum(res.n_decisions[rows]))
    fdec = int(np.sum(res.n_flagged[rows]))
    return checked, flagged, dec, fdec
