"""The no-allocation entry point spec_verify_noalloc (for callers that cannot
allocate device memory), through the C ABI, against spec_verify on the same
inputs: bit-exact outputs on two calls in a row, the second smaller, on the
fixed per-device scratch array the library never allocates or frees; a call
too large for the array is refused with SV_ETOOBIG."""

import numpy as np
import pytest
import torch

from gpu_helpers import check_parity, run_oracle, say, to_device
from rejection_sampling_verifier_amd import binding
from rejection_sampling_verifier_amd import workloads as W

pytestmark = pytest.mark.gpu


def _pair(inp, top_p=None):
    t, d, x, dl = to_device(inp)
    T = float(inp.temperature)
    tp = float(inp.top_p if top_p is None else top_p)
    out_t = torch.full((inp.B, inp.K + 1), -7, dtype=torch.int32, device="cuda")
    out_n = torch.full((inp.B,), -7, dtype=torch.int32, device="cuda")
    binding.verify(t, d, x, dl, T, tp, inp.seed, out_tokens=out_t, out_n_accepted=out_n, noalloc=True)
    ref_t, ref_n = binding.verify(t, d, x, dl, T, tp, inp.seed)
    torch.cuda.synchronize()
    return (out_t.cpu().numpy(), out_n.cpu().numpy()), (ref_t.cpu().numpy(), ref_n.cpu().numpy())


@pytest.mark.parametrize("cfg", [2, 4])
def test_noalloc_matches_spec_verify_twice(cfg):
    assert torch.cuda.is_available()
    binding.load()
    # full batched shape first, then a smaller call on the same array
    for label, inp in (("full", W.make_inputs(cfg, 30)), ("smaller", W.make_inputs(cfg, 31, B=9, V=5003))):
        say(f"[noalloc] cfg={cfg} {label} B={inp.B} V={inp.V} top_p={inp.top_p}")
        (gt, gn), (rt, rn) = _pair(inp)
        np.testing.assert_array_equal(gn, rn)
        np.testing.assert_array_equal(gt, rt)
        rows = np.arange(0, inp.B, max(1, inp.B // 8))
        res = run_oracle(inp, rows=rows)
        st = check_parity(inp, res, [gt, gn], rows=rows, check_probes=False)
        say(f"    {st}")


def test_noalloc_refuses_calls_beyond_its_array():
    # 2048 rows of the filtered shape need far more than 16 MiB of candidate
    # lists; the host refuses before any launch, so the logits' values are
    # never read
    B, K, V = 2048, 5, 40000
    t = torch.empty((B, K + 1, V), dtype=torch.bfloat16, device="cuda")
    d = torch.empty((B, K, V), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((B, K), dtype=torch.int32, device="cuda")
    with pytest.raises(binding.SpecVerifyError) as err:
        binding.verify(t, d, x, None, 0.7, 0.9, 5, noalloc=True)
    assert err.value.status == -8
    # and still works afterwards
    small = W.make_inputs(2, 32, B=4, V=3000)
    (gt, gn), (rt, rn) = _pair(small)
    np.testing.assert_array_equal(gn, rn)
    np.testing.assert_array_equal(gt, rt)
