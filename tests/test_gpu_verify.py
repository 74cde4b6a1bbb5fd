"""GPU parity: the HIP library against the float64 oracle on the same seeded
inputs, element by element, through the C ABI.

Bar (tests/gpu_helpers.py): accepted counts and emitted tokens equal the
oracle's decision by decision, except at decisions within the library's own
rounding bound of their boundary, where the alternative is checked for
validity instead; probe values (normalisers, p'(x_j), q'(x_j), kept masses,
Z, t) to 1e-5 relative.  The workload tests print the fraction of flagged
decisions; tests/test_gpu_fullsize.py holds the full-size runs that assert it.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import ParityStats, check_parity, dev_array, run_gpu, run_oracle, say, to_device
from rejection_sampling_verifier_amd import binding
from rejection_sampling_verifier_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.load()
    yield
    torch.cuda.synchronize()


def _parity(inp, rows=None, label=""):
    say(f"[parity] {label} B={inp.B} K={inp.K} V={inp.V} {inp.target.dtype} T={inp.temperature} "
        f"top_p={inp.top_p} seed={inp.seed:#x}")
    gpu = run_gpu(inp)
    res = run_oracle(inp, rows=rows)
    st = check_parity(inp, res, gpu)
    say(f"    {st}")
    assert st.rows > 0
    return st


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def test_tiny_fp32_many_steps():
    tot = ParityStats()
    for step in range(60):
        tot.add(_parity(W.make_inputs(0, step), label=f"tiny step {step}"))
    say(f"[tiny, 60 steps] {tot}")
    assert tot.n_flagged <= max(1, tot.decisions // 10000)


def test_single_stream_llama_vocab_fp32():
    for step in range(3):
        _parity(W.make_inputs(1, step), label=f"single-stream step {step}")


def test_batched_bf16_full_size():
    _parity(W.make_inputs(2, 0), label="batched full")


def test_batched_bf16_ragged_vocab_tail():
    # V = 5003: several statistics chunks and a ragged last 16-byte vector
    for step in range(6):
        _parity(W.make_inputs(2, 100 + step, B=64, V=5003), label="batched V=5003")


def test_ragged_batch_full_size_sampled_rows():
    inp = W.make_inputs(3, 0)
    rows = np.arange(0, inp.B, 8)
    _parity(inp, rows=rows, label="ragged full, every 8th row")


def test_ragged_batch_shrunk():
    for step in range(3):
        _parity(W.make_inputs(3, 50 + step, B=48, V=9001), label="ragged V=9001")


def test_filtered_shrunk():
    for step in range(3):
        _parity(W.make_inputs(4, 10 + step, B=16, V=20011), label="filtered V=20011")


def test_filtered_full_size_sampled_rows():
    inp = W.make_inputs(4, 0)
    _parity(inp, rows=np.arange(0, inp.B, 16), label="filtered full, every 16th row")


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 7, 64, 1000, 4099])
def test_small_vocabularies(dtype, V):
    for s in range(3):
        inp = W.synthetic(5, 3, V, dtype=dtype, temperature=0.8, seed=1000 + s, gen_seed=V * 10 + s)
        _parity(inp, label=f"V={V} {dtype}")


@pytest.mark.parametrize("top_p", [1.0, 0.8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [16384, 32768])
def test_vocabularies_filling_whole_chunks(V, dtype, top_p):
    """Aligned rows whose 16-byte vector count is a multiple of the
    statistics chunk (2048 vectors): each row's last chunk is empty, and the
    row is the last thing in its buffer, so a load past it can leave the
    allocation."""
    inp = W.synthetic(3, 2, V, dtype=dtype, temperature=0.7, top_p=top_p, seed=31 + V, gen_seed=V + int(top_p * 10))
    _parity(inp, label=f"V={V} {dtype} top_p={top_p}")


def test_many_rows_small_vocabulary():
    """4096 rows of 64 ids: tens of thousands of statistics workgroups, one
    row-pass item per row (rows sampled for the oracle)."""
    inp = W.synthetic(4096, 3, 64, dtype="f32", temperature=0.9, seed=4096, gen_seed=4096)
    _parity(inp, rows=np.arange(0, inp.B, 61), label="B=4096 V=64")


def test_large_batch_full_vocabulary():
    """384 rows of the batched recipe at V = 128256: 6144 row-pass items, six
    rounds of the resident workgroups (rows sampled for the oracle)."""
    inp = W.make_inputs(2, 7, B=384)
    _parity(inp, rows=np.arange(0, inp.B, 24), label="batched recipe B=384")


@pytest.mark.parametrize("K", [1, 2, 16])
def test_draft_lengths(K):
    inp = W.synthetic(9, K, 3001, dtype="bf16", temperature=0.7, sigma=0.3, seed=77 + K, gen_seed=K)
    _parity(inp, label=f"K={K}")


def test_zero_and_mixed_draft_lengths():
    inp = W.synthetic(12, 4, 2500, dtype="f32", seed=5, gen_seed=41,
                      draft_len=[0, 1, 2, 3, 4, 0, 4, 1, 0, 2, 3, 4])
    _parity(inp, label="mixed L incl. 0")


@pytest.mark.parametrize("top_p", [0.3, 0.6, 0.95])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_top_p_values(top_p, dtype):
    inp = W.synthetic(8, 3, 6007, dtype=dtype, temperature=0.9, top_p=top_p, seed=3, gen_seed=int(top_p * 1000))
    # drafts outside the draft's nucleus are legal inputs (q'(x) = 0 rule)
    _parity(inp, label=f"top_p={top_p} {dtype}")


@pytest.mark.parametrize("case", ["window", "wide", "large_offsets", "cold", "mixed_rows"])
def test_top_p_bf16_exponential_table_paths(case):
    # the top-p row pass on bfloat16 rows takes 2^(l*c) from its table for
    # 2^-8 <= |l| < 2^6 and computes the rest; rows whose offsets exceed
    # 256 compute every exponential (offsets kept), and for c > 14 the
    # table is off for the call
    T, scale = (0.09, 3.0) if case == "cold" else (0.7, {"wide": 25.0, "large_offsets": 100.0}.get(case, 3.0))
    inp = W.synthetic(8, 3, 6007, dtype="bf16", temperature=T, top_p=0.9, scale=scale, sigma=1.0, seed=21,
                      gen_seed={"window": 31, "wide": 32, "large_offsets": 33, "cold": 34, "mixed_rows": 35}[case])
    if case == "mixed_rows":
        t = W.bf16_bits_to_f32(inp.target)
        d = W.bf16_bits_to_f32(inp.draft)
        t[0] *= 40.0                       # offsets above 256: every exponential computed
        d[0] *= 40.0
        t[1, :, 5000:] = -np.inf           # masked tail
        d[1, :, 5000:] = -np.inf
        inp.draft_tokens[1] = [7, 70, 700]
        t[2] *= 1e-3                       # logits below the window
        d[2] *= 1e-3
        inp.target[:] = W.f32_to_bf16_bits(t)
        inp.draft[:] = W.f32_to_bf16_bits(d)
    _parity(inp, label=f"bf16 top-p exponential table: {case}")


def test_top_p_flat_rows_split_tie_groups():
    # all-equal logits: the whole row is one tie group; the cut keeps the
    # lowest ids; rows 2-3 draft ids outside the nucleus (r = 0/0 = 0, a
    # degenerate residual the oracle flags)
    inp = W.synthetic(4, 2, 1000, dtype="bf16", top_p=0.3705, seed=9, gen_seed=9)
    inp.target[:] = W.f32_to_bf16_bits(np.zeros((4, 3, 1000), np.float32))
    inp.draft[:] = W.f32_to_bf16_bits(np.zeros((4, 2, 1000), np.float32))
    inp.draft_tokens[:] = [[3, 5], [1, 370], [800, 3], [10, 900]]
    _parity(inp, label="flat rows, top_p=0.3705")


def test_top_p_coarse_logits_many_ties():
    rng = np.random.default_rng(3)
    inp = W.synthetic(6, 3, 20000, dtype="bf16", top_p=0.8, seed=10, gen_seed=10)
    t = np.round(rng.normal(0, 2, size=(6, 4, 20000)) * 2) / 2
    d = t[:, :3] + np.round(rng.normal(0, 1, size=(6, 3, 20000)) * 2) / 2
    inp.target[:] = W.f32_to_bf16_bits(t.astype(np.float32))
    inp.draft[:] = W.f32_to_bf16_bits(d.astype(np.float32))
    _parity(inp, label="coarse logits, top_p=0.8")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_top_p_several_chunks(dtype):
    # V = 40009: three (bf16) or five (fp32) statistics chunks, each listing
    # its own nucleus candidates
    inp = W.make_inputs(4, 31, B=6, V=40009, dtype=dtype)
    _parity(inp, label=f"filtered V=40009 {dtype}")


def test_top_p_candidates_skewed_chunks():
    # row 0 has its largest logits in the first statistics chunk, row 1 in
    # the last: the chunks' candidate bounds differ widely
    V = 3 * 16384 + 123
    inp = W.make_inputs(4, 32, B=4, V=V)
    t = W.bf16_bits_to_f32(inp.target).copy()
    d = W.bf16_bits_to_f32(inp.draft).copy()
    t[0, :, :16384] += 2.5
    d[0, :, :16384] += 2.5
    t[1, :, -16000:] += 2.5
    d[1, :, -16000:] += 2.5
    inp.target[:] = W.f32_to_bf16_bits(t)
    inp.draft[:] = W.f32_to_bf16_bits(d)
    _parity(inp, label="filtered, skewed chunks")


def test_top_p_tie_group_larger_than_sort_list():
    # 600 tokens share the largest logit, 200 in each statistics chunk: every
    # chunk lists its share, but the cut falls inside a tie group larger than
    # one sort list holds; the lowest ids of the group are kept
    V = 3 * 16384
    rng = np.random.default_rng(17)
    inp = W.synthetic(3, 2, V, dtype="bf16", temperature=1.0, top_p=0.5, seed=17, gen_seed=17)
    t = rng.normal(0, 1, size=(3, 3, V)).astype(np.float32)
    d = (t[:, :2] + rng.normal(0, 0.5, size=(3, 2, V))).astype(np.float32)
    for c in range(3):
        ids = c * 16384 + rng.choice(16384, 200, replace=False)
        t[:, :, ids] = 6.0
        d[:, :, ids] = 6.0
    inp.target[:] = W.f32_to_bf16_bits(t)
    inp.draft[:] = W.f32_to_bf16_bits(d)
    _parity(inp, label="600-way tie at the top, top_p=0.5")


def test_extreme_and_masked_logits():
    inp = W.synthetic(6, 3, 3000, dtype="f32", temperature=0.5, seed=11, gen_seed=11)
    inp.target[0] *= 3000.0            # logits of order 1e4
    inp.draft[0] *= 3000.0
    inp.target[1, :, 100:] = -np.inf   # masked vocabulary
    inp.draft[1, :, 100:] = -np.inf
    inp.draft_tokens[1] = [5, 17, 99]
    inp.target[2, :, ::2] = -np.inf
    _parity(inp, label="extreme / masked")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lane_offsets_moved_up(dtype):
    """Rows whose statistics lanes see their larger logits only in later
    vectors: the first vector of every lane of the chunk all -inf (then the
    lane's offset starts at -inf), or a far larger logit in a later vector
    (the offset moves up and the partial sums rescale)."""
    V = 5000
    first = 256 * (8 if dtype == "bf16" else 4)   # ids of the lanes' first vectors
    inp = W.synthetic(4, 3, V, dtype="f32", temperature=0.7, seed=14, gen_seed=14)
    inp.target[0, :, :first] = -np.inf
    inp.draft[0, :, :first] = -np.inf
    inp.draft_tokens[0] = [first + 17, first + 900, V - 3]
    inp.target[1, :, first + 5::7] += 60.0    # far above each lane's first vector
    inp.draft[1, :, first + 5::7] += 60.0
    inp.target[2, :, :first] -= 40.0
    if dtype == "bf16":
        inp = W.Inputs(inp.workload, inp.step, W.f32_to_bf16_bits(inp.target), W.f32_to_bf16_bits(inp.draft),
                       inp.draft_tokens, inp.draft_len, inp.temperature, inp.top_p, inp.seed)
    _parity(inp, label=f"lane offsets moved up {dtype}")


def test_identical_models_accept_all():
    inp = W.synthetic(10, 5, 4000, dtype="bf16", seed=12, gen_seed=12)
    inp.draft[:] = inp.target[:, :5]
    gpu = run_gpu(inp)
    assert np.all(gpu[1] == 5)
    np.testing.assert_array_equal(gpu[0][:, :5], inp.draft_tokens)
    _parity(inp, label="identical models")


def test_invalid_rows_emit_sentinels():
    inp = W.synthetic(8, 3, 500, dtype="f32", seed=13, gen_seed=13, draft_len=[3, 3, 3, 3, 2, 3, 3, 3])
    inp.target[1, 2, 7] = np.nan          # NaN in a needed target row
    inp.draft[2, 0, 0] = np.inf           # +inf in a needed draft row
    inp.target[3, 0, :] = -np.inf         # a needed row of only -inf
    inp.draft[4, 2, :] = np.nan           # past L = 2: never read
    inp.target[4, 3, :] = np.nan
    inp.draft_tokens[5, 1] = 500          # id out of range
    inp.draft_tokens[6, 2] = -3
    inp.draft_len[7] = 4                  # length out of range
    gpu = run_gpu(inp)
    res = run_oracle(inp)
    for b in (1, 2, 3, 5, 6, 7):
        assert gpu[1][b] == -1 and np.all(gpu[0][b] == -1), b
        assert res.n_accepted[b] == -1
    check_parity(inp, res, gpu)


def test_strided_unaligned_views():
    # logits as views into larger buffers: row starts off the 16-byte grid
    base = W.synthetic(7, 3, 3010, dtype="bf16", temperature=0.8, seed=14, gen_seed=14)
    inp = W.synthetic(7, 3, 3001, dtype="bf16", temperature=0.8, seed=14, gen_seed=14)
    inp.target = np.ascontiguousarray(base.target[:, :, 3:3004])
    inp.draft = np.ascontiguousarray(base.draft[:, :, 5:3006])
    inp.draft_tokens = np.minimum(base.draft_tokens, 3000).astype(np.int32)
    tb = dev_array(base.target)
    db = dev_array(base.draft)
    t = tb[:, :, 3:3004]
    d = db[:, :, 5:3006]
    x = torch.from_numpy(inp.draft_tokens).cuda()
    gpu = run_gpu(inp, tensors=(t, d, x, None))
    res = run_oracle(inp)
    st = check_parity(inp, res, gpu)
    assert st.rows == 7


def test_deterministic_repeats():
    inp = W.make_inputs(2, 3, B=32, V=20000)
    tensors = to_device(inp)
    first = run_gpu(inp, probe=False, tensors=tensors)
    for _ in range(20):
        again = run_gpu(inp, probe=False, tensors=tensors)
        np.testing.assert_array_equal(again[0], first[0])
        np.testing.assert_array_equal(again[1], first[1])


def test_release_then_fresh_calls():
    # spec_verify_release frees every scratch buffer; the next call on the
    # stream allocates anew and returns the same outputs
    inp = W.synthetic(6, 3, 5003, dtype="bf16", temperature=0.8, top_p=0.9, seed=15, gen_seed=15)
    first = run_gpu(inp)
    binding.release()
    again = run_gpu(inp)
    binding.release()
    binding.release()
    third = run_gpu(inp, probe=False)
    for a, b in zip(first, again):
        assert np.array_equal(a, b, equal_nan=True)
    assert np.array_equal(first[0], third[0]) and np.array_equal(first[1], third[1])
    check_parity(inp, run_oracle(inp), again)


def test_stream_argument_and_plain_entry_point():
    inp = W.make_inputs(2, 4, B=8, V=3000)
    t, d, x, dl = to_device(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tok, n = binding.verify(t, d, x, dl, float(inp.temperature), float(inp.top_p), inp.seed)
    s.synchronize()
    ref = run_gpu(inp, probe=True, tensors=(t, d, x, dl))
    np.testing.assert_array_equal(tok.cpu().numpy(), ref[0])
    np.testing.assert_array_equal(n.cpu().numpy(), ref[1])


@pytest.mark.parametrize("top_p", [1.0, 0.6])
def test_graph_capture_replays(top_p):
    """One call captured into a HIP graph and replayed on new inputs copied
    into the captured buffers gives, replay after replay, the outputs of the
    same call made eagerly (the replays reuse the captured record tag, so
    this also checks that every call leaves the scratch ready for the next)."""
    cfg = 4 if top_p < 1.0 else 2
    sets = [W.make_inputs(cfg, s, B=12, V=9000) for s in range(3)]
    T = float(sets[0].temperature)
    seed = 0x5EEDF00D
    stream = torch.cuda.Stream()
    t, d, x, _ = to_device(sets[0])
    out_t = torch.empty((t.shape[0], t.shape[1]), dtype=torch.int32, device="cuda")
    out_n = torch.empty((t.shape[0],), dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        # first call on this stream allocates the scratch: outside capture
        binding.verify(t, d, x, None, T, top_p, seed, stream=stream, out_tokens=out_t, out_n_accepted=out_n)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        binding.verify(t, d, x, None, T, top_p, seed, stream=stream, out_tokens=out_t, out_n_accepted=out_n)
    torch.cuda.synchronize()
    for rep in range(6):
        inp = sets[rep % 3]
        nt, nd, nx, _ = to_device(inp)
        t.copy_(nt)
        d.copy_(nd)
        x.copy_(nx)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_t, got_n = out_t.cpu().numpy(), out_n.cpu().numpy()
        ref_t, ref_n = binding.verify(nt, nd, nx, None, T, top_p, seed)
        torch.cuda.synchronize()
        say(f"[graph] top_p={top_p} replay {rep}: accepted {got_n.tolist()}")
        np.testing.assert_array_equal(got_n, ref_n.cpu().numpy(), err_msg=f"replay {rep}")
        np.testing.assert_array_equal(got_t, ref_t.cpu().numpy(), err_msg=f"replay {rep}")


@pytest.mark.parametrize("runs", [1, 2, 4, 16])
@pytest.mark.parametrize("unroll", [4, 8])
def test_kernel_variants(runs, unroll, monkeypatch):
    """Every compiled variant of the statistics kernel (4 or 8 vectors per
    lane) and of the row pass (items of 1, 2, 4 or 16 runs of 2048 ids)
    against the oracle, with and without top-p; the library picks a variant
    per call from the shapes, the environment forces one here.  Sixteen-run
    items also at a vocabulary of three items, the last one partial."""
    monkeypatch.setenv("SPECVERIFY_STATS_UNROLL", str(unroll))
    monkeypatch.setenv("SPECVERIFY_ROW_RUNS", str(runs))
    for V in ((20011, 70001) if runs == 16 else (20011,)):
        for cfg, top_p in ((2, None), (4, 0.6)):
            inp = W.make_inputs(cfg, 5, B=6, V=V, top_p=top_p)
            _parity(inp, label=f"variant unroll={unroll} runs={runs} cfg={cfg} V={V}")


@pytest.mark.parametrize("top_p", [1.0, 0.9])
def test_large_vocabulary(top_p):
    """A vocabulary twice the batched workload's and not a multiple of the
    chunk (V = 262147: 17 statistics chunks per bf16 row, a ragged last
    vector), with and without top-p."""
    cfg = 4 if top_p < 1.0 else 2
    for step in range(2):
        _parity(W.make_inputs(cfg, 200 + step, B=6, V=262147), label=f"V=262147 top_p={top_p} step {step}")


@pytest.mark.parametrize("band", ["0", "1e-3", "0.05"])
@pytest.mark.parametrize("cfg", [2, 4])
def test_draw_paths_second_round_and_groups(cfg, band, monkeypatch):
    """The exact draw through its rarer paths, forced by SPECVERIFY_AMB_BAND
    (the assumed relative error of the earlier passes' kept-mass ratio):
    0 sends every row to the second round (the row's last item recomputes
    every item's exact mass), 1e-3 leaves ambiguous groups of equal d in many
    items (a holding item with groups is recomputed whole), 0.05 overflows
    the groups (second round again).  The draw is exact on every path."""
    monkeypatch.setenv("SPECVERIFY_AMB_BAND", band)
    for step in range(2):
        inp = W.make_inputs(cfg, 300 + step, B=12, V=30011)
        _parity(inp, label=f"cfg {cfg} SPECVERIFY_AMB_BAND={band}")


@pytest.mark.parametrize("dtype,top_p", [("bf16", 1.0), ("f32", 1.0), ("bf16", 0.9)])
def test_largest_accepted_vocabulary(dtype, top_p):
    """The largest vocabulary, V = 2^21: 256 row-pass items per row (1024 in
    the one-run items of a small batch), whose last arrival finishes the
    draw; no item waits for another, so no residency limit applies.  One
    more id is refused with SV_ESHAPE."""
    V = 1 << 21
    inp = W.synthetic(4, 2, V, dtype=dtype, temperature=0.7, top_p=top_p, seed=90 + int(top_p * 10),
                      gen_seed=V + (dtype == "f32"))
    _parity(inp, label=f"V={V} {dtype} top_p={top_p}")
    if dtype == "f32":
        big = W.synthetic(1, 1, V + 1, dtype="f32", temperature=0.7, seed=91, gen_seed=91)
        with pytest.raises(binding.SpecVerifyError) as err:
            run_gpu(big)
        assert err.value.status == -2
