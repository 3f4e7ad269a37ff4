"""GPU parity of the vocabulary-parallel logits + cross-entropy
(tp_vocab_ce_fwd / _combine / _bwd) against the fp64 oracle on the same seeded
inputs: every rank's logits and aggregates, the combined loss and
log-sum-exp, and each backward rank's input and table gradients, at the
tiny fp32 shape, a ragged bf16 shape, the 8.3B-like hidden size with the
padded GPT-2 vocabulary over 8 ranks, and that shard's full token count
(sampled tokens); plus slice-boundary and out-of-range labels, the empty
batch and determinism."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import compare, f64

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("tensor_transformer_layer_tp_amd")

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()
    yield
    torch.cuda.synchronize()


def tp_shape(w, rank):
    return tp.TpShape.make(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                           head_dim=w.head_dim, tp_rank=rank, tp_size=w.tp_size, dtype=w.dtype)


def run_gpu(w, vocab, inp, bwd_ranks):
    p, T, h = w.tp_size, w.tokens, w.hidden
    n, dt, nan = vocab // p, _DT[w.dtype], float("nan")
    X = inp["X"].cuda()
    labels = inp["labels"].cuda()
    dloss = inp["dloss"].cuda()
    ws = torch.empty(max(tp.tp_vocab_workspace_bytes(tp_shape(w, 0), vocab), 1), dtype=torch.uint8, device="cuda")
    W = {r: inp["W"][r].cuda() for r in inp["W"]}
    logits, stats = {}, {}
    for r in range(p):
        logits[r] = torch.full((T, n), nan, dtype=dt, device="cuda")
        stats[r] = torch.full((3 * T,), nan, dtype=torch.float32, device="cuda")
        tp.tp_vocab_ce_fwd(tp_shape(w, r), vocab, X, W[r], labels, logits[r], stats[r], workspace=ws)
    loss = torch.full((T,), nan, dtype=torch.float32, device="cuda")
    lse = torch.full((T,), nan, dtype=torch.float32, device="cuda")
    tp.tp_vocab_ce_combine(tp_shape(w, 0), [stats[r] for r in range(p)], loss, lse)
    grads = {}
    for r in bwd_ranks:
        dX = torch.full((T, h), nan, dtype=dt, device="cuda")
        dW = torch.full((n, h), nan, dtype=dt, device="cuda")
        tp.tp_vocab_ce_bwd(tp_shape(w, r), vocab, X, W[r], labels, logits[r], lse, dloss, dX, dW, workspace=ws)
        grads[r] = (dX, dW)
    torch.cuda.synchronize()
    return logits, stats, loss, lse, grads


def run_oracle(w, vocab, inp, bwd_ranks, rows=None):
    p, n = w.tp_size, vocab // w.tp_size
    X, labels, dloss = f64(inp["X"]), inp["labels"].numpy().astype(np.int64), f64(inp["dloss"])
    if rows is not None:
        X, labels, dloss = X[rows], labels[rows], dloss[rows]
    Ws = {r: f64(inp["W"][r]) for r in inp["W"]}
    logits = {r: oracle.logits_fwd(X, Ws[r]) for r in range(p)}
    stats = {r: oracle.ce_partial_stats(logits[r], labels, r * n) for r in range(p)}
    loss, lse = oracle.ce_combine([stats[r] for r in range(p)])
    grads = {r: oracle.ce_bwd(X, Ws[r], labels, r * n, lse, dloss)[1:] for r in bwd_ranks}
    return logits, stats, loss, lse, grads


def check(w, got, ref, ranks_logits, bwd_ranks, rows=None):
    sel = (lambda t: t) if rows is None else (lambda t: t[torch.as_tensor(rows, device=t.device)])  # noqa: E731
    T = w.tokens
    for r in ranks_logits:
        compare(f"logits[{r}]", sel(got[0][r]), ref[0][r], w.dtype)
        st = got[1][r].view(3, T)
        for k, name in enumerate(("max", "sumexp", "z")):
            compare(f"{name}[{r}]", sel(st[k]), ref[1][r][k], w.dtype)
    compare("loss", sel(got[2]), ref[2], w.dtype)
    compare("lse", sel(got[3]), ref[3], w.dtype)
    for r in bwd_ranks:
        compare(f"dX[{r}]", sel(got[4][r][0]), ref[4][r][0], w.dtype)
        if rows is None:
            compare(f"dW[{r}]", got[4][r][1], ref[4][r][1], w.dtype)


# name, workload, tokens (batch 1 x seq), vocab, ranks with a backward
CASES = [
    ("c1_fp32_h64_v512_tp2", "tiny_fp32_tp2", 64, 512, (0, 1)),
    ("c2_h1536_v8192_tp4_ragged", "gpt2_1p2b_tp1", 300, 8192, (0, 3)),
    ("c3_h3072_v51200_tp8_1024_tokens", "gpt_8p3b_tp8", 1024, synth.VOCAB_PADDED, (0, 7)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_vocab_ce_matches_oracle(case):
    name, wname, rows, vocab, bwd = case
    w = synth.WORKLOADS[wname].with_(batch=1, seq=rows)
    if w.tp_size == 1:
        w = w.with_(tp_size=4, n_heads=16)
    print(f"\n  [vocab case {name}] T={w.tokens} h={w.hidden} V={vocab} p={w.tp_size}", flush=True)
    inp = synth.draw_vocab(w, vocab, seed=5, dloss="normal")
    got = run_gpu(w, vocab, inp, bwd)
    ref = run_oracle(w, vocab, inp, bwd)
    check(w, got, ref, range(w.tp_size), bwd)


def test_vocab_ce_full_size_8p3b_shard_sampled_tokens():
    # the configuration the benchmark times: 16384 tokens, hidden 3072, vocab 51200
    # over 8 ranks; every rank's forward and the exchange on the GPU, rank 0's
    # backward; the oracle recomputes sampled tokens across all ranks
    w = synth.WORKLOADS["gpt_8p3b_tp8"]
    vocab = synth.VOCAB_PADDED
    print(f"\n  [vocab full] T={w.tokens} h={w.hidden} V={vocab} p={w.tp_size}", flush=True)
    inp = synth.draw_vocab(w, vocab, seed=0, dloss="mean")
    got = run_gpu(w, vocab, inp, (0,))
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 1, w.tokens - 1], rng.choice(w.tokens, 189, replace=False)]))
    ref = run_oracle(w, vocab, inp, (0,), rows=rows)
    check(w, got, ref, (0, w.tp_size - 1), (0,), rows=rows)


def test_vocab_ce_boundary_and_unowned_labels():
    w = synth.WORKLOADS["tiny_fp32_tp2"].with_(batch=1, seq=8, tp_size=4)
    vocab, n = 256, 64
    inp = synth.draw_vocab(w, vocab, seed=7, dloss="normal")
    # first and last id of every slice, and one id past the vocabulary (owned by no rank)
    inp["labels"] = torch.tensor([0, n - 1, n, 2 * n - 1, 2 * n, 3 * n, vocab - 1, vocab], dtype=torch.int32)
    got = run_gpu(w, vocab, inp, range(4))
    ref = run_oracle(w, vocab, inp, range(4))
    check(w, got, ref, range(4), range(4))
    assert torch.equal(got[2][-1], got[3][-1])  # unowned label: loss = lse


def test_vocab_ce_empty_batch_and_determinism():
    w = synth.WORKLOADS["gpt2_1p2b_tp1"].with_(batch=0, seq=16, tp_size=2, n_heads=16)
    inp = synth.draw_vocab(w, 4096, seed=2)
    got = run_gpu(w, 4096, inp, (0, 1))
    for r in (0, 1):
        assert torch.all(got[4][r][1] == 0), "dW of an empty batch must be zero"
    w = synth.WORKLOADS["gpt_8p3b_tp8"].with_(batch=1, seq=700)
    inp = synth.draw_vocab(w, synth.VOCAB_PADDED, seed=3, dloss="normal")
    a = run_gpu(w, synth.VOCAB_PADDED, inp, (2,))
    b = run_gpu(w, synth.VOCAB_PADDED, inp, (2,))
    for x, y in ((a[2], b[2]), (a[3], b[3]), (a[4][2][0], b[4][2][0]), (a[4][2][1], b[4][2][1])):
        assert torch.equal(x, y)
