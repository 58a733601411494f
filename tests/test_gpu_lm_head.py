"""GPU checks of pf_lm_head_argmax: the logits against the fp64 CPU oracle to the f32
bar, and the token against the oracle's greedy pick (the largest index among equal
maxima) made over the GPU's own f32 logits, so that both sides take the integer
decision in the same precision. Planted ties (a weight row copied to another
index gives bitwise-equal logits) must resolve to the later index.
"""
import numpy as np
import pytest

import oracle
from oracle import tolerance
from quantized_weight_prefill_gguf_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = synth.Q4_0, synth.Q8_0


def run(gpu, qtype, W, n, k, x):
    import torch
    logits = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    token = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    gpu.lm_head_argmax(qtype, parity.to_dev(W), n, k, parity.to_dev(x), logits, token)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), int(token.cpu().numpy()[0])


def check(qtype, W, n, k, x, logits, token):
    acc = oracle.matmul(qtype, W, n, k, x.reshape(1, k))
    ok, err = tolerance.check_linear(logits.reshape(1, n), acc, oracle.row_norms(qtype, W, n, k),
                                     np.linalg.norm(x.astype(np.float64)).reshape(1), "f32")
    assert ok, "logits parity failed: metric %.3e" % err
    assert token == oracle.argmax_last(logits), (token, oracle.argmax_last(logits))


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("n,k", [(1, 256), (7, 512), (33, 1024), (4099, 2048), (32000, 4096)])
def test_lm_head_argmax(gpu, qtype, n, k):
    wid = 400 + n % 97
    W = synth.quantized_weight(qtype, n, k, workload_id=wid)
    x = synth.activations(1, k, workload_id=wid).reshape(k)
    print("case lm_head qtype=%d n=%d k=%d" % (qtype, n, k), flush=True)
    logits, token = run(gpu, qtype, W, n, k, x)
    check(qtype, W, n, k, x, logits, token)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_lm_head_argmax_planted_ties(gpu, qtype):
    """The winning row copied to a later index wins there; copied to an earlier
    index, the original (later) one still wins."""
    n, k = 3001, 1024
    W = synth.quantized_weight(qtype, n, k, workload_id=410).reshape(n, -1).copy()
    x = synth.activations(1, k, workload_id=410).reshape(k)
    logits, token = run(gpu, qtype, W, n, k, x)
    check(qtype, W, n, k, x, logits, token)
    for dst in (n - 1 if token < n - 1 else 0, 0 if token > 0 else n - 1):
        W2 = W.copy()
        W2[dst] = W[token]
        print("case lm_head tie qtype=%d best=%d copy_to=%d" % (qtype, token, dst), flush=True)
        l2, t2 = run(gpu, qtype, W2, n, k, x)
        assert l2[dst] == l2[token] == l2.max()
        assert t2 == max(dst, token)
        check(qtype, W2, n, k, x, l2, t2)


def test_lm_head_argmax_negative_and_zero_logits(gpu):
    """All logits <= 0 with several exact zeros of either sign: the last zero wins.
    Rows of zero blocks give +0; a row whose scale is -0 gives -0 (q = 8 for Q4_0)."""
    n, k = 40, 256
    W = synth.quantized_weight(Q8_0, n, k, workload_id=420).reshape(n, -1).copy()
    x = np.abs(synth.activations(1, k, workload_id=420).reshape(k))
    # make every row's weights non-positive (q -> -|q|), so every logit is <= 0
    blocks = W.reshape(n, k // 32, 34)
    qs = blocks[:, :, 2:].view(np.int8)
    qs[...] = (-np.abs(qs.astype(np.int16))).clip(-127, 0).astype(np.int8)
    d = blocks[:, :, :2].copy().view(np.float16)
    d[...] = np.abs(d)
    blocks[:, :, :2] = d.view(np.uint8)
    blocks[5, :, 2:] = 0            # +0 logit
    blocks[17, :, :2] = [0, 0x80]   # scale -0: d * q = -0 or +0
    blocks[17, :, 2:] = 0
    blocks[23, :, 2:] = 0           # +0 logit
    W = blocks.reshape(n, -1)
    logits, token = run(gpu, Q8_0, W, n, k, x)
    assert logits.max() == 0.0
    assert token == 23
    check(Q8_0, W, n, k, x, logits, token)
