"""Activations past 2^30 elements: X [5][2^28] f32 (5.4 GB), so row 4 starts 2^32 bytes
in. A 32-bit byte offset would wrap there and read row 0 instead. X and W are zero
outside two 256-wide windows of k (row 0 is nonzero only in the first, row 4 only in
the last), so the exact result is the oracle on those windows alone, and the row
norms of W and X are the windows' norms: the bar is the ordinary one. A wrapped
offset would give row 4 the zeros of row 0's last window instead of its own values.

One test per kernel family that reads f32 X: the f16 leg's 4-wave GEMM without a
workspace (it rounds X while staging it), the f32 GEMM and the GEMV.
"""
import numpy as np
import pytest

import oracle
from oracle import tolerance
from quantized_weight_prefill_gguf_amd import synth

pytestmark = pytest.mark.gpu

K = 1 << 28
T = 5
WIN = 256


@pytest.fixture(scope="module")
def big_case():
    import torch
    qtype, n = synth.Q4_0, 3
    nb = K // 32
    sub_w = synth.quantized_weight(qtype, n, 2 * WIN, workload_id=950).reshape(n, 2 * WIN // 32, 18)
    W = np.zeros((n, nb, 18), np.uint8)           # scale +0, codes 0: every weight -0
    W[:, :WIN // 32] = sub_w[:, :WIN // 32]
    W[:, nb - WIN // 32:] = sub_w[:, WIN // 32:]
    xs = synth.activations(T, 2 * WIN, workload_id=950)
    Xsub = np.zeros((T, 2 * WIN), np.float32)
    Xsub[0, :WIN] = xs[0, :WIN]                   # row 0: first window only
    Xsub[4, WIN:] = xs[4, WIN:]                   # row 4: last window only
    Xsub[2, :WIN] = xs[2, :WIN]
    Xsub[2, WIN:] = xs[2, WIN:]                   # row 2: both
    Xd = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    Xd[:, :WIN] = torch.from_numpy(Xsub[:, :WIN]).cuda()
    Xd[:, K - WIN:] = torch.from_numpy(Xsub[:, WIN:]).cuda()
    Wd = torch.from_numpy(W.reshape(-1)).cuda()
    Wsub = sub_w.reshape(-1)
    acc = oracle.matmul(qtype, Wsub, n, 2 * WIN, Xsub)
    wn = oracle.row_norms(qtype, Wsub, n, 2 * WIN)
    xn = np.linalg.norm(Xsub.astype(np.float64), axis=1)
    torch.cuda.synchronize()
    yield qtype, n, Wd, Xd, acc, wn, xn
    del Xd, Wd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("leg,path", [(1, 1), (0, 1), (0, 2)], ids=["f16_gemm", "f32_gemm", "gemv"])
def test_x_beyond_2_30_elements(gpu, big_case, leg, path):
    import torch
    qtype, n, Wd, Xd, acc, wn, xn = big_case
    print("case large-x leg=%d path=%d" % (leg, path), flush=True)
    Y = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    gpu.gemm(qtype, Wd, n, K, Xd, Y, oracle.PLAIN, leg, path=path)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    ok, err = tolerance.check_linear(y, acc, wn, xn, "f16" if leg == 1 else "f32")
    assert ok, "parity failed: metric %.3e, rows 0 and 4: %s %s" % (err, y[0], y[4])
    assert np.all(y[4] != 0) and np.all(y[[1, 3]] == 0)
