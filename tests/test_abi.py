"""The C-ABI library on the host: it loads, exports every declared symbol, and
refuses bad arguments with the documented codes before touching the GPU.

No call here reaches a kernel launch: each one fails a check (or is the T = 0
no-op) on the host first, so these run without a GPU.
"""
import ctypes
import os
import re

import pytest

import quantized_weight_prefill_gguf_amd as pf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pf_gemm.h")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced by these calls


@pytest.fixture(scope="module")
def lib():
    return pf.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(pf_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(pf.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_header_enums_match_binding():
    src = open(HEADER).read()
    for name in ["PF_Q4_0", "PF_Q8_0", "PF_PLAIN", "PF_RESIDUAL", "PF_GATE_UP_SWIGLU",
                 "PF_LEG_F32", "PF_LEG_F16", "PF_PATH_AUTO", "PF_PATH_GEMM", "PF_PATH_GEMV",
                 "PF_OK", "PF_E_NULL", "PF_E_QTYPE", "PF_E_EPILOGUE", "PF_E_LEG", "PF_E_SHAPE",
                 "PF_E_ALIGN", "PF_E_ALIAS", "PF_E_LAUNCH", "PF_E_PATH", "PF_E_WORKSPACE",
                 "PF_E_SCRATCH"]:
        m = re.search(r"\b%s\s*=\s*(\d+)" % name, src)
        assert m and int(m.group(1)) == getattr(pf, name), name
    assert int(re.search(r"#define PF_GEMV_MAX_T (\d+)", src).group(1)) == pf.PF_GEMV_MAX_T
    m = re.search(r"#define PF_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", src)
    assert int(m.group(1)) << int(m.group(2)) == pf.PF_NOALLOC_SCRATCH_BYTES


def test_weight_bytes(lib):
    assert lib.pf_weight_bytes(pf.PF_Q4_0, 4096, 4096) == 4096 * 128 * 18
    assert lib.pf_weight_bytes(pf.PF_Q8_0, 4096, 12288) == 4096 * 384 * 34
    assert lib.pf_weight_bytes(pf.PF_Q4_0, 0, 32) == 0
    assert lib.pf_weight_bytes(7, 1, 32) == -pf.PF_E_QTYPE
    assert lib.pf_weight_bytes(pf.PF_IQ4_XS, 3, 512) == 3 * 2 * 136
    assert lib.pf_weight_bytes(pf.PF_IQ4_XS, 3, 288) == -pf.PF_E_SHAPE
    assert lib.pf_weight_bytes(pf.PF_Q4_0, 1, 33) == -pf.PF_E_SHAPE
    assert lib.pf_weight_bytes(pf.PF_Q4_0, -1, 32) == -pf.PF_E_SHAPE
    assert lib.pf_weight_bytes(pf.PF_F16, 3, 64) == 3 * 2 * 64
    assert lib.pf_weight_bytes(pf.PF_Q4_K, 3, 512) == 3 * 2 * 144
    assert lib.pf_weight_bytes(pf.PF_Q5_K, 3, 512) == 3 * 2 * 176
    assert lib.pf_weight_bytes(pf.PF_Q6_K, 3, 512) == 3 * 2 * 210
    assert lib.pf_weight_bytes(pf.PF_Q6_K, 3, 288) == -pf.PF_E_SHAPE   # not whole super-blocks


def test_strerror(lib):
    for code in range(12):
        s = lib.pf_strerror(code).decode()
        assert s.startswith("PF_"), s
    assert lib.pf_strerror(99).decode() == "unknown status"


def test_select_path(lib):
    sel = lib.pf_select_path
    assert sel(pf.PF_Q4_0, 4096, 4096, 0, pf.PF_PLAIN, pf.PF_LEG_F32) == 0
    for T in (1, 2, 8):
        assert sel(pf.PF_Q4_0, 4096, 4096, T, pf.PF_PLAIN, pf.PF_LEG_F32) == pf.PF_PATH_GEMV
    # f16 leg, SwiGLU: the GEMM from five rows on
    for T, want in ((1, pf.PF_PATH_GEMV), (4, pf.PF_PATH_GEMV), (5, pf.PF_PATH_GEMM), (8, pf.PF_PATH_GEMM)):
        assert sel(pf.PF_Q4_0, 4096, 4096, T, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16) == want
    # f16 leg, PLAIN and RESIDUAL: the GEMM from three rows on
    for T, want in ((1, pf.PF_PATH_GEMV), (2, pf.PF_PATH_GEMV), (3, pf.PF_PATH_GEMM), (8, pf.PF_PATH_GEMM)):
        assert sel(pf.PF_Q4_0, 4096, 4096, T, pf.PF_PLAIN, pf.PF_LEG_F16) == want
        assert sel(pf.PF_Q8_0, 4096, 4096, T, pf.PF_RESIDUAL, pf.PF_LEG_F16) == want
    for T in (9, 16, 512, 2048):
        assert sel(pf.PF_Q8_0, 4096, 12288, T, pf.PF_RESIDUAL, pf.PF_LEG_F16) == pf.PF_PATH_GEMM
    # the further types: the GEMV up to 8 rows, then the GEMM; on the f16 leg those the
    # 4-wave GEMM takes (Q4_K, Q5_K, IQ4_XS, Q6_K with k % 512 == 0) cross over as Q4_0
    for qt in (pf.PF_F16, pf.PF_Q4_K, pf.PF_Q5_K, pf.PF_Q6_K, pf.PF_IQ4_XS):
        for k in (4096, 4352):
            f16_gemm = qt != pf.PF_F16 and (qt != pf.PF_Q6_K or k % 512 == 0)
            for leg in (pf.PF_LEG_F32, pf.PF_LEG_F16):
                for epi in (pf.PF_PLAIN, pf.PF_RESIDUAL, pf.PF_GATE_UP_SWIGLU):
                    first = 5 if epi == pf.PF_GATE_UP_SWIGLU else 3
                    for T in (1, 2, 3, 4, 5, 8, 9):
                        early = leg == pf.PF_LEG_F16 and f16_gemm and T >= first
                        want = pf.PF_PATH_GEMM if T > 8 or early else pf.PF_PATH_GEMV
                        assert sel(qt, 4096, k, T, epi, leg) == want, (qt, k, leg, epi, T)
    assert sel(7, 1, 256, 1, 0, 0) == -pf.PF_E_QTYPE
    assert sel(-1, 1, 256, 1, 0, 0) == -pf.PF_E_QTYPE
    assert sel(0, 1, 256, 1, 3, 0) == -pf.PF_E_EPILOGUE
    assert sel(0, 1, 256, 1, 0, 2) == -pf.PF_E_LEG
    assert sel(0, 1, 128, 1, 0, 0) == -pf.PF_E_SHAPE


def _gemm(lib, qtype=0, W=FAKE, n=64, k=256, X=FAKE + 1 << 32, T=16, Y=FAKE + 2 << 32,
          epi=0, leg=0, path=0):
    P = ctypes.c_void_p
    return lib.pf_gemm_path(qtype, P(W), n, k, P(X), T, P(Y), epi, leg, None, path)


def test_gemm_argument_checks(lib):
    W, X, Y = FAKE, FAKE + (1 << 32), FAKE + (2 << 32)
    g = lambda **kw: _gemm(lib, **{**dict(W=W, X=X, Y=Y), **kw})
    assert g(qtype=10) == pf.PF_E_QTYPE
    assert g(qtype=-1) == pf.PF_E_QTYPE
    assert g(epi=3) == pf.PF_E_EPILOGUE
    assert g(leg=2) == pf.PF_E_LEG
    assert g(path=3) == pf.PF_E_PATH
    assert g(path=pf.PF_PATH_GEMV, T=9) == pf.PF_E_PATH
    for bad in [dict(n=0), dict(k=0), dict(k=128), dict(k=288), dict(k=4000), dict(T=-1),
                dict(T=1 << 20, k=4096), dict(n=1 << 30, k=4096, T=1)]:
        assert g(**bad) == pf.PF_E_SHAPE, bad
    assert g(W=0) == pf.PF_E_NULL
    assert g(X=0) == pf.PF_E_NULL
    assert g(Y=0) == pf.PF_E_NULL
    assert g(W=W + 2) == pf.PF_E_ALIGN
    assert g(X=X + 4) == pf.PF_E_ALIGN
    assert g(Y=Y + 8) == pf.PF_E_ALIGN
    # Y overlapping X or W
    assert g(Y=X) == pf.PF_E_ALIAS
    assert g(Y=X + 16 * 256 * 4 - 16) == pf.PF_E_ALIAS
    assert g(Y=W + 16) == pf.PF_E_ALIAS
    assert g(X=Y + 16 * 64 * 4 - 16, Y=Y) == pf.PF_E_ALIAS
    # T = 0: a no-op that succeeds without looking at the pointers
    assert g(T=0) == pf.PF_OK
    assert g(T=0, W=0, X=0, Y=0) == pf.PF_OK
    # the public pf_gemm performs the same checks
    P = ctypes.c_void_p
    assert lib.pf_gemm(0, P(W), 64, 100, P(X), 16, P(Y), 0, 0, None) == pf.PF_E_SHAPE
    assert lib.pf_gemm(0, P(W), 64, 256, P(X), 0, P(Y), 0, 0, None) == pf.PF_OK


def _split_blocks(total, x_bytes, T, n):
    """Number of [T][n] f32 partial-sum blocks (each rounded up to 4 floats) that
    follow x_bytes of fp16 X in a workspace of `total` bytes, or None if it does not
    divide."""
    per = (T * n + 3) // 4 * 4 * 4
    extra = total - x_bytes
    return extra // per if extra > 0 and extra % per == 0 else None


def test_workspace_bytes(lib):
    wb = lib.pf_workspace_bytes
    # the f16 leg's matrix-core GEMM takes k halves per token row, T rounded up to a
    # multiple of 32; the GEMV and the f32 leg none
    assert wb(pf.PF_Q4_0, 12288, 4096, 512, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16) == 512 * 4096 * 2
    # below 256 rows a K split of the narrow down projection stores 2..32 blocks of
    # [T][n] partial sums behind X (X rounded up to 256 bytes)
    assert 2 <= _split_blocks(wb(pf.PF_Q8_0, 4096, 12288, 9, pf.PF_RESIDUAL, pf.PF_LEG_F16),
                              32 * 12288 * 2, 9, 4096) <= 32
    # SwiGLU on up to 64 rows adds G_s [T][2n] f32 (the gate and up products, one block
    # per K split); from 65 rows it does not split
    assert 1 <= _split_blocks(wb(pf.PF_Q4_0, 12288, 4096, 16, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16),
                              32 * 4096 * 2, 16, 24576) <= 32
    assert 1 <= _split_blocks(wb(pf.PF_Q4_0, 12288, 4096, 64, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16),
                              64 * 4096 * 2, 64, 24576) <= 32
    assert wb(pf.PF_Q4_0, 12288, 4096, 65, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16) == 96 * 4096 * 2
    # a K split adds S blocks of [T][n] f32 partial sums behind X (256-byte boundary):
    # 4096^2 at T = 300 is 2 x 22 tiles of 256 x 192, split 4 ways (16 chunks of 256
    # k, at least 4 per split); at T = 512, 43 tiles of 512 x 96, again 4 ways; the
    # down projection (k = 12288, 48 chunks) at T = 512 splits 5 ways (256 / 43); at
    # T = 2048 its 172 tiles need no split.
    xb = 320 * 4096 * 2
    assert wb(pf.PF_Q4_0, 4096, 4096, 300, pf.PF_PLAIN, pf.PF_LEG_F16) == xb + 4 * 300 * 4096 * 4
    assert wb(pf.PF_Q4_0, 4096, 4096, 512, pf.PF_RESIDUAL, pf.PF_LEG_F16) == \
        512 * 4096 * 2 + 4 * 512 * 4096 * 4
    assert wb(pf.PF_Q8_0, 4096, 12288, 512, pf.PF_RESIDUAL, pf.PF_LEG_F16) == \
        512 * 12288 * 2 + 5 * 512 * 4096 * 4
    assert wb(pf.PF_Q8_0, 4096, 12288, 2048, pf.PF_RESIDUAL, pf.PF_LEG_F16) == 2048 * 12288 * 2
    # ragged: X bytes rounded up to 256, each split's block to 4 floats (12 chunks: 3
    # splits)
    assert wb(pf.PF_Q4_0, 1001, 3072, 300, pf.PF_PLAIN, pf.PF_LEG_F16) == \
        320 * 3072 * 2 + 3 * ((300 * 1001 + 3) // 4 * 4) * 4
    assert wb(pf.PF_Q4_0, 17, 256, 300, pf.PF_PLAIN, pf.PF_LEG_F16) == 320 * 256 * 2
    # 5 chunks of k are too few to split in two
    assert wb(pf.PF_Q4_0, 17, 1280, 290, pf.PF_RESIDUAL, pf.PF_LEG_F16) == 320 * 1280 * 2
    assert wb(pf.PF_Q4_0, 4096, 4096, 512, pf.PF_PLAIN, pf.PF_LEG_F32) == 0
    # the further types take no workspace on the f32 leg; on the f16 leg Q4_K, Q5_K,
    # IQ4_XS and Q6_K (k % 512 == 0: rows a multiple of 4 bytes) wherever the GEMM runs
    # (from 3 rows, 5 for SwiGLU; the 4-wave tiles below 256, or up to 128 for Q6_K;
    # the cooperative kernel above), and F16 above 128 rows, take Q4_0's GEMMs and their
    # workspace layout (X, then the split count these types take).
    # Elsewhere on the f16 leg their own GEMM (64- or 128-row x 128-column tiles) splits K
    # through the workspace when the tiles leave the resident slots (3 per CU) idle:
    # 768 / tiles splits, each at least 512 k, at most 16, one [T][rows] f32 block each;
    # SwiGLU up to 64 rows as one PLAIN GEMM over its 2n rows.
    def own_splits(T, n, k, epi):
        if T <= 8 or (epi == pf.PF_GATE_UP_SWIGLU and T > 64):
            return 1
        rows = 2 * n if epi == pf.PF_GATE_UP_SWIGLU else n
        mt = 128 if -(-T // 128) * -(-rows // 128) >= 256 else 64
        tiles = -(-T // mt) * -(-rows // 128)
        return 1 if tiles >= 768 else max(1, min(768 // tiles, k // 512, 16))
    for qt in (pf.PF_F16, pf.PF_Q4_K, pf.PF_Q5_K, pf.PF_Q6_K, pf.PF_IQ4_XS):
        for T in (1, 8, 9, 300, 511, 512, 2048):
            for epi in (pf.PF_PLAIN, pf.PF_RESIDUAL, pf.PF_GATE_UP_SWIGLU):
                kq = qt in (pf.PF_Q4_K, pf.PF_Q5_K, pf.PF_IQ4_XS, pf.PF_Q6_K)
                coop = T > 128 if qt == pf.PF_F16 else (T >= 512 or (kq and T >= (5 if epi == pf.PF_GATE_UP_SWIGLU else 3)))
                sp = own_splits(T, 4096, 4096, epi)
                rows = 8192 if epi == pf.PF_GATE_UP_SWIGLU else 4096
                want = wb(pf.PF_Q4_0, 4096, 4096, T, epi, pf.PF_LEG_F16) if coop else \
                    (sp * ((T * rows + 3) // 4 * 4) * 4 if sp > 1 else 0)
                if qt in (pf.PF_Q6_K, pf.PF_F16) and 256 <= T < 512:
                    # the cooperative kernel's 512-row tile, where Q4_0 takes its 256 x 192
                    want = wb(qt, 4096, 4096, T, epi, pf.PF_LEG_F16)
                    assert want >= -(-T // 32) * 32 * 4096 * 2
                assert wb(qt, 4096, 4096, T, epi, pf.PF_LEG_F16) == want
                assert wb(qt, 4096, 4096, T, epi, pf.PF_LEG_F32) == 0
    # the narrow down projection at T = 32: on Q6_K's own GEMM (k = 12544, 49 super-blocks
    # a row) 32 tiles, 16 splits; on the short-chunk tiles (k = 12288) X, then 32 tiles
    # over 512 slots (two workgroups per CU), 16 splits. Q4_K gate/up at T = 32 on the
    # short-chunk tiles: X, then G [32][24576] in 4 splits (192 tiles of 32 x 128 over 768
    # resident slots, three workgroups per CU, as Q4_0); at 64 rows two workgroups per
    # CU (512 slots): 2 splits
    assert wb(pf.PF_Q6_K, 4096, 12544, 32, pf.PF_RESIDUAL, pf.PF_LEG_F16) == 16 * 32 * 4096 * 4
    assert wb(pf.PF_Q6_K, 4096, 12288, 32, pf.PF_RESIDUAL, pf.PF_LEG_F16) == \
        32 * 12288 * 2 + 16 * 32 * 4096 * 4
    for qt in (pf.PF_Q4_0, pf.PF_Q4_K):
        assert wb(qt, 12288, 4096, 32, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16) == \
            32 * 4096 * 2 + 4 * 32 * 24576 * 4
    assert wb(pf.PF_IQ4_XS, 12288, 4096, 64, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16) == \
        64 * 4096 * 2 + 2 * 64 * 24576 * 4
    # from 129 rows they choose among the 4-wave kernel's tiles without its 256 x 192
    # one: PLAIN 12288 x 4096 at T = 200 takes 256 x 128 tiles split 8 ways where Q4_0
    # and Q8_0 take 256 x 192 split 4 ways
    assert wb(pf.PF_Q4_0, 12288, 4096, 200, pf.PF_PLAIN, pf.PF_LEG_F16) == \
        224 * 4096 * 2 + 4 * 200 * 12288 * 4
    assert wb(pf.PF_Q4_K, 12288, 4096, 200, pf.PF_PLAIN, pf.PF_LEG_F16) == \
        224 * 4096 * 2 + 8 * 200 * 12288 * 4
    # Q6_K and F16 above 128 rows take the cooperative kernel's 512-row tile: 43 tiles of
    # 512 x 96 at T = 300, 4 splits (at least 4 chunks each)
    for qt in (pf.PF_Q6_K, pf.PF_F16):
        assert wb(qt, 4096, 4096, 300, pf.PF_PLAIN, pf.PF_LEG_F16) == 320 * 4096 * 2 + 4 * 300 * 4096 * 4
    # Q6_K rows of an odd number of super-blocks (2-byte aligned rows) keep its own GEMM
    # (512 rows, 4096 columns: 256 tiles, 3 splits)
    assert own_splits(512, 4096, 4352, pf.PF_PLAIN) == 3
    assert wb(pf.PF_Q6_K, 4096, 4352, 512, pf.PF_PLAIN, pf.PF_LEG_F16) == 3 * 512 * 4096 * 4
    assert wb(pf.PF_Q6_K, 4096, 4608, 512, pf.PF_PLAIN, pf.PF_LEG_F16) > 0
    # the GEMV (f16 leg: up to 2 rows, or up to 4 with the SwiGLU epilogue) takes none;
    # from 3 rows the f16 leg's PLAIN and RESIDUAL run the GEMM
    assert wb(pf.PF_Q4_0, 4096, 4096, 2, pf.PF_PLAIN, pf.PF_LEG_F16) == 0
    assert wb(pf.PF_Q4_0, 4096, 4096, 4, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16) == 0
    assert 2 <= _split_blocks(wb(pf.PF_Q4_0, 4096, 4096, 8, pf.PF_PLAIN, pf.PF_LEG_F16),
                              32 * 4096 * 2, 8, 4096) <= 32
    assert 2 <= _split_blocks(wb(pf.PF_Q8_0, 4096, 4096, 3, pf.PF_RESIDUAL, pf.PF_LEG_F16),
                              32 * 4096 * 2, 3, 4096) <= 32
    # a single K chunk cannot split: X alone
    assert wb(pf.PF_Q4_0, 64, 256, 40, pf.PF_PLAIN, pf.PF_LEG_F16) == 64 * 256 * 2
    assert wb(pf.PF_Q4_0, 4096, 4096, 0, pf.PF_PLAIN, pf.PF_LEG_F16) == 0
    assert wb(7, 64, 256, 16, 0, 1) == -pf.PF_E_QTYPE
    assert wb(0, 64, 300, 16, 0, 1) == -pf.PF_E_SHAPE
    assert wb(0, 64, 256, 16, 0, 5) == -pf.PF_E_LEG


def test_gemm_ws_argument_checks(lib):
    P = ctypes.c_void_p
    W, X, Y, WS = FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32)
    n, k, T = 64, 256, 16
    need = 32 * k * 2

    def g(ws=WS, ws_bytes=need, leg=pf.PF_LEG_F16, **kw):
        a = dict(qtype=0, W=W, n=n, k=k, X=X, T=T, Y=Y, epi=0)
        a.update(kw)
        return lib.pf_gemm_ws(a["qtype"], P(a["W"]), a["n"], a["k"], P(a["X"]), a["T"], P(a["Y"]),
                              a["epi"], leg, P(ws), ws_bytes, None)

    assert g(ws=0) == pf.PF_E_WORKSPACE
    assert g(ws_bytes=need - 1) == pf.PF_E_WORKSPACE
    assert g(ws=WS + 8) == pf.PF_E_WORKSPACE
    assert g(ws=X + 16) == pf.PF_E_WORKSPACE
    assert g(ws=Y) == pf.PF_E_WORKSPACE
    assert g(ws=W + 16) == pf.PF_E_WORKSPACE
    assert g(ws=X - need + 16) == pf.PF_E_WORKSPACE
    # the ordinary checks come first and are the same as pf_gemm's
    assert g(qtype=9) == pf.PF_E_QTYPE
    assert g(k=100) == pf.PF_E_SHAPE
    assert g(X=0) == pf.PF_E_NULL
    assert g(Y=X) == pf.PF_E_ALIAS
    assert g(T=0, ws=0, ws_bytes=0) == pf.PF_OK


def test_gemm_ex_argument_checks(lib):
    """pf_gemm_ex: ldy >= n, the strided Y span ((T-1) ldy + n floats) in the alias
    checks, and the workspace rules of pf_gemm_ws when a workspace is given."""
    P = ctypes.c_void_p
    W, X, Y, WS = FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32)
    n, k, T, ldy = 64, 256, 16, 100

    def g(ws=0, ws_bytes=0, leg=pf.PF_LEG_F32, **kw):
        a = dict(qtype=0, W=W, n=n, k=k, X=X, T=T, Y=Y, ldy=ldy, epi=0)
        a.update(kw)
        return lib.pf_gemm_ex(a["qtype"], P(a["W"]), a["n"], a["k"], P(a["X"]), a["T"], P(a["Y"]),
                              a["ldy"], a["epi"], leg, P(ws), ws_bytes, None)

    assert g(ldy=n - 1) == pf.PF_E_SHAPE
    assert g(ldy=0, T=0) == pf.PF_E_SHAPE          # a bad stride is refused even when T = 0
    assert g(T=4096, ldy=1 << 19) == pf.PF_E_SHAPE  # T * ldy >= 2^31
    assert g(T=0) == pf.PF_OK
    span = ((T - 1) * ldy + n) * 4
    assert g(X=Y + span - 16) == pf.PF_E_ALIAS      # X starts inside the last row
    assert g(X=Y + 4 * 80) == pf.PF_E_ALIAS         # X inside the gap after row 0: still Y's span
    assert g(Y=X + T * k * 4 - 16) == pf.PF_E_ALIAS
    assert g(Y=Y + 8) == pf.PF_E_ALIGN
    assert g(qtype=10) == pf.PF_E_QTYPE
    # f16 leg with a workspace: too small, or NULL with a size, is refused
    need = lib.pf_workspace_bytes(0, n, k, T, 0, pf.PF_LEG_F16)
    assert need == 32 * k * 2
    assert g(leg=pf.PF_LEG_F16, ws=WS, ws_bytes=need - 16) == pf.PF_E_WORKSPACE
    assert g(leg=pf.PF_LEG_F16, ws=0, ws_bytes=need) == pf.PF_E_WORKSPACE
    assert g(leg=pf.PF_LEG_F16, ws=Y + 16, ws_bytes=need) == pf.PF_E_WORKSPACE


def test_rmsnorm_workspace_bytes(lib):
    wb = lib.pf_rmsnorm_workspace_bytes
    # 1 / rms per row (rounded up to 256 bytes), then the f16 GEMM's workspace ...
    assert wb(pf.PF_Q4_0, 12288, 4096, 512, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16) == \
        2048 + lib.pf_workspace_bytes(pf.PF_Q4_0, 12288, 4096, 512, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16)
    assert wb(pf.PF_Q4_0, 4096, 4096, 300, pf.PF_PLAIN, pf.PF_LEG_F16) == \
        1280 + lib.pf_workspace_bytes(pf.PF_Q4_0, 4096, 4096, 300, pf.PF_PLAIN, pf.PF_LEG_F16)
    # ... or the normalised rows in f32 for the GEMV and the f32 leg
    assert wb(pf.PF_Q8_0, 4096, 12288, 2, pf.PF_PLAIN, pf.PF_LEG_F16) == 256 + 2 * 12288 * 4
    assert wb(pf.PF_Q8_0, 4096, 12288, 3, pf.PF_GATE_UP_SWIGLU, pf.PF_LEG_F16) == 256 + 3 * 12288 * 4
    assert wb(pf.PF_Q8_0, 4096, 12288, 3, pf.PF_PLAIN, pf.PF_LEG_F16) == \
        256 + lib.pf_workspace_bytes(pf.PF_Q8_0, 4096, 12288, 3, pf.PF_PLAIN, pf.PF_LEG_F16)
    assert wb(pf.PF_Q4_0, 200, 768, 40, pf.PF_RESIDUAL, pf.PF_LEG_F32) == 256 + 40 * 768 * 4
    assert wb(pf.PF_Q4_0, 200, 768, 0, pf.PF_RESIDUAL, pf.PF_LEG_F32) == 0
    assert wb(pf.PF_Q4_0, 200, 700, 4, pf.PF_PLAIN, pf.PF_LEG_F32) == -pf.PF_E_SHAPE


def test_gemm_rmsnorm_argument_checks(lib):
    P = ctypes.c_void_p
    W, X, Y, WS, NW = FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32), FAKE + (4 << 32)
    n, k, T = 64, 256, 16
    need = lib.pf_rmsnorm_workspace_bytes(0, n, k, T, 0, pf.PF_LEG_F32)
    assert need == 256 + T * k * 4

    def g(ws=WS, ws_bytes=need, eps=1e-6, nw=NW, ldy=n, **kw):
        a = dict(qtype=0, W=W, n=n, k=k, X=X, T=T, Y=Y, epi=0, leg=pf.PF_LEG_F32)
        a.update(kw)
        return lib.pf_gemm_rmsnorm(a["qtype"], P(a["W"]), a["n"], a["k"], P(a["X"]), a["T"], P(nw), eps,
                                   P(a["Y"]), ldy, a["epi"], a["leg"], P(ws), ws_bytes, None)

    assert g(eps=float("nan")) == pf.PF_E_SHAPE
    assert g(eps=-1.0) == pf.PF_E_SHAPE
    assert g(eps=float("inf")) == pf.PF_E_SHAPE
    assert g(ldy=n - 4) == pf.PF_E_SHAPE
    assert g(nw=0) == pf.PF_E_NULL
    assert g(nw=NW + 4) == pf.PF_E_ALIGN
    assert g(nw=Y + 16) == pf.PF_E_ALIAS
    assert g(ws=0) == pf.PF_E_WORKSPACE
    assert g(ws_bytes=need - 16) == pf.PF_E_WORKSPACE
    assert g(ws=NW - 16) == pf.PF_E_WORKSPACE          # overlaps norm_w
    assert g(ws=X + 64) == pf.PF_E_WORKSPACE
    assert g(qtype=7) == pf.PF_E_QTYPE
    assert g(T=0, ws=0, ws_bytes=0, nw=0) == pf.PF_OK


def test_lm_head_argmax_argument_checks(lib):
    P = ctypes.c_void_p
    W, x, L, tok = FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32)
    n, k = 1000, 256

    def g(**kw):
        a = dict(qtype=0, W=W, n=n, k=k, x=x, L=L, tok=tok)
        a.update(kw)
        return lib.pf_lm_head_argmax(a["qtype"], P(a["W"]), a["n"], a["k"], P(a["x"]), P(a["L"]),
                                     P(a["tok"]), None)

    assert g(qtype=8) == pf.PF_E_QTYPE
    assert g(k=300) == pf.PF_E_SHAPE
    assert g(n=0) == pf.PF_E_SHAPE
    for name in ("W", "x", "L", "tok"):
        assert g(**{name: 0}) == pf.PF_E_NULL, name
    assert g(L=L + 8) == pf.PF_E_ALIGN
    assert g(tok=tok + 2) == pf.PF_E_ALIGN
    assert g(L=x + 16) == pf.PF_E_ALIAS
    assert g(tok=L + 4 * (n - 1)) == pf.PF_E_ALIAS
    assert g(tok=x) == pf.PF_E_ALIAS


def test_prepared_argument_checks(lib):
    P = ctypes.c_void_p
    W, X, Y, WS = FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32)
    n, k, T = 64, 256, 40
    xneed = 64 * k * 2
    px = lambda **kw: lib.pf_prepare_x(kw.get("qtype", 0), kw.get("k", k), P(kw.get("X", X)), kw.get("T", T),
                                       P(kw.get("ws", WS)), kw.get("wsb", xneed), None)
    assert px(qtype=7) == pf.PF_E_QTYPE
    # the further types have a prepared form where the f16 GEMMs take them (their own
    # GEMM reads f32 X): Q4_K, Q5_K, IQ4_XS, Q6_K with k % 512 == 0, F16 above 128 rows
    for qt in (pf.PF_Q4_K, pf.PF_Q5_K, pf.PF_Q6_K, pf.PF_IQ4_XS):
        assert px(qtype=qt, k=512, X=0) == pf.PF_E_NULL  # past the type check
    assert px(qtype=pf.PF_Q6_K, k=768) == pf.PF_E_QTYPE  # rows of an odd number of super-blocks
    assert px(qtype=pf.PF_F16) == pf.PF_E_QTYPE  # F16 up to 128 rows
    assert px(qtype=pf.PF_F16, T=128) == pf.PF_E_QTYPE
    assert px(qtype=pf.PF_F16, T=129, X=0) == pf.PF_E_NULL
    assert px(qtype=pf.PF_F16, T=0) == pf.PF_OK
    assert px(k=300) == pf.PF_E_SHAPE
    assert px(T=0) == pf.PF_OK
    assert px(X=0) == pf.PF_E_NULL
    assert px(X=X + 4) == pf.PF_E_ALIGN
    assert px(wsb=xneed - 16) == pf.PF_E_WORKSPACE
    assert px(ws=X + 64) == pf.PF_E_WORKSPACE
    need = lib.pf_workspace_bytes(0, n, k, T, 0, pf.PF_LEG_F16)
    gp = lambda **kw: lib.pf_gemm_prepared(kw.get("qtype", 0), P(kw.get("W", W)), kw.get("n", n), k,
                                           kw.get("T", T), P(kw.get("Y", Y)), kw.get("ldy", n), kw.get("epi", 0),
                                           P(kw.get("ws", WS)), kw.get("wsb", need), None)
    for qt in (pf.PF_Q4_K, pf.PF_Q5_K, pf.PF_IQ4_XS):
        assert gp(qtype=qt, W=0) == pf.PF_E_NULL  # past the type check
    assert gp(qtype=pf.PF_F16) == pf.PF_E_QTYPE
    # where pf_gemm_ws runs the GEMV (which reads f32 X) there is no prepared GEMM
    assert gp(T=2) == pf.PF_E_PATH
    assert gp(T=4, epi=pf.PF_GATE_UP_SWIGLU) == pf.PF_E_PATH
    assert gp(ldy=n - 1) == pf.PF_E_SHAPE
    assert gp(epi=4) == pf.PF_E_EPILOGUE
    assert gp(W=0) == pf.PF_E_NULL
    assert gp(Y=Y + 8) == pf.PF_E_ALIGN
    assert gp(Y=W + 16) == pf.PF_E_ALIAS
    assert gp(wsb=need - 16) == pf.PF_E_WORKSPACE
    assert gp(ws=Y + 16) == pf.PF_E_WORKSPACE
    assert gp(T=0) == pf.PF_OK


def test_dequant_argument_checks(lib):
    P = ctypes.c_void_p
    W, out = P(FAKE), P(FAKE + (1 << 32))
    for fn in (lib.pf_dequant_f32, lib.pf_dequant_f16):
        assert fn(7, W, 4, 64, out, None) == pf.PF_E_QTYPE
        assert fn(0, W, 0, 64, out, None) == pf.PF_E_SHAPE
        assert fn(0, W, 4, 48, out, None) == pf.PF_E_SHAPE
        assert fn(0, P(0), 4, 64, out, None) == pf.PF_E_NULL
        assert fn(0, W, 4, 64, P(0), None) == pf.PF_E_NULL
        assert fn(0, P(FAKE + 2), 4, 64, out, None) == pf.PF_E_ALIGN
        assert fn(0, W, 4, 64, P(FAKE + 16), None) == pf.PF_E_ALIAS


def test_binding_refuses_host_tensors():
    import torch
    W = torch.zeros(18 * 8, dtype=torch.uint8)
    X = torch.zeros(1, 256)
    Y = torch.zeros(1, 1)
    with pytest.raises(ValueError):
        pf.gemm(pf.PF_Q4_0, W, 1, 256, X, Y, pf.PF_PLAIN, pf.PF_LEG_F32)


def test_binding_y_view_stride_rules():
    """The strided-Y check of the binding (gemm_ex, gemm_rmsnorm, gemm_prepared):
    the library writes n consecutive floats per row, so a row with more than one
    element must have unit stride, also when T = 1 (a view such as buf[:1, ::2]
    would otherwise have the columns between its elements overwritten)."""
    import torch
    buf = torch.zeros((4, 64), dtype=torch.float32)
    assert pf.y_view_ldy(buf[:, :10], 4, 10) == 64
    assert pf.y_view_ldy(buf[:1, :10], 1, 10) == 10
    assert pf.y_view_ldy(buf[:, 3:4], 4, 1) == 64          # one column: any column stride
    assert pf.y_view_ldy(buf[:1, ::64], 1, 1) == 1
    for bad, T, n in [(buf[:1, ::2], 1, 32), (buf[:, ::2], 4, 32), (buf[:, :10], 4, 11),
                      (buf[:, :10].reshape(-1), 4, 10)]:
        with pytest.raises(ValueError):
            pf.y_view_ldy(bad, T, n)


def test_gemm_noalloc_argument_checks(lib):
    """pf_gemm_noalloc refuses on the host, before its first HIP call (the scratch
    lookup): the codes of pf_gemm, and PF_E_SCRATCH where pf_workspace_bytes()
    exceeds the static scratch."""
    P = ctypes.c_void_p
    W, X, Y = FAKE, FAKE + (1 << 36), FAKE + (2 << 36)
    f16, f32 = pf.PF_LEG_F16, pf.PF_LEG_F32

    def g(qtype=pf.PF_Q4_0, W=W, n=64, k=256, X=X, T=16, Y=Y, epi=pf.PF_PLAIN, leg=f16):
        return lib.pf_gemm_noalloc(qtype, P(W), n, k, P(X), T, P(Y), epi, leg, None)

    assert g(qtype=10) == pf.PF_E_QTYPE
    assert g(epi=7) == pf.PF_E_EPILOGUE
    assert g(leg=3) == pf.PF_E_LEG
    assert g(k=100) == pf.PF_E_SHAPE
    assert g(W=0) == pf.PF_E_NULL
    assert g(X=X + 4) == pf.PF_E_ALIGN
    assert g(Y=X) == pf.PF_E_ALIAS
    assert g(T=0) == pf.PF_OK and g(T=0, W=0, X=0, Y=0) == pf.PF_OK
    # the down projection at T = 4096: 100 MB of fp16 X alone
    need = lib.pf_workspace_bytes(pf.PF_Q8_0, 4096, 12288, 4096, pf.PF_RESIDUAL, f16)
    assert need > pf.PF_NOALLOC_SCRATCH_BYTES
    assert g(qtype=pf.PF_Q8_0, n=4096, k=12288, T=4096, epi=pf.PF_RESIDUAL) == pf.PF_E_SCRATCH
    # the FFN's shapes up to T = 2048 fit
    for qt, n, k, epi in [(pf.PF_Q4_0, 12288, 4096, pf.PF_GATE_UP_SWIGLU),
                          (pf.PF_Q8_0, 4096, 12288, pf.PF_RESIDUAL), (pf.PF_Q4_0, 4096, 4096, pf.PF_PLAIN)]:
        for T in (16, 64, 300, 512, 2048):
            assert 0 <= lib.pf_workspace_bytes(qt, n, k, T, epi, f16) <= pf.PF_NOALLOC_SCRATCH_BYTES
