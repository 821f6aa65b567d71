"""Host-side checks of libfusedproj (no GPU needed, no compute call).

The library loads, exports every function include/fusedproj.h declares, and
every argument check returns its status before any HIP call (fake device
addresses are never dereferenced because validation fails first).  The
tiling logic is checked for the property the bitwise guarantees rest on:
the summation-order fields never depend on the rows of a launch.
"""
import ctypes

import pytest

import projection_gemm_sparse_amd as P
from projection_gemm_sparse_amd import _lib as L

FAKE = 0x7f0000000000  # 256-byte aligned, never dereferenced


def test_exports_every_declared_symbol():
    names = L.header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L._lib, n), n
        assert n in L._SIGS, "binding lacks %s" % n


def test_status_strings():
    for st in range(5):
        assert P.fp_status_str(st) and P.fp_status_str(st) != "unknown status"
    assert P.fp_status_str(99) == "unknown status"


@pytest.mark.parametrize("args", [
    (5, 5120, [1280, 512], 8),      # bad dtype
    (0, 0, [1280, 512], 8),         # K < 1
    (0, 5121, [1280, 512], 8),      # K*2 not a multiple of 16
    (1, 7170, [128], 8),            # K*4 not a multiple of 16
    (0, 5120, [], 8),               # no projection
    (0, 5120, [0, 512], 8),         # empty projection
    (0, 5120, [1] * 17, 8),         # too many projections
    (0, 5120, [1280], 0),           # max_M < 1
    (0, 5120, [1280], 257),         # max_M too large
])
def test_workspace_bytes_rejects(args):
    assert P.fp_workspace_bytes(*args) == 0


def test_workspace_bytes_values():
    # counters (one per possible row block, 256-byte rounded) + partials
    ws1 = P.fp_workspace_bytes(0, 5120, [1280, 512], 8)
    assert ws1 >= 1792 * 4
    ws128 = P.fp_workspace_bytes(0, 5120, [1280, 512], 128)
    assert ws128 > ws1  # MFMA split-K partials for large M
    wsf = P.fp_workspace_bytes(1, 7168, [128, 64], 8)
    st, t = P.fp_default_tiling(1, 7168, 192, 8, 192)
    # the fp32 indexer rows fit one workgroup each: no K split by default
    assert st == 0 and t[3] == 1 and t[1] * 64 * t[2] >= 7168 * 4 // 16
    assert wsf >= 256
    # a K longer than one workgroup covers (16 waves x 64 lanes x 2 chunks)
    st, t = P.fp_default_tiling(0, 32768, 300, 2, 300)
    assert st == 0 and t[3] == 2
    assert P.fp_workspace_bytes(0, 32768, [300], 8) >= 512 + 2 * 300 * 8 * 4


def _create(dtype=0, K=5120, N=(1280, 512), w_cat=FAKE, ws=FAKE, ws_bytes=None, max_M=8):
    if ws_bytes is None:
        ws_bytes = P.fp_workspace_bytes(dtype, K, list(N), max_M)
    return P.fp_plan_create(dtype, K, list(N), None, w_cat, ws, ws_bytes, max_M, 0)


def test_plan_create_validation_before_any_hip_call():
    assert _create(dtype=5)[0] == P.FP_ERR_INVALID_ARG
    assert _create(K=-1)[0] == P.FP_ERR_INVALID_ARG
    assert _create(N=(0,))[0] == P.FP_ERR_INVALID_ARG
    assert _create(max_M=0)[0] == P.FP_ERR_INVALID_ARG
    assert _create(w_cat=0)[0] == P.FP_ERR_INVALID_ARG
    assert _create(ws=0)[0] == P.FP_ERR_INVALID_ARG
    assert _create(K=5124)[0] == P.FP_ERR_UNSUPPORTED          # rows not 16-B aligned
    assert _create(w_cat=FAKE + 16)[0] == P.FP_ERR_UNSUPPORTED  # w_cat not 256-B aligned
    assert _create(ws=FAKE + 64)[0] == P.FP_ERR_UNSUPPORTED
    assert _create(ws_bytes=16)[0] == P.FP_ERR_WORKSPACE
    # null out pointer
    N = (ctypes.c_int64 * 1)(1280)
    assert L._lib.fp_plan_create(0, 5120, 1, N, None, FAKE, FAKE, 1 << 30, 8, None, None) \
        == P.FP_ERR_INVALID_ARG


def test_calls_on_a_stale_or_null_plan():
    for plan in (0, FAKE, 12345678):
        assert P.fp_plan_destroy(plan) == P.FP_ERR_INVALID_ARG
        assert P.fp_supported(plan, 1, FAKE, 5120) == P.FP_ERR_INVALID_ARG
        assert P.fp_forward(FAKE, 1, 5120, plan, 0, [FAKE, FAKE]) == P.FP_ERR_INVALID_ARG
        assert P.fp_forward_separate(FAKE, 1, 5120, plan, 0, [FAKE, FAKE]) == P.FP_ERR_INVALID_ARG
        assert L.fp_forward_noalloc(FAKE, 1, 5120, plan, 0, [FAKE, FAKE]) == P.FP_ERR_INVALID_ARG
        assert P.fp_plan_view(plan, 0)[0] == P.FP_ERR_INVALID_ARG
        assert P.fp_plan_query(plan, 1)[0] == P.FP_ERR_INVALID_ARG
        assert P.fp_plan_set_mfma_min_m(plan, 9) == P.FP_ERR_INVALID_ARG
        assert P.fp_plan_set_tiling(plan, 1, None) == P.FP_ERR_INVALID_ARG
        assert P.fp_plan_get_tiling(plan, 1, 1)[0] == P.FP_ERR_INVALID_ARG


def test_default_tiling_argument_checks():
    assert P.fp_default_tiling(0, 5120, 1792, 0, 1792)[0] == P.FP_ERR_INVALID_ARG
    assert P.fp_default_tiling(0, 5120, 1792, 1, 1793)[0] == P.FP_ERR_INVALID_ARG
    assert P.fp_default_tiling(0, 5120, 1792, 257, 1792)[0] == P.FP_ERR_INVALID_ARG
    assert P.fp_default_tiling(5, 5120, 1792, 1, 1792)[0] == P.FP_ERR_INVALID_ARG
    assert P.fp_default_tiling(0, 5122, 1792, 1, 1792)[0] == P.FP_ERR_UNSUPPORTED
    # fp32 is served for M <= 8 only
    assert P.fp_default_tiling(1, 7168, 192, 9, 192)[0] == P.FP_ERR_UNSUPPORTED


SHAPES = [(0, 5120, (1280, 512)), (1, 7168, (128, 64)), (0, 6144, (2048, 576, 128)),
          (0, 4096, (100, 28, 3)), (1, 1024, (5,))]


@pytest.mark.parametrize("dtype,K,N", SHAPES)
def test_summation_order_independent_of_launch_rows(dtype, K, N):
    """path/kparts/chunks/splits (the summation order) must be the same for
    the fused launch (all rows) and each separate launch (one projection):
    that is what makes fused == separate bitwise."""
    n_total = sum(N)
    maxm = 8 if dtype == 1 else 256
    for M in list(range(1, 17)) + [31, 32, 33, 64, 100, 128, 200, 256]:
        if M > maxm:
            continue
        st, fused = P.fp_default_tiling(dtype, K, n_total, M, n_total)
        assert st == 0, (M, st)
        for n in N:
            st, sep = P.fp_default_tiling(dtype, K, n_total, M, n)
            assert st == 0
            # the fields that fix the summation order: the tile kernel's
            # row tiles per workgroup and register bound are per launch
            order = (lambda t: (t[0], t[3])) if fused[0] == P.FP_PATH_MFMA else (lambda t: t[:4])
            assert order(sep) == order(fused), (M, n, fused, sep)


@pytest.mark.parametrize("dtype,K,N", SHAPES)
def test_default_tiling_covers_k_and_fits_workspace(dtype, K, N):
    n_total = sum(N)
    esize = 2 if dtype == 0 else 4
    kc = K * esize // 16
    maxm = 8 if dtype == 1 else 256
    ws = P.fp_workspace_bytes(dtype, K, list(N), maxm)
    counters = ((n_total * 4 + 255) // 256) * 256
    for M in range(1, maxm + 1):
        st, (path, kp, ch, S, rows, groups) = P.fp_default_tiling(dtype, K, n_total, M, n_total)
        assert st == 0
        if path == P.FP_PATH_MFMA and ch in (3, 4, 6):
            # the ring tile kernel (33 tokens and more, or from 9 tokens on
            # plans of more 64-row blocks than the tile kernels run in one
            # round): 64-row blocks, chunks = stage buffers
            assert (M >= 33 or (M >= 9 and n_total > 1792)) and kp == 4
            assert (ch == 3) == (M > 128)
        elif path == P.FP_PATH_MFMA and ch == 2:
            # the weight-resident tile kernel (17..32 and 65..128 tokens):
            # 64-row blocks, a slice of at most 16 (12) stages of 64 k
            assert (17 <= M <= 32 or 65 <= M <= 128) and kp == 4
            assert -(-(-(-kc // 4) // S) // 2) <= (16 if M <= 32 else 12)
        elif path == P.FP_PATH_MFMA:
            # kparts = row tiles per workgroup, chunks = compiled register
            # bound of k steps (4 pieces of 16 bytes) per slice
            assert 17 <= M <= 32 and kp in (2, 4, 8) and ch in (8, 10, 16, 20, 40)
            n_steps = -(-kc // 4)
            assert -(-n_steps // S) <= ch
        elif path == P.FP_PATH_MFMA_SMALL:
            assert dtype == 0 and 3 <= M <= 24
            assert S == 1 and kp <= 16 and kp * ch * 8 >= kc
            # rows per row group: one tile of 1..8 rows, or two tiles of
            # rows / 2 sharing the activations
            assert (1 <= rows <= 8 or rows in (10, 12, 14, 16)) and groups >= 1
        else:
            assert M <= 8
            assert S * kp * 64 * ch >= kc
            assert (S > 1) == (path == P.FP_PATH_SKINNY_SPLITK)
        if S > 1:
            mt16 = -(-M // 16)
            mcols = (16 * min(b for b in (1, 2, 4, 8, 16) if b >= mt16)
                     if path == P.FP_PATH_MFMA else M)
            assert counters + S * n_total * mcols * 4 <= ws


def test_default_crossover():
    # bf16: vector-ALU kernel up to M = 2, small-M matrix-core kernel for
    # M = 3..24 (one token half up to 8, two to 16, three above), tile
    # kernels above;
    # fp32: vector-ALU kernel (M <= 8)
    for M in range(1, 3):
        assert P.fp_default_tiling(0, 5120, 1792, M, 1792)[1][0] == P.FP_PATH_SKINNY
    for M in range(3, 17):
        assert P.fp_default_tiling(0, 5120, 1792, M, 1792)[1][0] == P.FP_PATH_MFMA_SMALL
    for M in range(1, 9):
        assert P.fp_default_tiling(1, 7168, 192, M, 192)[1][0] in (1, 2)
    # three token halves through M = 24, the tile kernels above
    for M in (17, 20, 24):
        st, t = P.fp_default_tiling(0, 5120, 1792, M, 1792)
        assert t[0] == P.FP_PATH_MFMA_SMALL and t[4] == 7
    for M in (25, 32, 64, 128):
        assert P.fp_default_tiling(0, 5120, 1792, M, 1792)[1][0] == P.FP_PATH_MFMA
    # more rows than one 8-row tile per CU (the three-way fused-A shape):
    # the vector-ALU kernel through M = 4, the small-M kernel with two row
    # tiles of 6 per wave for 5..16 (one or two token halves), the ring
    # tile kernel from 17 on, its 43 row blocks in 11 slices (473
    # workgroups: the busiest CU's share 2/11 against 2/9 with 9 slices)
    for M in range(1, 5):
        assert P.fp_default_tiling(0, 6144, 2752, M, 2752)[1][0] == P.FP_PATH_SKINNY
    for M in range(5, 17):
        st, t = P.fp_default_tiling(0, 6144, 2752, M, 2752)
        assert t[0] == P.FP_PATH_MFMA_SMALL and t[4] == 12 and t[5] == 1
    for M in (17, 32, 48, 64):
        st, t = P.fp_default_tiling(0, 6144, 2752, M, 2752)
        assert t[0] == P.FP_PATH_MFMA and t[1] == 4 and t[2] == 4 and t[3] == 11
    # the ring's slice count from the busiest CU's share among slices of an
    # even number of k steps, at most two workgroups per CU: 41 blocks take
    # 12 slices (492 workgroups), 28 blocks keep 9 (one per CU), K = 7168
    # at 2048 rows 16 (14 steps each), at 4096 rows 8 (not 9: 25 steps,
    # three workgroups on some CUs), K = 4096 at 8192 rows 4; a 192-row
    # plan, one workgroup per CU, is not held to the 16-slice bound
    for M in (17, 64):
        assert P.fp_default_tiling(0, 6144, 2624, M, 2624)[1][3] == 12
        assert P.fp_default_tiling(0, 7168, 2048, M, 2048)[1][3] == 16
        assert P.fp_default_tiling(0, 7168, 4096, M, 4096)[1][3] == 8
        assert P.fp_default_tiling(0, 4096, 8192, M, 8192)[1][3] == 4
    for M in (48, 64):
        assert P.fp_default_tiling(0, 5120, 1792, M, 1792)[1][3] == 9
        assert P.fp_default_tiling(0, 7168, 192, M, 192)[1][3] == 56
    # 25..32 tokens: the weight-resident kernel with balanced slices of one
    # workgroup per CU, or the ring where it reaches an equal or smaller
    # share with more slices
    t = P.fp_default_tiling(0, 5120, 1024, 32, 1024)[1]
    assert t[0] == P.FP_PATH_MFMA and t[2] == 2 and t[3] == 16
    t = P.fp_default_tiling(0, 7168, 2048, 32, 2048)[1]
    assert t[0] == P.FP_PATH_MFMA and t[2] == 4 and t[3] == 16
    t = P.fp_default_tiling(0, 5120, 1792, 32, 1792)[1]
    assert t[0] == P.FP_PATH_MFMA and t[2] == 2 and t[3] == 9
    for n_rows, K in ((1792, 5120), (2624, 6144), (2752, 6144), (2048, 7168), (4096, 4096)):
        for M in (17, 32, 64):
            t = P.fp_default_tiling(0, K, n_rows, M, n_rows)[1]
            if t[0] == P.FP_PATH_MFMA and t[2] == 4:
                steps = -(-K * 2 // 16 // 4)
                assert (-(-steps // t[3])) % 2 == 0, (n_rows, K, M, t)
    # above 64 tokens one slice per CU's share of the 43 row blocks
    for M in (96, 128):
        st, t = P.fp_default_tiling(0, 6144, 2752, M, 2752)
        assert t[0] == P.FP_PATH_MFMA and t[2] == 4 and t[3] == 5
    # long K with two token halves (the small-M workgroup would exceed its
    # thread bound): the tile kernels, not a refusal
    for M in (9, 16):
        assert P.fp_default_tiling(0, 7168, 1536, M, 1536)[1][0] == P.FP_PATH_MFMA
        assert P.fp_default_tiling(0, 7168, 2112, M, 2112)[1][0] == P.FP_PATH_MFMA
    # two row tiles per wave only for workgroups of eight K parts or more
    # (K >= 2048) while a one-round layout exists, up to four small
    # workgroups per CU, ties to fewer row groups: the dense-MLP down
    # projection [6144, 768] takes workgroups of one 8-row tile (three per
    # CU), the three-way fused-A shape (12 K parts) keeps two tiles of 6,
    # and a 65536-row plan (no one-round layout) keeps the largest rows
    for M in (5, 8, 16):
        t = P.fp_default_tiling(0, 768, 6144, M, 6144)[1]
        assert t[0] == P.FP_PATH_MFMA_SMALL and (t[4], t[5]) == (8, 1)
        assert P.fp_default_tiling(0, 6144, 2752, M, 2752)[1][4:6] == (12, 1)
    assert P.fp_default_tiling(0, 1024, 65536, 8, 65536)[1][4:6] == (16, 4)
    # where the small-M kernel starts: from M = 3 at four to eight rows per
    # CU; above eight, from M = 3 only at K <= 4096 up to 25.2 MB of weights;
    # at most two rows per CU never (the vector-ALU kernel through M = 8);
    # three or four rows per CU from M = 3 at K <= 2048
    assert P.fp_default_tiling(0, 5120, 2048, 3, 2048)[1][0] == P.FP_PATH_MFMA_SMALL
    assert P.fp_default_tiling(0, 5120, 2049, 3, 2049)[1][0] == P.FP_PATH_SKINNY
    assert P.fp_default_tiling(0, 2048, 6144, 3, 6144)[1][0] == P.FP_PATH_MFMA_SMALL
    assert P.fp_default_tiling(0, 4096, 6144, 4, 6144)[1][0] == P.FP_PATH_SKINNY
    for M in (1, 3, 5, 8):
        assert P.fp_default_tiling(0, 7168, 512, M, 512)[1][0] == P.FP_PATH_SKINNY
    assert P.fp_default_tiling(0, 2048, 1024, 3, 1024)[1][0] == P.FP_PATH_MFMA_SMALL
    assert P.fp_default_tiling(0, 5120, 1024, 4, 1024)[1][0] == P.FP_PATH_SKINNY
    assert P.fp_default_tiling(0, 5120, 1024, 5, 1024)[1][0] == P.FP_PATH_MFMA_SMALL


def test_epilogue_argument_checks_before_any_hip_call():
    # standalone steps: every refusal happens before a launch
    assert P.fp_rmsnorm(FAKE, -1, 1280, FAKE, 1e-6, FAKE, 0) == P.FP_ERR_INVALID_ARG
    assert P.fp_rmsnorm(FAKE, 0, 1280, FAKE, 1e-6, FAKE, 0) == P.FP_OK  # nothing to do
    assert P.fp_rmsnorm(FAKE, 2, 1280, FAKE, -1.0, FAKE + (1 << 20), 0) == P.FP_ERR_INVALID_ARG
    assert P.fp_rmsnorm(FAKE, 2, 1280, FAKE, float("inf"), FAKE, 0) == P.FP_ERR_INVALID_ARG
    assert P.fp_rmsnorm(FAKE, 2, 1284, FAKE + (1 << 24), 1e-6, FAKE + (2 << 24), 0) \
        == P.FP_ERR_UNSUPPORTED
    assert P.fp_rmsnorm(FAKE, 2, 4096, FAKE + (1 << 24), 1e-6, FAKE + (2 << 24), 0) \
        == P.FP_ERR_UNSUPPORTED  # wider than one wave's four chunks per lane
    assert P.fp_rmsnorm(FAKE + 8, 2, 1280, FAKE + (1 << 24), 1e-6, FAKE + (2 << 24), 0) \
        == P.FP_ERR_UNSUPPORTED  # misaligned
    assert P.fp_rmsnorm(FAKE, 2, 1280, FAKE + (1 << 24), 1e-6, FAKE + 16, 0) \
        == P.FP_ERR_INVALID_ARG  # partial overlap of out and y
    assert P.fp_swiglu(FAKE, FAKE, -1, 768, FAKE, 0) == P.FP_ERR_INVALID_ARG
    assert P.fp_swiglu(FAKE, FAKE, 0, 768, FAKE, 0) == P.FP_OK
    assert P.fp_swiglu(FAKE, FAKE + (1 << 24), 2, 770, FAKE + (2 << 24), 0) \
        == P.FP_ERR_UNSUPPORTED
    assert P.fp_swiglu(FAKE, FAKE + (1 << 24), 2, 768, FAKE + 16, 0) == P.FP_ERR_INVALID_ARG
    # fused forms on a null plan
    assert P.fp_forward_rmsnorm(FAKE, 1, 5120, None, 0, [None, None], 1e-6,
                                [FAKE, FAKE]) == P.FP_ERR_INVALID_ARG
    assert P.fp_forward_swiglu(FAKE, 1, 5120, None, 0, FAKE) == P.FP_ERR_INVALID_ARG


def test_out_dtype_on_a_null_plan():
    assert P.fp_plan_set_out_dtype(None, P.FP_F32) == P.FP_ERR_INVALID_ARG


def test_mxfp8_geometry_checks():
    # packed rows need K a multiple of 512; the dequantiser refuses before any launch
    assert P.fp_workspace_bytes(P.FP_MXFP8, 5120, [1280, 512], 8) > 0
    assert P.fp_workspace_bytes(P.FP_MXFP8, 5136, [1280, 512], 8) == 0
    assert P.fp_mxfp8_to_bf16(FAKE, 2, 528, FAKE + (1 << 24), 0) == P.FP_ERR_UNSUPPORTED
    assert P.fp_mxfp8_to_bf16(FAKE, -1, 512, FAKE + (1 << 24), 0) == P.FP_ERR_INVALID_ARG
    assert P.fp_mxfp8_to_bf16(FAKE, 0, 512, FAKE + (1 << 24), 0) == P.FP_OK
    assert P.fp_mxfp8_to_bf16(FAKE, 4, 512, FAKE + 64, 0) == P.FP_ERR_INVALID_ARG  # overlap
    # vector-ALU kernel up to 4 tokens, the small-M matrix-core kernel for
    # 5..16 (K = 5120: 80 MFMA steps of 64 k over 10 waves), nothing above 16
    st, t = P.fp_default_tiling(P.FP_MXFP8, 5120, 1792, 4, 1792)
    assert st == P.FP_OK and t[0] == P.FP_PATH_SKINNY and t[1] * 64 * t[2] >= 320
    for M in (8, 9, 16):
        st, t = P.fp_default_tiling(P.FP_MXFP8, 5120, 1792, M, 1792)
        assert st == P.FP_OK and t[0] == P.FP_PATH_MFMA_SMALL and t[1] * t[2] * 8 >= 640
    st, _ = P.fp_default_tiling(P.FP_MXFP8, 5120, 1792, 17, 1792)
    assert st == P.FP_ERR_UNSUPPORTED


def test_mxfp4_geometry_checks():
    assert P.fp_workspace_bytes(P.FP_MXFP4, 5120, [1280, 512], 8) > 0
    assert P.fp_workspace_bytes(P.FP_MXFP4, 5136, [1280, 512], 8) == 0
    assert P.fp_mxfp4_to_bf16(FAKE, 2, 528, FAKE + (1 << 24), 0) == P.FP_ERR_UNSUPPORTED
    assert P.fp_mxfp4_to_bf16(FAKE, 0, 512, FAKE + (1 << 24), 0) == P.FP_OK
    assert P.fp_mxfp4_to_bf16(FAKE, 4, 512, FAKE + 64, 0) == P.FP_ERR_INVALID_ARG  # overlap
    st, t = P.fp_default_tiling(P.FP_MXFP4, 5120, 1792, 4, 1792)
    assert st == P.FP_OK and t[0] == P.FP_PATH_SKINNY


def test_stream_read_refusals_before_any_hip_call():
    assert P.fp_stream_read(FAKE, 0, FAKE + (1 << 24), 0) == P.FP_OK  # nothing to read
    assert P.fp_stream_read(FAKE, -16, FAKE + (1 << 24), 0) == P.FP_ERR_INVALID_ARG
    assert P.fp_stream_read(0, 1024, FAKE + (1 << 24), 0) == P.FP_ERR_INVALID_ARG
    assert P.fp_stream_read(FAKE, 1024, 0, 0) == P.FP_ERR_INVALID_ARG
    assert P.fp_stream_read(FAKE + 8, 1024, FAKE + (1 << 24), 0) == P.FP_ERR_UNSUPPORTED
    assert P.fp_stream_read(FAKE, 1000, FAKE + (1 << 24), 0) == P.FP_ERR_UNSUPPORTED
    assert P.fp_stream_read(FAKE, 1 << 31, FAKE + (1 << 32), 0) == P.FP_ERR_UNSUPPORTED
    assert P.fp_stream_read(FAKE, 4096, FAKE + 2048, 0) == P.FP_ERR_INVALID_ARG  # overlap


def test_nvfp4_geometry_and_refusals():
    # rows of K/2 code bytes and K/16 E4M3 scales, K a multiple of 512
    assert P.fp_workspace_bytes(P.FP_NVFP4, 5120, [1280, 512], 8) > 0
    assert P.fp_workspace_bytes(P.FP_NVFP4, 5136, [1280, 512], 8) == 0
    st, t = P.fp_default_tiling(P.FP_NVFP4, 5120, 1792, 4, 1792)
    assert st == P.FP_OK and t[0] == P.FP_PATH_SKINNY
    st, t = P.fp_default_tiling(P.FP_NVFP4, 5120, 1792, 8, 1792)
    assert st == P.FP_OK and t[0] == P.FP_PATH_MFMA_SMALL
    assert P.fp_default_tiling(P.FP_NVFP4, 5120, 1792, 16, 1792)[1][0] == P.FP_PATH_MFMA_SMALL
    assert P.fp_default_tiling(P.FP_NVFP4, 5120, 1792, 17, 1792)[0] == P.FP_ERR_UNSUPPORTED
    # dequantiser: argument checks before any launch
    assert P.fp_nvfp4_to_bf16(FAKE, 2, 528, 1.0, FAKE + (1 << 24), 0) == P.FP_ERR_UNSUPPORTED
    assert P.fp_nvfp4_to_bf16(FAKE, 2, 512, float("nan"), FAKE + (1 << 24), 0) == \
        P.FP_ERR_INVALID_ARG
    assert P.fp_nvfp4_to_bf16(FAKE, 0, 512, 1.0, FAKE + (1 << 24), 0) == P.FP_OK
    assert P.fp_nvfp4_to_bf16(FAKE, 4, 512, 1.0, FAKE + 64, 0) == P.FP_ERR_INVALID_ARG
    # tensor scales on a null plan
    assert P.fp_plan_set_tensor_scales(None, [1.0]) == P.FP_ERR_INVALID_ARG
    assert P.fp_plan_set_tensor_scales(FAKE, [1.0]) == P.FP_ERR_INVALID_ARG


def test_outputs_beyond_32_bit_indexing_are_refused():
    # 8 tokens x 310M rows: an output index m * N + r past 2^31 - 1
    n = 310 * 1000 * 1000
    assert P.fp_default_tiling(P.FP_BF16, 8, n, 8, n)[0] == P.FP_ERR_UNSUPPORTED
    assert P.fp_default_tiling(P.FP_BF16, 8, n, 6, n)[0] == P.FP_OK  # 1.86e9 < 2^31


def _random_shapes(n, seed):
    """Seeded (K, projection sizes) pairs: K a multiple of 8 from 8 to 16384
    and one to four projections of 1..4096 rows, both log-uniform."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        K = 8 * int(round(np.exp(rng.uniform(0.0, np.log(2048.0)))))
        N = tuple(int(round(np.exp(rng.uniform(0.0, np.log(4096.0)))))
                  for _ in range(int(rng.integers(1, 5))))
        out.append((K, N))
    return out


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_default_tiling_on_random_shapes(seed):
    """Every M a plan may be called with gets a default tiling (bf16 up to
    256 tokens, fp32 up to 8, block-scaled weights up to 16), and a launch
    of one projection keeps the summation order of the fused launch, on
    shapes no other test names.  (fp32 at 5..8 tokens with long rows was
    refused before the row layout search kept to layouts that fit the
    kernel's thread bound: [1792, 5120] at M = 5; block-scaled weights at
    9..16 tokens with K = 6656..8192 were refused before two token halves
    took sixteen K steps per wave there.)"""
    for K, N in _random_shapes(40, 1000 + seed):
        n_total = sum(N)
        kmx = max(512, K // 512 * 512)  # block-scaled K: a multiple of 512
        for dtype, maxm, k in ((0, 256, K), (1, 8, K), (P.FP_MXFP8, 16, kmx),
                               (P.FP_MXFP4, 16, kmx), (P.FP_NVFP4, 16, kmx)):
            for M in range(1, maxm + 1):
                st, fused = P.fp_default_tiling(dtype, k, n_total, M, n_total)
                if dtype >= P.FP_MXFP8 and M > 8 and k > 8192:
                    # two token halves of block-scaled weights span K in one
                    # workgroup: longer rows are refused at 9..16 tokens
                    assert st == P.FP_ERR_UNSUPPORTED, (dtype, k, N, M, st)
                    continue
                assert st == 0, (dtype, k, N, M, st)
                order = (lambda t: (t[0], t[3])) if fused[0] == P.FP_PATH_MFMA else (lambda t: t[:4])
                for n in set(N):
                    st, sep = P.fp_default_tiling(dtype, k, n_total, M, n)
                    assert st == 0, (dtype, k, N, M, n, st)
                    assert order(sep) == order(fused), (dtype, k, N, M, n, fused, sep)
