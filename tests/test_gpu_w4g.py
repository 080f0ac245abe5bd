"""GPU parity of the general-grid 4-bit GEMM (group length 64 / 128 / ... / K,
stored zero points, fp16 or bf16 activations) against the CPU oracle, through
the C ABI.

Bars: repacked blobs byte-identical to the independent layout oracle; one-hot
activations reproduce round((q - z) * s) bit-exactly in the activation type
(the kernel forms the exact integer q - z and multiplies by s once in fp32);
codes equal to their zero points give exactly zero (fp16; bf16 up to the fp32
rounding of its post-MFMA zero-point removal); every other output within
the fp16 rule (max|e| <= 2e-3 sqrt(K) rms(C_ref), rel. Frobenius <= 1e-3) or
the bf16 rule (same max term plus 2^-8 max|C_ref|, rel. Frobenius <= 4e-3).
"""

import sys

import numpy as np
import pytest
import torch

import bit_weight_quantized_qgemm_amd as qg
from oracle import compare, layout, ref
from synth import gen

from sampling import block_cols

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ACTS = ["fp16", "bf16"]


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _t(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def _act_t(x, act):
    return _t(x) if act == "fp16" else _t(x.view(np.int16), torch.bfloat16)


def _upload(p):
    s = _t(p["scales"]) if p["act"] == "fp16" else _t(p["scales"].view(np.int16))
    z = None if p["zeros"] is None else _t(p["zeros"])
    return qg.repack_w4g(_t(p["codes"].view(np.int32)), s, z, p["group_size"])


def _run(p, A=None, M=None):
    A = p["A"] if A is None else A
    C = qg.w4g(_act_t(A, p["act"]), _upload(p), p["K"], p["N"], p["group_size"], p["zeros"] is not None)
    return C.cpu().view(torch.int16).numpy().view(np.uint16) if p["act"] == "bf16" else C.cpu().numpy()


def _ok(C_gpu, C_ref, K, act, what):
    r = compare.check_fp16(C_gpu, C_ref, K) if act == "fp16" else compare.check_bf16(C_gpu, C_ref, K)
    assert r["ok"], (what, r)
    return r


@pytest.fixture(autouse=True)
def _reset_plan():
    qg.set_plan_override()
    yield
    qg.set_plan_override()


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("K,N,gs,zeros", [(128, 64, 64, True), (1152, 320, 128, True), (1152, 320, 384, False),
                                          (1024, 1024, 64, False), (4096, 11008, 4096, True)])
def test_repack_w4g_bytes(K, N, gs, zeros, act):
    _say("repack w4g", K, N, gs, zeros, act)
    p = gen.w4g_problem(1, K, N, gs, zeros, act, seed=K ^ N, activations=False)
    blob = _upload(p).cpu().numpy().tobytes()
    assert blob == layout.blob_w4g(p["codes"], p["scales"], p["zeros"], gs, act)


def _one_hot(M, K, rng, act):
    ks = rng.choice(K, size=M, replace=False)
    A = np.zeros((M, K), dtype=np.float16 if act == "fp16" else np.uint16)
    A[np.arange(M), ks] = 1.0 if act == "fp16" else 0x3F80
    return A, ks


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("gs,zeros,M,K,N,force", [(64, True, 16, 1024, 512, None), (128, True, 5, 2048, 256, (1, 8, 2)),
                                                  (256, False, 32, 1024, 384, (2, 16, 1)),
                                                  (1024, True, 20, 1024, 128, (2, 4, 3)),
                                                  (64, False, 33, 512, 256, None)])
def test_w4g_one_hot_bit_exact(act, gs, zeros, M, K, N, force):
    _say("w4g one-hot", act, gs, zeros, M, K, N, force)
    rng = np.random.default_rng(M * 7 + K + gs)
    p = gen.w4g_problem(1, K, N, gs, zeros, act, seed=M + K, activations=False)
    A, ks = _one_hot(M, K, rng, act)
    if force:
        qg.set_plan_override(*force)
    C = _run(p, A)
    q = ref.unpack_u4(p["codes"])
    z = 8 if p["zeros"] is None else p["zeros"][ks // gs].astype(np.int64)
    w = (q[ks] - z).astype(np.float64) * ref.act_to_f64(p["scales"], act)[ks // gs]
    if act == "fp16":
        expect = w.astype(np.float16).view(np.uint16)
        assert np.array_equal(C.view(np.uint16), expect)
    else:
        expect = gen.to_bf16_bits(w.astype(np.float32))   # (q - z) * s is exact in fp32
        assert np.array_equal(C, expect)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("gs", [64, 128, 512])
def test_w4g_codes_at_zero_points_give_zero(act, gs):
    _say("w4g zero", act, gs)
    K, N, M = 1024, 256, 9
    p = gen.w4g_problem(M, K, N, gs, True, act, seed=5)
    q = np.repeat(p["zeros"], gs, axis=0)
    p = dict(p, codes=gen.pack_nibbles_u32(q))
    C = _run(p)
    if act == "fp16":
        # B = q - z is exactly zero
        assert np.all(C.view(np.uint16) & 0x7FFF == 0)   # +0 or -0
    else:
        # bf16 removes the zero point after the MFMA: sum a (128 + z) - (128 + z) sum a
        # cancels up to fp32 rounding of the two sums (~1e-5 here, against rms(C) ~ 1)
        assert np.abs(ref.bf16_to_f64(C)).max() < 1e-3


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("gs,zeros", [(64, False), (64, True), (128, True), (256, True), (2048, False), (2048, True)])
@pytest.mark.parametrize("M", [1, 7, 16, 33])
def test_w4g_gemm(act, gs, zeros, M):
    K, N = 2048, 512
    _say("w4g gemm", act, gs, zeros, M)
    p = gen.w4g_problem(M, K, N, gs, zeros, act, seed=M + gs)
    C = _run(p)
    _ok(C, ref.gemm_w4g(p["A"], p["codes"], p["scales"], p["zeros"], gs, act), K, act, (gs, zeros, M))


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("force", [(1, 4, 1), (2, 8, 2), (2, 16, 1), (1, 4, 5), (2, 4, 7)])
def test_w4g_forced_splits(act, force):
    K, N, M, gs = 4096, 1024, 20, 64
    _say("w4g forced", act, force)
    p = gen.w4g_problem(M, K, N, gs, True, act, seed=13)
    qg.set_plan_override(*force)
    blob = _upload(p)
    A = _act_t(p["A"], act)
    C1 = qg.w4g(A, blob, K, N, gs, True)
    C2 = qg.w4g(A, blob, K, N, gs, True)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    C = C1.cpu().view(torch.int16).numpy().view(np.uint16) if act == "bf16" else C1.cpu().numpy()
    _ok(C, ref.gemm_w4g(p["A"], p["codes"], p["scales"], p["zeros"], gs, act), K, act, force)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("kernel", [1, 3])   # grid entries staged in LDS / loaded per lane
@pytest.mark.parametrize("gs,zeros,M,force", [(64, True, 1, (1, 16, 1)), (64, False, 40, (2, 8, 3)),
                                             (128, True, 17, (2, 4, 2)), (512, False, 7, (1, 8, 5)),
                                             (2048, True, 64, (0, 0, 0))])
def test_w4g_entry_variants(act, kernel, gs, zeros, M, force):
    K, N = 2048, 512
    _say("w4g variant", act, kernel, gs, zeros, M, force)
    p = gen.w4g_problem(M, K, N, gs, zeros, act, seed=M * 3 + gs + kernel)
    qg.set_plan_override(*force, kernel=kernel)
    assert qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros)["kernel"] == kernel
    C = _run(p)
    _ok(C, ref.gemm_w4g(p["A"], p["codes"], p["scales"], p["zeros"], gs, act), K, act, (kernel, gs, zeros, M))


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("gs,zeros", [(128, True), (64, False), (11008, True)])
def test_w4g_7b_layer(act, gs, zeros):
    K, N, M = 11008, 4096, 16
    _say("w4g 7b", act, gs, zeros)
    p = gen.w4g_problem(M, K, N, gs, zeros, act, seed=21)
    C = _run(p)
    _ok(C, ref.gemm_w4g(p["A"], p["codes"], p["scales"], p["zeros"], gs, act), K, act, (gs, zeros))


@pytest.mark.parametrize("kernel", [0, 1, 3])
def test_w4g_70b_up_projection_sampled(kernel):
    # 8192 x 28672 at M = 64 in the automatic plan and in both entry variants;
    # the oracle computes one column of every 16-column block plus a whole
    # staged 128-column tile
    K, N, M, gs, act = 8192, 28672, 64, 64, "fp16"
    _say("w4g 70b sampled", kernel)
    p = gen.w4g_problem(M, K, N, gs, True, act, seed=77)
    qg.set_plan_override(kernel=kernel)
    C = _run(p)
    cols = np.unique(np.concatenate([np.arange(5 * 128, 6 * 128), block_cols(N, seed=7)]))
    ref_cols = ref.gemm_w4g(p["A"], p["codes"][:, cols], p["scales"][:, cols], p["zeros"][:, cols], gs, act)
    _ok(C[:, cols], ref_cols, K, act, ("70b", kernel))


@pytest.mark.parametrize("gs,zeros,act", [(64, True, "fp16"), (128, True, "bf16"), (128, False, "fp16")])
def test_w4g_70b_down_projection_m64_automatic_plan(gs, zeros, act):
    # 28672 x 8192 at M = 64 in the automatic plan: the shape whose launch once
    # asked for all 160 KB of LDS as dynamic memory (leaving none for the
    # kernel's static arrival flag) and aborted the queue; plans now keep 256
    # bytes of headroom. Compared on one column of every 16-column block plus
    # a whole 128-column tile.
    K, N, M = 28672, 8192, 64
    pl = qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros)
    _say("w4g 70b down m64", gs, zeros, act, pl)
    p = gen.w4g_problem(M, K, N, gs, zeros, act, seed=78)
    C = _run(p)
    cols = np.unique(np.concatenate([np.arange(3 * 128, 4 * 128), block_cols(N, seed=8)]))
    z = None if p["zeros"] is None else p["zeros"][:, cols]
    ref_cols = ref.gemm_w4g(p["A"], p["codes"][:, cols], p["scales"][:, cols], z, gs, act)
    _ok(C[:, cols], ref_cols, K, act, ("70b down", gs, zeros))


def test_w4g_matches_w4a16_on_its_grid():
    # group 128 with stored zero points 8, fp16: the W4A16 GEMM within tolerance
    K, N, M = 4096, 1024, 16
    _say("w4g vs w4a16")
    p = gen.w4a16_problem(M, K, N, seed=3)
    blob16 = qg.repack_w4a16(_t(p["codes"].view(np.int32)), _t(p["scales"]))
    C16 = qg.w4a16(_t(p["A"]), blob16, K, N).cpu().numpy()
    blobg = qg.repack_w4g(_t(p["codes"].view(np.int32)), _t(p["scales"]),
                          _t(np.full((K // 128, N), 8, np.uint8)), 128)
    Cg = qg.w4g(_t(p["A"]), blobg, K, N, 128, True).cpu().numpy()
    C_ref = ref.gemm_w4a16(p["A"], p["codes"], p["scales"])
    _ok(Cg, C_ref, K, "fp16", "w4g")
    _ok(C16, C_ref, K, "fp16", "w4a16")


# ----------------------------------------------------------------------------- wide kernel
# fp16 activations on layers whose width is a multiple of 256 may take the wide
# kernel (64 x 256 tiles, 32 x 32 x 16 MFMAs); these cases force it.

@pytest.mark.parametrize("gs,zeros,M,force", [(64, True, 33, (4, 8, 0)), (64, False, 70, (4, 16, 3)),
                                              (128, True, 130, (4, 8, 2)), (256, False, 64, (4, 16, 0)),
                                              (1024, True, 40, (4, 8, 5)), (1024, False, 97, (4, 8, 1)),
                                              (64, True, 50, (2, 8, 0)), (64, False, 128, (2, 8, 3)),
                                              (128, False, 33, (2, 8, 1)), (512, True, 100, (2, 8, 2))])
def test_w4g_wide_one_hot_bit_exact(gs, zeros, M, force):
    K, N, act = 1024, 512, "fp16"
    _say("w4g wide one-hot", gs, zeros, M, force)
    rng = np.random.default_rng(M * 5 + gs)
    p = gen.w4g_problem(1, K, N, gs, zeros, act, seed=M + 2 * K, activations=False)
    A, ks = _one_hot(M, K, rng, act)
    qg.set_plan_override(*force, kernel=2)
    pl = qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros)
    assert pl["kernel"] == 2 and pl["nb"] == force[0]
    C = _run(p, A)
    q = ref.unpack_u4(p["codes"])
    z = 8 if p["zeros"] is None else p["zeros"][ks // gs].astype(np.int64)
    w = (q[ks] - z).astype(np.float64) * ref.act_to_f64(p["scales"], act)[ks // gs]
    assert np.array_equal(C.view(np.uint16), w.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("gs", [64, 128, 512])
def test_w4g_wide_codes_at_zero_points_give_zero(gs):
    K, N, M = 1024, 256, 45
    _say("w4g wide zero", gs)
    p = gen.w4g_problem(M, K, N, gs, True, "fp16", seed=6)
    p = dict(p, codes=gen.pack_nibbles_u32(np.repeat(p["zeros"], gs, axis=0)))
    qg.set_plan_override(kernel=2)
    C = _run(p)
    assert np.all(C.view(np.uint16) & 0x7FFF == 0)


@pytest.mark.parametrize("gs,zeros", [(64, False), (64, True), (128, False), (128, True), (384, True), (3072, False)])
@pytest.mark.parametrize("M,force", [(33, (4, 8, 0)), (64, (4, 16, 4)), (100, (4, 8, 1)), (128, (4, 16, 0)),
                                     (48, (2, 8, 0)), (128, (2, 8, 2))])
def test_w4g_wide_gemm(gs, zeros, M, force):
    K, N, act = 3072, 768, "fp16"     # group length 3072: one group per column
    _say("w4g wide gemm", gs, zeros, M, force)
    p = gen.w4g_problem(M, K, N, gs, zeros, act, seed=M * 11 + gs)
    qg.set_plan_override(*force, kernel=2)
    pl = qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros)
    assert pl["kernel"] == 2 and pl["nb"] == force[0]
    C = _run(p)
    _ok(C, ref.gemm_w4g(p["A"], p["codes"], p["scales"], p["zeros"], gs, act), K, act, (gs, zeros, M, pl))


@pytest.mark.parametrize("gs,zeros", [(128, True), (64, False)])
def test_w4g_wide_70b_down_projection_m128_sampled(gs, zeros):
    # 28672 x 8192 at M = 128 in the automatic plan (two row tiles of the wide
    # kernel, 16 waves); one column of every 16-column block plus a whole
    # 256-column tile against the oracle
    K, N, M, act = 28672, 8192, 128, "fp16"
    pl = qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros)
    _say("w4g wide 70b down m128", gs, zeros, pl)
    assert pl["kernel"] == 2
    p = gen.w4g_problem(M, K, N, gs, zeros, act, seed=79)
    C = _run(p)
    cols = np.unique(np.concatenate([np.arange(5 * 256, 6 * 256), block_cols(N, seed=9)]))
    z = None if p["zeros"] is None else p["zeros"][:, cols]
    ref_cols = ref.gemm_w4g(p["A"], p["codes"][:, cols], p["scales"][:, cols], z, gs, act)
    _ok(C[:, cols], ref_cols, K, act, ("70b down m128", gs, zeros))


@pytest.mark.parametrize("act", ACTS)
def test_w4g_7b_layer_two_row_tiles_automatic_plan(act):
    # 4096 x 11008 at M = 48: fp16 takes the unsplit plan of two 32-row tiles
    # (16-wave two-block workgroups); bf16, whose instance of that shape spills,
    # keeps its scored plan. One column of every 16-column block plus a whole
    # 128-column tile against the oracle.
    K, N, M, gs = 4096, 11008, 48, 128
    pl = qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=True, act_dtype=qg.DT_F16 if act == "fp16" else qg.DT_BF16)
    _say("w4g 7b two row tiles", act, pl)
    if act == "fp16":
        assert (pl["kernel"], pl["mb"], pl["nb"], pl["wpt"], pl["splits"]) == (1, 2, 2, 16, 1)
    p = gen.w4g_problem(M, K, N, gs, True, act, seed=83)
    C = _run(p)
    cols = np.unique(np.concatenate([np.arange(7 * 128, 8 * 128), block_cols(N, seed=10)]))
    ref_cols = ref.gemm_w4g(p["A"], p["codes"][:, cols], p["scales"][:, cols], p["zeros"][:, cols], gs, act)
    _ok(C[:, cols], ref_cols, K, act, ("7b two row tiles", act))
