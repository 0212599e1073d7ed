"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on identical seeded inputs.

Quantization, double quantization and dequantization must match bit for bit; the linear layer's
outputs and gradients must satisfy rel-Frobenius <= 5e-3 and max-abs <= 2e-2 * max|ref| against
the float64 oracle.  Full-size workloads are checked on sampled rows that the oracle computes
directly, plus the full (small) adapter gradients.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_nf4_quantized_codebook_amd as nf4  # noqa: E402

DEV = torch.device("cuda:0")
CB = nf4.nf4_build_codebook()


def _say(msg):
    print(msg, flush=True)


def d16(bits: np.ndarray):
    """bf16 bit patterns (uint16) -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def h16(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t) -> np.ndarray:
    return t.float().cpu().numpy()


def check_tol(name, got, ref):
    rf, ma = oracle.rel_fro(got, ref), oracle.max_abs_ratio(got, ref)
    _say(f"  {name}: rel_fro {rf:.3e}  max_abs/max|ref| {ma:.3e}")
    assert rf <= oracle.REL_FRO_TOL, (name, rf)
    assert ma <= oracle.MAX_ABS_TOL, (name, ma)


# ------------------------------------------------------------------------------------------
# Quantize / double quant / dequant: bit-exact
# ------------------------------------------------------------------------------------------

def _special_tensors():
    out = {}
    W = synth.normal_f32(101, (64, 256), 0.02)
    W[3, :64] = 0.0                                # all-zero block
    W[5, 64:128] = 0.0371                          # constant block
    W[7, 0] = 1e4                                  # single huge outlier
    W[9, 64:128] = synth.normal_f32(102, (64,), 1e-41)   # subnormal block
    W[11, 128:192] = -0.0
    out["specials"] = W.reshape(-1)
    e = np.concatenate([np.tile(CB, 4) * np.float32(2.0 ** k) for k in (-30, -3, 0, 9)])
    out["codebook_round_trip"] = e.astype(np.float32)
    mids = ((CB[:-1].astype(np.float64) + CB[1:]) / 2).astype(np.float32)
    adv = np.concatenate([mids, np.nextafter(mids, np.float32(2)), np.nextafter(mids, np.float32(-2))])
    blk = np.resize(np.concatenate([[np.float32(1.0)], adv]), 64).astype(np.float32)
    out["midpoints"] = np.concatenate([blk * np.float32(s) for s in (1.0, 0.37, 3e-5, 1700.0)])
    out["ragged_odd"] = synth.normal_f32(103, (64 * 5 + 37,), 1.0)
    out["single"] = np.array([0.5], dtype=np.float32)
    return out


def _quant_case(W):
    Wd = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    packed, absmax = nf4.nf4_quantize(Wd, CB)
    torch.cuda.synchronize()
    p_ref, a_ref = oracle.quantize(W, CB)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), a_ref.view(np.uint32))
    return absmax, a_ref


@pytest.mark.parametrize("name", list(_special_tensors().keys()))
def test_quantize_special_tensors_bit_exact(name):
    _say(f"quantize special: {name}")
    W = _special_tensors()[name]
    absmax, a_ref = _quant_case(W)
    q, sc, mean = nf4.nf4_double_quant(absmax)
    c_ref, s_ref, m_ref = oracle.double_quant(a_ref)
    assert np.array_equal(q.cpu().numpy(), c_ref)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert mean.cpu().numpy().view(np.uint32)[0] == np.float32(m_ref).view(np.uint32)


@pytest.mark.parametrize("wl_name", ["tiny", "llama7b_attn"])
def test_quantize_dq_dequant_bit_exact(wl_name):
    wl = synth.WORKLOADS[wl_name]
    lin = wl.linears[0]
    _say(f"quantize+dq+dequant: {wl_name} {lin.N}x{lin.K}")
    W = synth.weight_f32(wl, lin)
    w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), CB)
    q = oracle.quantize_dq(W, CB)
    assert np.array_equal(w.packed.cpu().numpy(), q["packed"])
    assert np.array_equal(w.absmax_q.cpu().numpy(), q["codes"])
    assert np.array_equal(w.absmax_scale.cpu().numpy().view(np.uint32), q["scales"].view(np.uint32))
    assert w.absmax_mean.cpu().numpy()[0] == q["mean"]
    assert np.array_equal(h16(nf4.nf4_dequant(w)).reshape(-1), oracle.dequant_weight(q, CB).reshape(-1))


def test_gemv_weight_dequant_bit_exact_full_size():
    """28672 x 8192 (three summation levels in the double-quant mean)."""
    wl = synth.WORKLOADS["gemv"]
    lin = wl.linears[0]
    _say(f"quantize+dq+dequant: gemv {lin.N}x{lin.K}")
    W = synth.weight_f32(wl, lin)
    w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), CB)
    q = oracle.quantize_dq(W, CB)
    assert np.array_equal(w.packed.cpu().numpy(), q["packed"])
    assert np.array_equal(w.absmax_q.cpu().numpy(), q["codes"])
    assert np.array_equal(w.absmax_scale.cpu().numpy().view(np.uint32), q["scales"].view(np.uint32))
    assert w.absmax_mean.cpu().numpy()[0] == q["mean"]
    got = h16(nf4.nf4_dequant(w)).reshape(-1)
    assert np.array_equal(got, oracle.dequant_weight(q, CB).reshape(-1))


@pytest.mark.parametrize("nb", [1, 255, 257, 1000, 65537, 300000, 4194305])
def test_double_quant_ragged_bit_exact(nb):
    _say(f"double quant nb={nb}")
    a = np.abs(synth.normal_f32(110 + nb % 97, (nb,), 0.05)).astype(np.float32)
    if nb > 600:
        a[256:512] = 0.0371                       # a constant 256-block
    q, sc, mean = nf4.nf4_double_quant(torch.from_numpy(a).to(DEV))
    c_ref, s_ref, m_ref = oracle.double_quant(a)
    assert np.array_equal(q.cpu().numpy(), c_ref)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert mean.cpu().numpy()[0] == m_ref


def test_double_quant_nan_constants_match_oracle():
    """A NaN block constant (an all-NaN weight block) makes the mean NaN, so every centred
    constant is NaN: each group's max then passes over them (scale 0, codes 0), as the oracle's
    does; 8204 groups, so some workgroups encode a second group."""
    nb = 2_100_000
    _say(f"double quant with NaN constants nb={nb}")
    a = np.abs(synth.normal_f32(1234, (nb,), 0.05)).astype(np.float32)
    a[300:304] = np.float32("nan")
    q, sc, mean = nf4.nf4_double_quant(torch.from_numpy(a).to(DEV))
    c_ref, s_ref, m_ref = oracle.double_quant(a)
    assert np.isnan(m_ref) and np.isnan(mean.cpu().numpy()[0])
    assert np.array_equal(q.cpu().numpy(), c_ref)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


# ------------------------------------------------------------------------------------------
# Linear layer: tolerance against the float64 oracle
# ------------------------------------------------------------------------------------------

def _make_layer(M, N, K, r, seed, w_std=0.02, zero_w=False, zero_l2=False):
    W = np.zeros((N, K), np.float32) if zero_w else synth.normal_f32(seed, (N, K), w_std)
    X = synth.to_bf16_bits(synth.normal_f32(seed + 1, (M, K), 1.0))
    L1 = synth.to_bf16_bits(synth.normal_f32(seed + 2, (K, r), 1.0 / r))
    L2 = np.zeros((r, N), np.uint16) if zero_l2 else synth.to_bf16_bits(synth.normal_f32(seed + 3, (r, N), 0.01))
    dY = synth.to_bf16_bits(synth.normal_f32(seed + 4, (M, N), 1.0))
    w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), CB)
    Wd = oracle.dequant_weight(oracle.quantize_dq(W, CB), CB)
    assert np.array_equal(h16(nf4.nf4_dequant(w)), Wd)
    return w, Wd, X, L1, L2, dY


SHAPES = [
    # M, N, K, r
    (8, 256, 256, 8),          # the tiny workload's shape
    (300, 520, 384, 16),       # several tiles, ragged M and N
    (17, 64, 128, 64),         # 17 tokens: the wide GEMV's two token groups, one row group
    (1, 512, 256, 64),
    (4, 256, 512, 32),
    (16, 1024, 1024, 128),
    (513, 264, 640, 24),
    (3, 200, 1344, 16),        # decode-size path: ragged K (not a multiple of 256 or 1024)
    (16, 72, 2112, 64),
    (2, 1032, 3072, 8),
    (1, 3000, 8192, 64),       # decode-size: four waves per row, ragged last row group
    (2, 3000, 11008, 128),     # decode-size: six waves per row (the last part-filled), r = 128
    (4, 1000, 22016, 64),      # decode-size, four tokens: eleven waves per row
    (4, 64, 26624, 8),         # a row too long for one workgroup's waves: the wide GEMV takes it
    (3, 8, 64, 8),             # one quantization block per row, a single row group
    (1, 8192, 16384, 64),      # decode-size: several reduction batches per row stream
    (2, 8192, 16384, 16),
    (8, 3000, 8192, 64),       # 4x4-MFMA decode layout, two token groups, ragged row group
    (12, 2000, 4096, 32),      # four token groups (tokens 12..15 padding), two row streams
    (5, 512, 8192, 16),
    (4, 520, 2048, 128),       # 4x4-MFMA decode layout with r = 128, four row streams
    (3, 1000, 4096, 64),       # 4x4-MFMA, 2-4 tokens: two row streams, ragged last workgroup (8 of 16 rows)
    (7, 1000, 2048, 32),       # 4x4-MFMA, 5-8 tokens: four row streams, each batch's sums in four passes
    (1, 1000, 4096, 128),      # one-token decode layout with r = 128
    (9, 1000, 2048, 16),       # the first token count past the row kernel: the 16x16x32 GEMV
    (1023, 264, 640, 24),      # the last token count of the fused dequant GEMMs, ragged
    # from 1024 tokens on: bf16 expansion of the weight + K-extended bf16 GEMM
    (1024, 520, 384, 16),      # ragged N (the backward's reduction), odd number of K steps
    (1100, 264, 640, 24),      # ragged M and N
    (1040, 1032, 320, 128),    # two LoRA extension steps
    # few output tiles: the products' reductions split over several workgroups per tile
    (32, 4096, 4096, 64),      # wide GEMV forward (two token groups); backward 16 splits
    (24, 1000, 2048, 16),      # wide GEMV, second token group part-filled, ragged row group
    (32, 72, 2112, 64),        # wide GEMV, fewer row groups than the block's four waves
    (33, 2048, 1024, 32),      # wide GEMV, four token groups (three of them padding)
    (64, 72, 2112, 64),        # wide GEMV, 64 tokens, fewer row groups than the block's waves
    (64, 4096, 4096, 64),      # wide GEMV, reduction split, s T reduced beforehand (256 KB of T partials)
    (50, 1000, 4096, 16),      # wide GEMV, fourth token group part-filled, reduction split
    (65, 2048, 1024, 32),      # the first token count of the fused GEMMs: split both ways
    (1, 4096, 8192, 16),       # decode GEMV forward; backward dX split over 8 workgroups
    (200, 1032, 2112, 16),     # fused: K not a multiple of 256, ragged last split both ways
    (700, 2048, 1024, 32),     # fused, three tile rows: 4 splits forward, 8 backward
    (1536, 1024, 2048, 64),    # expanded weight + bf16 GEMM: 8 splits forward, 4 backward
]


@pytest.mark.parametrize("M,N,K,r", SHAPES)
def test_linear_fwd_bwd_parity(M, N, K, r):
    _say(f"linear fwd/bwd M={M} N={N} K={K} r={r} {nf4.qlora_linear_route(M, N, K, r)}")
    s = 16.0 / r
    w, Wd, X, L1, L2, dY = _make_layer(M, N, K, r, seed=200 + M + N)
    Xd, L1d, L2d, dYd = d16(X), d16(L1), d16(L2), d16(dY)
    packed_before = w.packed.clone()
    Y, T = nf4.qlora_linear_fwd(w, Xd, L1d, L2d, s)
    dX, dL1, dL2 = nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, T, s)
    torch.cuda.synchronize()
    Yr, Tr = oracle.forward(X, Wd, L1, L2, s)
    g = oracle.backward(dY, X, Wd, L1, L2, s)
    check_tol("Y", f32(Y), Yr)
    check_tol("T", f32(T), Tr)
    check_tol("dX", f32(dX), g["dX"])
    check_tol("dL1", f32(dL1), g["dL1"])
    check_tol("dL2", f32(dL2), g["dL2"])
    assert torch.equal(w.packed, packed_before)          # the frozen weight is never written
    # T recomputed inside the backward gives the same bits
    dX2, dL12, dL22 = nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, None, s)
    assert torch.equal(dX2, dX) and torch.equal(dL12, dL1) and torch.equal(dL22, dL2)
    # no dX requested
    n, dL13, _ = nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, T, s, need_dX=False)
    assert n is None and torch.equal(dL13, dL1)
    # accumulate into an existing dX
    base = d16(synth.to_bf16_bits(synth.normal_f32(7, (M, K), 1.0)))
    acc = base.clone()
    nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, T, s, dX=acc, accumulate=True)
    torch.cuda.synchronize()
    check_tol("dX+=", f32(acc), g["dX"] + f32(base))


# ------------------------------------------------------------------------------------------
# The 4-bit types NF4 is compared with (Int4, FP4): same entry points, other 16-entry tables
# ------------------------------------------------------------------------------------------

ALT_CB = {"int4": (nf4.nf4_build_int4_codebook, oracle.codebook_int4),
          "fp4": (nf4.nf4_build_fp4_codebook, oracle.codebook_fp4)}


def _alt_cb(kind):
    lib_cb, ref_cb = ALT_CB[kind]
    cb = lib_cb()
    assert np.array_equal(cb.view(np.uint32), ref_cb().view(np.uint32))
    return cb


@pytest.mark.parametrize("kind", ["int4", "fp4"])
def test_alt_codebook_quantize_dq_dequant_bit_exact(kind):
    _say(f"alt codebook quantize/dq/dequant: {kind}")
    cb = _alt_cb(kind)
    c64 = cb.astype(np.float64)
    mids = ((c64[:-1] + c64[1:]) / 2).astype(np.float32)
    adv = np.concatenate([mids, np.nextafter(mids, np.float32(2)), np.nextafter(mids, np.float32(-2)),
                          np.float32([1e-30, -1e-30, 1e-8, -1e-8, 0.0, -0.0])])
    blk = np.resize(np.concatenate([[np.float32(1.0)], adv]), 64).astype(np.float32)
    W = np.concatenate([blk * np.float32(sc) for sc in (1.0, 0.37, 3e-5, 1700.0)] +
                       [np.tile(cb, 4) * np.float32(2.0 ** -3), np.zeros(64, np.float32),
                        synth.normal_f32(131, (520 * 384,), 0.02)]).astype(np.float32)
    W = W[: (W.size // 64) * 64]
    Wd = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    packed, absmax = nf4.nf4_quantize(Wd, cb)
    torch.cuda.synchronize()
    p_ref, a_ref = oracle.quantize(W, cb)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), a_ref.view(np.uint32))
    if kind == "fp4":     # the second zero slot (code 8) is never produced
        codes = oracle.unpack(p_ref, W.size)
        assert not np.any(codes == 8)
    w = nf4.NF4Weight.from_float(Wd.reshape(-1, 64), cb)
    q = oracle.quantize_dq(W.reshape(-1, 64), cb)
    assert np.array_equal(w.absmax_q.cpu().numpy(), q["codes"])
    assert np.array_equal(h16(nf4.nf4_dequant(w)).reshape(-1), oracle.dequant_weight(q, cb).reshape(-1))


# ---- the integer second level (eq. (1) at 8 bits on the centred constants) ----

@pytest.mark.parametrize("case", ["normal", "heavy_tail", "constant", "ragged"])
def test_int8_double_quant_dequant_bit_exact(case):
    _say(f"int8 double quant: {case}")
    if case == "normal":
        W = synth.normal_f32(151, (520, 384), 0.02)
    elif case == "heavy_tail":
        W = synth.heavy_tail_f32(152, 153, (1024, 1024), 0.02, 0.2, 0.01)
    elif case == "constant":
        W = np.tile(np.float32([0.03, -0.01] * 32), (64, 1))        # every block's absmax 0.03
    else:
        W = synth.normal_f32(154, (777, 64), 0.05)                  # 777 blocks: ragged 256-groups
    w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), CB, dq_format="int8")
    q = oracle.quantize_dq(W, CB, fmt="int8")
    assert np.array_equal(w.packed.cpu().numpy(), q["packed"])
    assert np.array_equal(w.absmax_q.cpu().numpy(), q["codes"])
    assert np.array_equal(w.absmax_scale.cpu().numpy().view(np.uint32), q["scales"].view(np.uint32))
    assert w.absmax_mean.cpu().numpy()[0] == q["mean"]
    assert np.array_equal(h16(nf4.nf4_dequant(w)).reshape(-1), oracle.dequant_weight(q, CB).reshape(-1))
    if case == "constant":
        assert np.all(q["codes"] == 0)


@pytest.mark.parametrize("M,N,K,r", [(1, 3000, 8192, 64), (4, 520, 2048, 128), (12, 2000, 4096, 32),
                                     (300, 520, 384, 16), (1100, 264, 640, 24)])
@pytest.mark.parametrize("table", ["nf4", "fp4"])
def test_int8_double_quant_linear_parity(M, N, K, r, table):
    _say(f"int8 DQ linear: {table} M={M} N={N} K={K} r={r}")
    CB = globals()["CB"] if table == "nf4" else _alt_cb("fp4")
    s = 16.0 / r
    seed = 950 + M + N
    W = synth.normal_f32(seed, (N, K), 0.02)
    X = synth.to_bf16_bits(synth.normal_f32(seed + 1, (M, K), 1.0))
    L1 = synth.to_bf16_bits(synth.normal_f32(seed + 2, (K, r), 1.0 / r))
    L2 = synth.to_bf16_bits(synth.normal_f32(seed + 3, (r, N), 0.01))
    dY = synth.to_bf16_bits(synth.normal_f32(seed + 4, (M, N), 1.0))
    w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), CB, dq_format="int8")
    Wq = oracle.dequant_weight(oracle.quantize_dq(W, CB, fmt="int8"), CB)
    assert np.array_equal(h16(nf4.nf4_dequant(w)), Wq)
    Xd, L1d, L2d, dYd = d16(X), d16(L1), d16(L2), d16(dY)
    Y, T = nf4.qlora_linear_fwd(w, Xd, L1d, L2d, s)
    dX, dL1, dL2 = nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, T, s)
    torch.cuda.synchronize()
    Yr, _ = oracle.forward(X, Wq, L1, L2, s)
    g = oracle.backward(dY, X, Wq, L1, L2, s)
    check_tol("Y", f32(Y), Yr)
    check_tol("dX", f32(dX), g["dX"])
    check_tol("dL1", f32(dL1), g["dL1"])
    check_tol("dL2", f32(dL2), g["dL2"])


@pytest.mark.parametrize("dist", ["normal", "heavy_tail"])
@pytest.mark.parametrize("kind", ["nf4", "int4", "fp4"])
@pytest.mark.parametrize("dq", ["e4m3", "int8", "none"])
def test_quant_error_statistics_match_oracle(dist, kind, dq):
    """The quantization-error workload (bench.py --qerror) on a 1024 x 1024 weight: statistics from
    the library's quantize / double quant / dequant against the oracle's."""
    import bench
    _say(f"quant error: {dist} {kind} dq={dq}")
    cb = nf4.nf4_build_codebook() if kind == "nf4" else _alt_cb(kind)
    W = (synth.normal_f32(141, (1024, 1024), 0.02) if dist == "normal"
         else synth.heavy_tail_f32(141, 142, (1024, 1024), 0.02, 0.2, 0.01))
    fmt = "e4m3" if dq == "none" else dq
    got = bench.qerror_gpu(torch, nf4, torch.from_numpy(W).to(DEV), cb, dq != "none", fmt)
    ref = oracle.quant_error(W, cb, dq != "none", fmt)
    assert np.array_equal(got["occupancy"], ref["occupancy"])
    assert got["max_abs"] == ref["max_abs"]
    assert abs(got["mse"] - ref["mse"]) <= 1e-12 * ref["mse"]
    assert abs(got["entropy_bits"] - ref["entropy_bits"]) <= 1e-12
    assert abs(got["bits_per_param"] - ref["bits_per_param"]) <= 32.0 / W.size   # + the stored mean


ALT_SHAPES = [
    (1, 3000, 8192, 64),       # one-token decode layout
    (4, 520, 2048, 128),       # 4x4-MFMA decode layout
    (12, 2000, 4096, 32),      # 16x16x32 GEMV
    (300, 520, 384, 16),       # fused dequant GEMM
    (1100, 264, 640, 24),      # bf16 expansion + K-extended GEMM
]


@pytest.mark.parametrize("kind", ["int4", "fp4"])
@pytest.mark.parametrize("M,N,K,r", ALT_SHAPES)
def test_alt_codebook_linear_parity(kind, M, N, K, r):
    _say(f"alt codebook linear: {kind} M={M} N={N} K={K} r={r}")
    cb = _alt_cb(kind)
    s = 16.0 / r
    seed = 900 + M + N
    W = synth.normal_f32(seed, (N, K), 0.02)
    X = synth.to_bf16_bits(synth.normal_f32(seed + 1, (M, K), 1.0))
    L1 = synth.to_bf16_bits(synth.normal_f32(seed + 2, (K, r), 1.0 / r))
    L2 = synth.to_bf16_bits(synth.normal_f32(seed + 3, (r, N), 0.01))
    dY = synth.to_bf16_bits(synth.normal_f32(seed + 4, (M, N), 1.0))
    w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), cb)
    Wq = oracle.dequant_weight(oracle.quantize_dq(W, cb), cb)
    assert np.array_equal(h16(nf4.nf4_dequant(w)), Wq)
    Xd, L1d, L2d, dYd = d16(X), d16(L1), d16(L2), d16(dY)
    Y, T = nf4.qlora_linear_fwd(w, Xd, L1d, L2d, s)
    dX, dL1, dL2 = nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, T, s)
    torch.cuda.synchronize()
    Yr, Tr = oracle.forward(X, Wq, L1, L2, s)
    g = oracle.backward(dY, X, Wq, L1, L2, s)
    check_tol("Y", f32(Y), Yr)
    check_tol("dX", f32(dX), g["dX"])
    check_tol("dL1", f32(dL1), g["dL1"])
    check_tol("dL2", f32(dL2), g["dL2"])


@pytest.mark.parametrize("M,N,K", [(1024, 520, 384), (1088, 264, 1024), (300, 264, 256)])
def test_one_hot_rows_select_the_weight_bit_exact(M, N, K):
    """L2 = 0 and one-hot activations: every output is one dequantized weight times 1.0 plus exact
    zeros, so the forward gives deq(W)^T and the backward deq(W) bit for bit.  From 1024 tokens this
    pins the bf16 expansion of the weight in both layouts (rows for the forward, transposed for the
    backward) through the GEMMs; below it, the fused dequantization."""
    _say(f"one-hot M={M} N={N} K={K}")
    r, s = 16, 0.5
    w, Wd, _, L1, L2, _ = _make_layer(M, N, K, r, seed=500 + M, zero_l2=True)
    X = np.zeros((M, K), np.float32)
    X[np.arange(min(M, K)), np.arange(min(M, K))] = 1.0
    dY = np.zeros((M, N), np.float32)
    dY[np.arange(min(M, N)), np.arange(min(M, N))] = 1.0
    Xd, dYd = d16(synth.to_bf16_bits(X)), d16(synth.to_bf16_bits(dY))
    Y, T = nf4.qlora_linear_fwd(w, Xd, d16(L1), d16(L2), s)
    dX, _, _ = nf4.qlora_linear_bwd(w, dYd, Xd, d16(L1), d16(L2), T, s)
    torch.cuda.synchronize()
    Wd2 = Wd.reshape(N, K)
    k, n = min(M, K), min(M, N)
    assert np.array_equal(h16(Y)[:k], Wd2.T[:k])
    assert not h16(Y)[k:].any()
    assert np.array_equal(h16(dX)[:n], Wd2[:n])


@pytest.mark.parametrize("M,N,K,r", [(64, 256, 256, 8), (40, 520, 384, 16)])
def test_lora_branch_alone(M, N, K, r):
    """W = 0 exactly: Y and dX are the pure LoRA terms (the branch is checked on its own)."""
    _say(f"lora branch alone M={M} N={N} K={K} r={r}")
    s = 2.0
    w, Wd, X, L1, L2, dY = _make_layer(M, N, K, r, seed=300 + M, zero_w=True)
    assert np.all(oracle.bf16_to_f32(Wd) == 0)
    Xd, L1d, L2d, dYd = d16(X), d16(L1), d16(L2), d16(dY)
    Y, T = nf4.qlora_linear_fwd(w, Xd, L1d, L2d, s)
    dX, dL1, dL2 = nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, T, s)
    torch.cuda.synchronize()
    Yr, _ = oracle.forward(X, Wd, L1, L2, s)
    g = oracle.backward(dY, X, Wd, L1, L2, s)
    check_tol("Y(lora)", f32(Y), Yr)
    check_tol("dX(lora)", f32(dX), g["dX"])


def test_base_branch_alone():
    """L2 = 0: Y is the dequantized product alone."""
    M, N, K, r = 96, 512, 512, 16
    _say("base branch alone")
    w, Wd, X, L1, L2, dY = _make_layer(M, N, K, r, seed=400, zero_l2=True)
    Y, _ = nf4.qlora_linear_fwd(w, d16(X), d16(L1), d16(L2), 1.0)
    torch.cuda.synchronize()
    ref = oracle.bf16_to_f32(X).astype(np.float64) @ oracle.bf16_to_f32(Wd).astype(np.float64).T
    check_tol("Y(base)", f32(Y), ref)


def test_full_size_attention_projection_sampled():
    """LLaMA-7B attention projection at full size, the bench's launch configuration."""
    wl = synth.WORKLOADS["llama7b_attn"]
    lin = wl.linears[0]
    M, N, K, r, s = wl.M, lin.N, lin.K, wl.r, wl.scale
    _say(f"full size {wl.name}: M={M} N={N} K={K} r={r}")
    W = synth.weight_f32(wl, lin)
    l1, l2 = synth.lora_f32(wl, lin)
    L1, L2 = synth.to_bf16_bits(l1), synth.to_bf16_bits(l2)
    X = synth.to_bf16_bits(synth.x_f32(wl))
    dY = synth.to_bf16_bits(synth.dy_f32(wl, M, N))
    w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), CB)
    Wd = oracle.dequant_weight(oracle.quantize_dq(W, CB), CB)
    Xd, L1d, L2d, dYd = d16(X), d16(L1), d16(L2), d16(dY)
    Y, T = nf4.qlora_linear_fwd(w, Xd, L1d, L2d, s)
    dX, dL1, dL2 = nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, T, s)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(M, 48, replace=False))
    rows = np.unique(np.concatenate([rows, [0, M - 1]]))
    Yr, _ = oracle.forward_rows(X, Wd, L1, L2, s, rows)
    check_tol("Y[rows]", f32(Y)[rows], Yr)
    g = oracle.backward_rows(dY, X, Wd, L1, L2, s, rows)
    check_tol("dX[rows]", f32(dX)[rows], g["dX"])
    check_tol("T", f32(T), g["T"])
    check_tol("dL2", f32(dL2), g["dL2"])
    check_tol("dL1", f32(dL1), g["dL1"])
    # deterministic: a second run gives the same bits
    Y2, _ = nf4.qlora_linear_fwd(w, Xd, L1d, L2d, s)
    dX2, dL12, dL22 = nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, T, s)
    assert torch.equal(Y, Y2) and torch.equal(dX, dX2) and torch.equal(dL1, dL12) and torch.equal(dL2, dL22)


def test_expanded_weight_past_2_gib_sampled():
    """From 1024 tokens the weight is expanded to bf16 before the GEMMs; here that copy is 2 GiB
    (W 32768 x 32768, 1024 tokens, r = 16), past what 32-bit buffer offsets from the base reach.

    W is a seeded 2048-row block repeated 16 times down the rows.  Quantization works per 64-block
    and the 256-groups of the second level align with the repeats (one repeat holds 2^20 blocks),
    so codes, constants and deq(W) repeat as well -- the test checks exactly that on the GPU's
    storage against the oracle's (computed on the whole weight's block constants), which lets the
    oracle's references be assembled from one 2048-row repeat: outputs by column range, the
    backward summed over the 16 column ranges of dY."""
    M, N, K, r, s = 1024, 32768, 32768, 16, 1.0
    tile = 2048
    nt = N // tile
    _say(f"expanded weight past 2 GiB: M={M} N={N} K={K} r={r}")
    Wt = synth.normal_f32(1600, (tile, K), 0.02)
    Wdev = torch.from_numpy(Wt).to(DEV).repeat(nt, 1)
    w = nf4.NF4Weight.from_float(Wdev, CB)
    del Wdev
    torch.cuda.synchronize()
    pt, at = oracle.quantize(Wt, CB)
    assert np.array_equal(w.packed.cpu().numpy(), np.tile(pt, nt))
    a_full = np.tile(at, nt)
    codes, scales, mean = oracle.double_quant(a_full)
    nbt = at.size
    assert np.array_equal(codes, np.tile(codes[:nbt], nt)) and np.array_equal(scales, np.tile(scales[:nbt // 256], nt))
    assert np.array_equal(w.absmax_q.cpu().numpy(), codes)
    assert np.array_equal(w.absmax_scale.cpu().numpy().view(np.uint32), scales.view(np.uint32))
    assert w.absmax_mean.cpu().numpy()[0] == mean
    Wd_t = oracle.dequant(pt, codes[:nbt], scales[:nbt // 256], mean, tile * K, CB).reshape(tile, K)
    X = synth.to_bf16_bits(synth.normal_f32(1601, (M, K), 1.0))
    L1 = synth.to_bf16_bits(synth.normal_f32(1602, (K, r), 1.0 / r))
    L2 = synth.to_bf16_bits(synth.normal_f32(1603, (r, N), 0.01))
    dY = synth.to_bf16_bits(synth.normal_f32(1604, (M, N), 1.0))
    Xd, L1d, L2d, dYd = d16(X), d16(L1), d16(L2), d16(dY)
    Y, T = nf4.qlora_linear_fwd(w, Xd, L1d, L2d, s)
    dX, dL1, dL2 = nf4.qlora_linear_bwd(w, dYd, Xd, L1d, L2d, T, s)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(9).choice(M, 24, replace=False), [0, M - 1]]))
    Yr = np.empty((rows.size, N))
    dXr, dL1r, dL2r = 0.0, 0.0, np.empty((r, N))
    for t in range(nt):
        c = slice(t * tile, (t + 1) * tile)
        Yr[:, c], _ = oracle.forward_rows(X, Wd_t, L1, L2[:, c], s, rows)
        g = oracle.backward_rows(dY[:, c], X, Wd_t, L1, L2[:, c], s, rows)
        dXr = dXr + g["dX"]
        dL1r = dL1r + g["dL1"]
        dL2r[:, c] = g["dL2"]
    check_tol("Y[rows]", f32(Y)[rows], Yr)
    check_tol("dX[rows]", f32(dX)[rows], dXr)
    check_tol("dL1", f32(dL1), dL1r)
    check_tol("dL2", f32(dL2), dL2r)


# ------------------------------------------------------------------------------------------
# SwiGLU glue
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [8, 1000, 4096 * 3 + 5])
def test_swiglu_parity(n):
    g = synth.to_bf16_bits(synth.normal_f32(500, (n,), 2.0))
    u = synth.to_bf16_bits(synth.normal_f32(501, (n,), 1.0))
    dh = synth.to_bf16_bits(synth.normal_f32(502, (n,), 1.0))
    h = nf4.qlora_swiglu_fwd(d16(g), d16(u))
    dg, du = nf4.qlora_swiglu_bwd(d16(dh), d16(g), d16(u))
    torch.cuda.synchronize()
    check_tol("h", f32(h), oracle.swiglu_fwd(g, u))
    rg, ru = oracle.swiglu_bwd(dh, g, u)
    check_tol("dg", f32(dg), rg)
    check_tol("du", f32(du), ru)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemv_full_size(M):
    """Decode-size forward at full size (W 28672 x 8192, r = 64), all outputs against the oracle."""
    wl = synth.WORKLOADS["gemv"]
    lin = wl.linears[0]
    N, K, r, s = lin.N, lin.K, wl.r, wl.scale
    _say(f"gemv full size M={M} N={N} K={K}")
    W = synth.weight_f32(wl, lin)
    l1, l2 = synth.lora_f32(wl, lin)
    L1, L2 = synth.to_bf16_bits(l1), synth.to_bf16_bits(l2)
    X = synth.to_bf16_bits(synth.x_f32(wl, M=M, K=K))
    w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), CB)
    Y, T = nf4.qlora_linear_fwd(w, d16(X), d16(L1), d16(L2), s)
    torch.cuda.synchronize()
    Wd = oracle.dequant_weight(oracle.quantize_dq(W, CB), CB)
    del W
    Yr, Tr = oracle.forward(X, Wd, L1, L2, s)
    check_tol("Y", f32(Y), Yr)
    check_tol("T", f32(T), Tr)
