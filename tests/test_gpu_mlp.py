"""GPU parity of the MLP workloads: the LLaMA-7B MLP chain and the heavy-tailed LLaMA-65B-shaped
MLP chain, plus the gated forms (gate and up as one product).

A chain is gate and up (QLoRA linears) -> SwiGLU -> down (QLoRA linear), forward and backward,
run through the C ABI exactly as a caller would, with dX of gate and up accumulated into one
buffer.  Each stage is checked against the float64 oracle on the GPU's own bf16 inputs to that
stage (so an error cannot hide behind the next stage's rounding): token rows are sampled for the
[M, N] outputs (oracle.forward_rows / oracle.backward_rows), the adapter gradients are checked in
full.  Tolerances: rel-Frobenius <= 5e-3 and max-abs <= 2e-2 * max|ref|.  The 65B chain adds a
bit-exact check of quantize, double quant and dequant of its three heavy-tailed weights (1 % of
the entries from a ten times wider normal).
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


def d16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def h16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def check_tol(name, got, ref):
    rf, ma = oracle.rel_fro(got, ref), oracle.max_abs_ratio(got, ref)
    _say(f"  {name}: rel_fro {rf:.3e}  max_abs/max|ref| {ma:.3e}")
    assert rf <= oracle.REL_FRO_TOL, (name, rf)
    assert ma <= oracle.MAX_ABS_TOL, (name, ma)


class Layer:
    """One QLoRA linear of a workload: device NF4 weight + adapters, and the oracle's pieces
    (quantized storage and the bf16 deq(W))."""

    def __init__(self, wl, lin, W, q, Wd):
        l1, l2 = synth.lora_f32(wl, lin)
        self.L1, self.L2 = synth.to_bf16_bits(l1), synth.to_bf16_bits(l2)
        self.w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), CB)
        self.q, self.Wd = q, Wd                            # Wd: bf16 bits [N, K]
        self.dL1d, self.dL2d = d16(self.L1), d16(self.L2)
        self.N, self.K, self.name = lin.N, lin.K, lin.name

    def check_storage(self):
        """Packed codes, second-level codes and scales, the mean and deq(W): bit for bit."""
        w = self.w
        assert np.array_equal(w.packed.cpu().numpy(), self.q["packed"]), self.name
        assert np.array_equal(w.absmax_q.cpu().numpy(), self.q["codes"]), self.name
        assert np.array_equal(w.absmax_scale.cpu().numpy().view(np.uint32), self.q["scales"].view(np.uint32))
        assert np.array_equal(w.absmax_mean.cpu().numpy().view(np.uint32),
                              np.asarray([self.q["mean"]], np.float32).view(np.uint32)), self.name
        assert np.array_equal(h16(nf4.nf4_dequant(w)).reshape(self.Wd.shape), self.Wd), self.name


def _layers(wl):
    """The workload's linears; the oracle's quantization of the three weights runs on a thread
    pool (its C code releases the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor

    def prep(lin):
        W = synth.weight_f32(wl, lin)
        q = oracle.quantize_dq(W, CB)
        return lin, W, q, oracle.dequant_weight(q, CB)

    with ThreadPoolExecutor(len(wl.linears)) as ex:
        preps = list(ex.map(prep, wl.linears))
    return [Layer(wl, *p) for p in preps]


def _rows(M, n=32, seed=11):
    r = np.random.default_rng(seed).choice(M, n, replace=False)
    return np.unique(np.concatenate([r, [0, M - 1]]))


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check_fwd(name, layer, Xbits, Ygpu, s, rows):
    Yr, _ = oracle.forward_rows(Xbits, layer.Wd, layer.L1, layer.L2, s, rows)
    check_tol(f"{name} Y[rows]", Ygpu[rows], Yr)


def _check_bwd(name, layer, dYbits, Xbits, dXgpu, dL1gpu, dL2gpu, s, rows):
    """dL1 and dL2 in full (they reduce over every token), dX on sampled rows; returns the oracle's
    gradients (dX on those rows)."""
    g = oracle.backward_rows(dYbits, Xbits, layer.Wd, layer.L1, layer.L2, s, rows)
    check_tol(f"{name} dL2", dL2gpu, g["dL2"])
    check_tol(f"{name} dL1", dL1gpu, g["dL1"])
    if dXgpu is not None:
        check_tol(f"{name} dX[rows]", dXgpu[rows], g["dX"])
    return g


def _mlp_chain(wl, check_storage):
    """gate and up (QLoRA linears) -> SwiGLU -> down (QLoRA linear), forward and backward, with dX
    of gate and up accumulated into one buffer; every stage checked against the oracle on the
    GPU's own bf16 inputs to that stage."""
    M, s = wl.M, wl.scale
    gate, up, down = _layers(wl)
    _say(f"{wl.name}: M={M}, gate/up {gate.N}x{gate.K}, down {down.N}x{down.K}, r={wl.r}")
    if check_storage:
        for layer in (gate, up, down):
            layer.check_storage()
    X = synth.to_bf16_bits(synth.x_f32(wl, M=M, K=gate.K))
    dY = synth.to_bf16_bits(synth.dy_f32(wl, M, down.N))
    Xd, dYd = d16(X), d16(dY)

    G, Tg = nf4.qlora_linear_fwd(gate.w, Xd, gate.dL1d, gate.dL2d, s)
    U, Tu = nf4.qlora_linear_fwd(up.w, Xd, up.dL1d, up.dL2d, s)
    H = nf4.qlora_swiglu_fwd(G, U)
    Y, Td = nf4.qlora_linear_fwd(down.w, H, down.dL1d, down.dL2d, s)
    dH, dL1_down, dL2_down = nf4.qlora_linear_bwd(down.w, dYd, H, down.dL1d, down.dL2d, Td, s)
    dG, dU = nf4.qlora_swiglu_bwd(dH, G, U)
    dX, dL1_gate, dL2_gate = nf4.qlora_linear_bwd(gate.w, dG, Xd, gate.dL1d, gate.dL2d, Tg, s)
    _, dL1_up, dL2_up = nf4.qlora_linear_bwd(up.w, dU, Xd, up.dL1d, up.dL2d, Tu, s, dX=dX,
                                             accumulate=True)
    torch.cuda.synchronize()

    rows = _rows(M)
    Gb, Ub, Hb, dHb, dGb, dUb = (h16(t) for t in (G, U, H, dH, dG, dU))
    _check_fwd("gate", gate, X, to64(G), s, rows)
    _check_fwd("up", up, X, to64(U), s, rows)
    check_tol("swiglu h[rows]", to64(H)[rows], oracle.swiglu_fwd(Gb[rows], Ub[rows]))
    _check_fwd("down", down, Hb, to64(Y), s, rows)
    _check_bwd("down", down, dY, Hb, to64(dH), to64(dL1_down), to64(dL2_down), s, rows)
    rg, ru = oracle.swiglu_bwd(dHb[rows], Gb[rows], Ub[rows])
    check_tol("swiglu dg[rows]", to64(dG)[rows], rg)
    check_tol("swiglu du[rows]", to64(dU)[rows], ru)
    # gate and up adapters in full; dX = both branches summed
    gg = _check_bwd("gate", gate, dGb, X, None, to64(dL1_gate), to64(dL2_gate), s, rows)
    gu = _check_bwd("up", up, dUb, X, None, to64(dL1_up), to64(dL2_up), s, rows)
    check_tol("dX[rows] (gate + up)", to64(dX)[rows], gg["dX"] + gu["dX"])


def test_llama7b_mlp_chain():
    """LLaMA-7B MLP: gate, up (11008 x 4096), SwiGLU, down (4096 x 11008); 4096 tokens, r = 64."""
    _mlp_chain(synth.WORKLOADS["llama7b_mlp"], check_storage=False)


def test_llama65b_mlp_chain():
    """LLaMA-65B-shaped MLP with 1 % heavy-tailed weight entries: gate, up (22016 x 8192), SwiGLU,
    down (8192 x 22016, the longest reduction on the expanded-weight GEMMs); 2048 tokens, r = 64.
    The storage of all three weights (codes, constants, mean, deq(W)) is checked bit for bit."""
    _mlp_chain(synth.WORKLOADS["llama65b_mlp"], check_storage=True)


# ------------------------------------------------------------------------------------------
# Gated forward: gate and up as the linears sharing X (one product over both weights), then the glue
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,F,K,r", [
    (1024, 2048, 1024, 64),    # one product over both weights, whole tiles
    (1100, 768, 640, 32),      # ragged tokens, one product
    (2048, 1280, 512, 128),    # r = 128: two LoRA steps per adapter, one product
    (300, 512, 384, 16),       # below the expanded-weight range: the two linears as calls
    (1024, 520, 256, 8),       # F not a multiple of 256: the two linears as calls
])
def test_gated_fwd_matches_separate_calls_and_oracle(M, F, K, r):
    _say(f"gated fwd M={M} F={F} K={K} r={r}")
    s = 16.0 / r
    sd = 700 + M + F
    Wg = synth.normal_f32(sd, (F, K), 0.02)
    Wu = synth.normal_f32(sd + 1, (F, K), 0.02)
    X = synth.to_bf16_bits(synth.normal_f32(sd + 2, (M, K), 1.0))
    ad = [synth.to_bf16_bits(synth.normal_f32(sd + 3 + i, shp, std))
          for i, (shp, std) in enumerate((((K, r), 1.0 / r), ((r, F), 0.01), ((K, r), 1.0 / r), ((r, F), 0.01)))]
    wg = nf4.NF4Weight.from_float(torch.from_numpy(Wg).to(DEV), CB)
    wu = nf4.NF4Weight.from_float(torch.from_numpy(Wu).to(DEV), CB)
    Xd = d16(X)
    L1g, L2g, L1u, L2u = (d16(a) for a in ad)
    G, U, H, Tg, Tu = nf4.qlora_gated_fwd(wg, wu, Xd, L1g, L2g, L1u, L2u, s, fuse=True)
    G0, U0, H0, Tg0, Tu0 = nf4.qlora_gated_fwd(wg, wu, Xd, L1g, L2g, L1u, L2u, s)
    Gs, Tgs = nf4.qlora_linear_fwd(wg, Xd, L1g, L2g, s)
    Us, Tus = nf4.qlora_linear_fwd(wu, Xd, L1u, L2u, s)
    Hs = nf4.qlora_swiglu_fwd(Gs, Us)
    torch.cuda.synchronize()
    # the same bits as the separate calls, fused or not
    for g_, u_, h_, tg_, tu_ in ((G, U, H, Tg, Tu), (G0, U0, H0, Tg0, Tu0)):
        assert torch.equal(g_, Gs) and torch.equal(u_, Us) and torch.equal(h_, Hs)
        assert torch.equal(tg_, Tgs) and torch.equal(tu_, Tus)
    # and within tolerance of the oracle
    Wgq = oracle.dequant_weight(oracle.quantize_dq(Wg, CB), CB)
    Wuq = oracle.dequant_weight(oracle.quantize_dq(Wu, CB), CB)
    Gr, _ = oracle.forward(X, Wgq, ad[0], ad[1], s)
    Ur, _ = oracle.forward(X, Wuq, ad[2], ad[3], s)
    check_tol("G", to64(G), Gr)
    check_tol("U", to64(U), Ur)
    check_tol("H", to64(H), oracle.swiglu_fwd(h16(G), h16(U)))


@pytest.mark.parametrize("M,F,K,r", [
    (1024, 2048, 1024, 64),    # dX as one product over both weights
    (1100, 544, 640, 32),      # ragged tokens and reduction segments (544 = 8.5 steps of 64)
    (2048, 1056, 512, 128),    # two LoRA steps per adapter
    (300, 512, 384, 16),       # below the fused range: the linears' backward as calls
    (1024, 520, 256, 8),       # ragged segments (520 = 8.1 steps of 64), one LoRA step each
])
def test_gated_bwd_fused_and_composed(M, F, K, r):
    _say(f"gated bwd M={M} F={F} K={K} r={r}")
    s = 16.0 / r
    sd = 800 + M + F
    Wg = synth.normal_f32(sd, (F, K), 0.02)
    Wu = synth.normal_f32(sd + 1, (F, K), 0.02)
    X = synth.to_bf16_bits(synth.normal_f32(sd + 2, (M, K), 1.0))
    dH = synth.to_bf16_bits(synth.normal_f32(sd + 3, (M, F), 1.0))
    ad = [synth.to_bf16_bits(synth.normal_f32(sd + 4 + i, shp, std))
          for i, (shp, std) in enumerate((((K, r), 1.0 / r), ((r, F), 0.01), ((K, r), 1.0 / r), ((r, F), 0.01)))]
    wg = nf4.NF4Weight.from_float(torch.from_numpy(Wg).to(DEV), CB)
    wu = nf4.NF4Weight.from_float(torch.from_numpy(Wu).to(DEV), CB)
    Xd, dHd = d16(X), d16(dH)
    L1g, L2g, L1u, L2u = (d16(a) for a in ad)
    G, U, H, Tg, Tu = nf4.qlora_gated_fwd(wg, wu, Xd, L1g, L2g, L1u, L2u, s)
    args = (wg, wu, dHd, Xd, G, U, L1g, L2g, L1u, L2u)
    comp = nf4.qlora_gated_bwd(*args, Tg, Tu, s)
    fused = nf4.qlora_gated_bwd(*args, Tg, Tu, s, fuse=True)
    recomputed = nf4.qlora_gated_bwd(*args, None, None, s, fuse=True)
    base = d16(synth.to_bf16_bits(synth.normal_f32(sd + 9, (M, K), 1.0)))
    acc = base.clone()
    nf4.qlora_gated_bwd(*args, Tg, Tu, s, dX=acc, accumulate=True, fuse=True)
    torch.cuda.synchronize()
    # adapter gradients: the same launches on every path; T recomputed gives the same bits
    for k in range(1, 5):
        assert torch.equal(comp[k], fused[k]) and torch.equal(fused[k], recomputed[k])
    assert torch.equal(fused[0], recomputed[0])
    no_dx = nf4.qlora_gated_bwd(*args, Tg, Tu, s, need_dX=False, fuse=True)
    torch.cuda.synchronize()
    assert no_dx[0] is None and all(torch.equal(no_dx[k], fused[k]) for k in range(1, 5))
    # against the oracle, fed the glue's backward of the GPU's own G and U (rounded to bf16)
    rg, ru = oracle.swiglu_bwd(dH, h16(G), h16(U))
    dGb, dUb = oracle.bf16_rne(rg.astype(np.float32)), oracle.bf16_rne(ru.astype(np.float32))
    Wgq = oracle.dequant_weight(oracle.quantize_dq(Wg, CB), CB)
    Wuq = oracle.dequant_weight(oracle.quantize_dq(Wu, CB), CB)
    gg = oracle.backward(dGb, X, Wgq, ad[0], ad[1], s)
    gu = oracle.backward(dUb, X, Wuq, ad[2], ad[3], s)
    dX_ref = gg["dX"] + gu["dX"]
    check_tol("dX fused", to64(fused[0]), dX_ref)
    check_tol("dX composed", to64(comp[0]), dX_ref)
    check_tol("dX += (fused)", to64(acc), dX_ref + to64(base))
    check_tol("dL1_gate", to64(fused[1]), gg["dL1"])
    check_tol("dL2_gate", to64(fused[2]), gg["dL2"])
    check_tol("dL1_up", to64(fused[3]), gu["dL1"])
    check_tol("dL2_up", to64(fused[4]), gu["dL2"])
