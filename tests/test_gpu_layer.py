"""GPU parity of the linears of a whole decoder layer.

* qlora_multi_fwd: up to three linears sharing their input (the q, k and v projections), forward
  as one bf16 GEMM over the concatenated weights from 1024 tokens (every weight but the last a
  whole number of 256-column tiles).  Its outputs must equal three qlora_linear_fwd calls bit for
  bit where the joined product splits its reduction as each separate one does (each output tile
  then runs the same arithmetic; qlora_linear_route gives the splits), and the oracle within
  tolerance everywhere.
* A decoder layer's linears in one chain: q/k/v (one product), the output projection o, and the
  gated MLP (gate and up with the glue, then down), forward and backward, every stage checked
  against the float64 oracle on the GPU's own bf16 inputs to that stage.  The attention core
  between q/k/v and o is not a step of the method: a seeded tensor stands in for its output, and
  seeded upstream gradients stand in for dQ, dK and dV.

Tolerances: rel-Frobenius <= 5e-3 and max-abs <= 2e-2 * max|ref|.
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


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_tol(name, got, ref):
    rf, ma = oracle.rel_fro(got, ref), oracle.max_abs_ratio(got, ref)
    _say(f"  {name}: rel_fro {rf:.3e}  max_abs/max|ref| {ma:.3e}")
    assert rf <= oracle.REL_FRO_TOL, (name, rf)
    assert ma <= oracle.MAX_ABS_TOL, (name, ma)


class Lin:
    """A QLoRA linear [N, K]: device weight and adapters, and the oracle's bf16 deq(W)."""

    def __init__(self, seed, N, K, r):
        W = synth.normal_f32(seed, (N, K), 0.02)
        self.w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), CB)
        self.Wd = oracle.dequant_weight(oracle.quantize_dq(W, CB), CB)
        self.L1 = synth.to_bf16_bits(synth.normal_f32(seed + 1, (K, r), 1.0 / r))
        self.L2 = synth.to_bf16_bits(synth.normal_f32(seed + 2, (r, N), 0.01))
        self.L1d, self.L2d = d16(self.L1), d16(self.L2)
        self.N, self.K = N, K


@pytest.mark.parametrize("M,Ns,K,r", [
    (1024, (512, 256, 256), 512, 16),      # one product over three weights (GQA-like k, v)
    (1100, (768, 256, 520), 384, 32),      # ragged tokens; the last weight ends in a part tile
    (2048, (1024, 1024, 1024), 1024, 64),  # equal q, k, v; the separate calls split 4 ways, the joined 2
    (1024, (256, 512), 256, 128),          # two weights, two LoRA steps
    (1024, (520, 256, 256), 256, 16),      # a first weight off the tile grid: separate calls
    (300, (512, 256, 256), 512, 16),       # below the expanded-weight range: separate calls
])
def test_multi_fwd_matches_separate_calls_and_oracle(M, Ns, K, r):
    _say(f"multi fwd M={M} Ns={Ns} K={K} r={r}")
    s = 16.0 / r
    lins = [Lin(1200 + 10 * i + M, N, K, r) for i, N in enumerate(Ns)]
    X = synth.to_bf16_bits(synth.normal_f32(1299 + M, (M, K), 1.0))
    Xd = d16(X)
    Ys, Ts = nf4.qlora_multi_fwd([l.w for l in lins], Xd, [l.L1d for l in lins], [l.L2d for l in lins], s)
    sep = [nf4.qlora_linear_fwd(l.w, Xd, l.L1d, l.L2d, s) for l in lins]
    torch.cuda.synchronize()
    # the documented condition for one product: 1024 tokens, every weight but the last whole tiles
    joined = len(Ns) > 1 and M >= 1024 and all(N % 256 == 0 for N in Ns[:-1])
    ks_joined = nf4.qlora_linear_route(M, sum(Ns), K, r)["fwd_split"]
    for i, (l, (Y1, T1)) in enumerate(zip(lins, sep)):
        same = not joined or nf4.qlora_linear_route(M, Ns[i], K, r)["fwd_split"] == ks_joined
        _say(f"  Y{i}: bit for bit against the separate call: {same}")
        if same:
            assert torch.equal(Ys[i].view(torch.int16), Y1.view(torch.int16)), i
        else:
            check_tol(f"Y{i} vs separate", to64(Ys[i]), to64(Y1))
        assert torch.equal(Ts[i].view(torch.int16), T1.view(torch.int16)), i
        Yr, Tr = oracle.forward(X, l.Wd, l.L1, l.L2, s)
        check_tol(f"Y{i}", to64(Ys[i]), Yr)
        check_tol(f"T{i}", to64(Ts[i]), Tr)


def _rows(M, n=24, seed=13):
    r = np.random.default_rng(seed).choice(M, n, replace=False)
    return np.unique(np.concatenate([r, [0, M - 1]]))


def test_decoder_layer_linears_chain():
    """q/k/v, o and the gated MLP of one layer: d = 1024, F = 2752, 1088 tokens, r = 16."""
    M, d, F, r = 1088, 1024, 2752, 16
    s = 16.0 / r
    _say(f"decoder layer linears: M={M} d={d} F={F} r={r}")
    q, k, v, o = (Lin(1400 + 10 * i, d, d, r) for i in range(4))
    gate, up = Lin(1450, F, d, r), Lin(1460, F, d, r)
    down = Lin(1470, d, F, r)
    X = synth.to_bf16_bits(synth.normal_f32(1480, (M, d), 1.0))
    Aatt = synth.to_bf16_bits(synth.normal_f32(1481, (M, d), 1.0))     # stands in for attention's output
    dQ, dK, dV = (synth.to_bf16_bits(synth.normal_f32(1482 + i, (M, d), 1.0)) for i in range(3))
    dY = synth.to_bf16_bits(synth.normal_f32(1485, (M, d), 1.0))
    Xd, Ad = d16(X), d16(Aatt)

    # forward
    (Q, Kp, V), (Tq, Tk, Tv) = nf4.qlora_multi_fwd([q.w, k.w, v.w], Xd, [q.L1d, k.L1d, v.L1d],
                                                   [q.L2d, k.L2d, v.L2d], s)
    O, To = nf4.qlora_linear_fwd(o.w, Ad, o.L1d, o.L2d, s)
    G, U, H, Tg, Tu = nf4.qlora_gated_fwd(gate.w, up.w, O, gate.L1d, gate.L2d, up.L1d, up.L2d, s)
    Y, Td = nf4.qlora_linear_fwd(down.w, H, down.L1d, down.L2d, s)
    # backward
    dH, dL1_d, dL2_d = nf4.qlora_linear_bwd(down.w, d16(dY), H, down.L1d, down.L2d, Td, s)
    dO, dL1_g, dL2_g, dL1_u, dL2_u = nf4.qlora_gated_bwd(gate.w, up.w, dH, O, G, U, gate.L1d, gate.L2d,
                                                         up.L1d, up.L2d, Tg, Tu, s, fuse=True)
    dA, dL1_o, dL2_o = nf4.qlora_linear_bwd(o.w, dO, Ad, o.L1d, o.L2d, To, s)
    dX, dL1_q, dL2_q = nf4.qlora_linear_bwd(q.w, d16(dQ), Xd, q.L1d, q.L2d, Tq, s)
    _, dL1_k, dL2_k = nf4.qlora_linear_bwd(k.w, d16(dK), Xd, k.L1d, k.L2d, Tk, s, dX=dX, accumulate=True)
    _, dL1_v, dL2_v = nf4.qlora_linear_bwd(v.w, d16(dV), Xd, v.L1d, v.L2d, Tv, s, dX=dX, accumulate=True)
    torch.cuda.synchronize()

    rows = _rows(M)
    Ob, Gb, Ub, Hb, dHb, dOb = (h16(t) for t in (O, G, U, H, dH, dO))
    for name, l, inp, out in (("q", q, X, Q), ("k", k, X, Kp), ("v", v, X, V), ("o", o, Aatt, O),
                              ("gate", gate, Ob, G), ("up", up, Ob, U), ("down", down, Hb, Y)):
        Yr, _ = oracle.forward_rows(inp, l.Wd, l.L1, l.L2, s, rows)
        check_tol(f"{name} Y[rows]", to64(out)[rows], Yr)
    check_tol("glue h[rows]", to64(H)[rows], oracle.swiglu_fwd(Gb[rows], Ub[rows]))
    # backward, stage by stage
    g = oracle.backward_rows(dY, Hb, down.Wd, down.L1, down.L2, s, rows)
    check_tol("down dX[rows]", to64(dH)[rows], g["dX"])
    check_tol("down dL1", to64(dL1_d), g["dL1"])
    check_tol("down dL2", to64(dL2_d), g["dL2"])
    rg, ru = oracle.swiglu_bwd(dHb, Gb, Ub)
    dGb, dUb = oracle.bf16_rne(rg.astype(np.float32)), oracle.bf16_rne(ru.astype(np.float32))
    gg = oracle.backward_rows(dGb, Ob, gate.Wd, gate.L1, gate.L2, s, rows)
    gu = oracle.backward_rows(dUb, Ob, up.Wd, up.L1, up.L2, s, rows)
    check_tol("gate+up dX[rows]", to64(dO)[rows], gg["dX"] + gu["dX"])
    check_tol("gate dL1", to64(dL1_g), gg["dL1"])
    check_tol("gate dL2", to64(dL2_g), gg["dL2"])
    check_tol("up dL1", to64(dL1_u), gu["dL1"])
    check_tol("up dL2", to64(dL2_u), gu["dL2"])
    go = oracle.backward_rows(dOb, Aatt, o.Wd, o.L1, o.L2, s, rows)
    check_tol("o dX[rows]", to64(dA)[rows], go["dX"])
    check_tol("o dL1", to64(dL1_o), go["dL1"])
    check_tol("o dL2", to64(dL2_o), go["dL2"])
    gq, gk, gv = (oracle.backward_rows(dz, X, l.Wd, l.L1, l.L2, s, rows) for dz, l in ((dQ, q), (dK, k), (dV, v)))
    check_tol("q+k+v dX[rows]", to64(dX)[rows], gq["dX"] + gk["dX"] + gv["dX"])
    for name, gr, dl1, dl2 in (("q", gq, dL1_q, dL2_q), ("k", gk, dL1_k, dL2_k), ("v", gv, dL1_v, dL2_v)):
        check_tol(f"{name} dL1", to64(dl1), gr["dL1"])
        check_tol(f"{name} dL2", to64(dl2), gr["dL2"])
