"""The forward that allocates nothing (qlora_linear_fwd_static): through the C ABI, its outputs
against qlora_linear_fwd's (same kernels, so the same bits) on calls in a row with shrinking inputs
that take every forward path: bf16 expansion + GEMM (4096 tokens), the fused dequant GEMM, the
16-token GEMV and the decode GEMV.  The static scratch keeps each call's contents, so a smaller
call after a larger one must not depend on what is left there."""
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


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(synth.to_bf16_bits(a)).view(np.int16)).to(DEV).view(torch.bfloat16)


def test_static_forward_matches_workspace_forward():
    N, K, r, s = 4096, 4096, 64, 0.25
    cb = nf4.nf4_build_codebook()
    W = synth.normal_f32(1700, (N, K), 0.02)
    w = nf4.NF4Weight.from_float(torch.from_numpy(W).to(DEV), cb)
    L1 = _bf16(synth.normal_f32(1701, (K, r), 1.0 / r))
    L2 = _bf16(synth.normal_f32(1702, (r, N), 0.01))
    Wd = None
    for i, M in enumerate((4096, 300, 12, 4, 1, 1100)):
        print(f"static forward call {i}: M={M} N={N} K={K} r={r}", flush=True)
        X = _bf16(synth.normal_f32(1710 + i, (M, K), 1.0))
        Y_ref, T_ref = nf4.qlora_linear_fwd(w, X, L1, L2, s)
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        T = torch.full((M, r), float("nan"), dtype=torch.bfloat16, device=DEV)
        nf4.qlora_linear_fwd_static(w, X, L1, L2, s, Y, T)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16)), M
        assert torch.equal(T.view(torch.int16), T_ref.view(torch.int16)), M
        if M <= 64:
            # and against the oracle, to the layer's tolerance
            if Wd is None:
                Wd = oracle.dequant_weight(oracle.quantize_dq(W, cb), cb)
            bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
            Yr, _ = oracle.forward(bits(X), Wd, bits(L1), bits(L2), s)
            assert oracle.within_tolerance(Y.float().cpu().numpy(), Yr), M
    # without T_out
    X = _bf16(synth.normal_f32(1720, (8, K), 1.0))
    Y = torch.empty((8, N), dtype=torch.bfloat16, device=DEV)
    nf4.qlora_linear_fwd_static(w, X, L1, L2, s, Y, None)
    Y_ref, _ = nf4.qlora_linear_fwd(w, X, L1, L2, s, keep_T=False)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16))


def test_static_forward_rejects_a_shape_beyond_the_scratch():
    w = nf4.NF4Weight.from_float(torch.zeros((8192, 8192), dtype=torch.float32, device=DEV))
    X = torch.zeros((1024, 8192), dtype=torch.bfloat16, device=DEV)
    L1 = torch.zeros((8192, 16), dtype=torch.bfloat16, device=DEV)
    L2 = torch.zeros((16, 8192), dtype=torch.bfloat16, device=DEV)
    Y = torch.empty((1024, 8192), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(nf4.NF4Error) as e:
        nf4.qlora_linear_fwd_static(w, X, L1, L2, 1.0, Y)
    assert e.value.status == -5
