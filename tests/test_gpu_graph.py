"""Graph capture (torch's CUDAGraph over the library's HIP launches).

The forward that allocates nothing (qlora_linear_fwd_static), the entry point for callers that
record their work into a graph: captured once per token count, then replayed with new inputs written
into the captured buffers, with eager work and device synchronisations between the replays; every
replay's Y and T against the eager forward's bits (qlora_linear_fwd runs the same kernels).  The
token counts take every forward path: the decode GEMV, the 16-token GEMV, the fused dequant GEMM and
the bf16 expansion + GEMM.  And a whole forward + backward step through the workspace entry points,
captured and replayed the same way."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_nf4_quantized_codebook_amd as nf4  # noqa: E402

DEV = torch.device("cuda:0")


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(synth.to_bf16_bits(a)).view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.mark.parametrize("M", [1, 4, 16, 300, 4096])
def test_static_forward_graph_replays_match_eager(M):
    N, K, r, s = 4096, 4096, 64, 0.25
    print(f"graph capture of the static forward: M={M} N={N} K={K} r={r} {nf4.qlora_linear_route(M, N, K, r)}",
          flush=True)
    cb = nf4.nf4_build_codebook()
    w = nf4.NF4Weight.from_float(torch.from_numpy(synth.normal_f32(1800, (N, K), 0.02)).to(DEV), cb)
    L1 = _bf16(synth.normal_f32(1801, (K, r), 1.0 / r))
    L2 = _bf16(synth.normal_f32(1802, (r, N), 0.01))
    X = _bf16(synth.normal_f32(1810, (M, K), 1.0))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    T = torch.empty((M, r), dtype=torch.bfloat16, device=DEV)
    # one eager call first (it also looks up the static scratch's device address)
    nf4.qlora_linear_fwd_static(w, X, L1, L2, s, Y, T)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nf4.qlora_linear_fwd_static(w, X, L1, L2, s, Y, T)
    torch.cuda.synchronize()
    for rep in range(3):
        X.copy_(_bf16(synth.normal_f32(1820 + rep, (M, K), 1.0)))
        Y.fill_(float("nan"))
        T.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        Y_ref, T_ref = nf4.qlora_linear_fwd(w, X, L1, L2, s)      # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16)), (M, rep)
        assert torch.equal(T.view(torch.int16), T_ref.view(torch.int16)), (M, rep)


@pytest.mark.parametrize("M", [16, 4096])
def test_training_step_graph_replays_match_eager(M):
    """A whole forward + backward step through the workspace entry points captured into one graph
    (outputs and workspaces come from the graph's memory pool), replayed with new X and dY: Y, T,
    dX, dL1 and dL2 of every replay bit for bit against eager calls."""
    N, K, r, s = 4096, 4096, 64, 0.25
    print(f"graph capture of a training step: M={M} N={N} K={K} r={r} {nf4.qlora_linear_route(M, N, K, r)}",
          flush=True)
    cb = nf4.nf4_build_codebook()
    w = nf4.NF4Weight.from_float(torch.from_numpy(synth.normal_f32(1900, (N, K), 0.02)).to(DEV), cb)
    L1 = _bf16(synth.normal_f32(1901, (K, r), 1.0 / r))
    L2 = _bf16(synth.normal_f32(1902, (r, N), 0.01))
    X = _bf16(synth.normal_f32(1910, (M, K), 1.0))
    dY = _bf16(synth.normal_f32(1911, (M, N), 1.0))

    def step():
        Y, T = nf4.qlora_linear_fwd(w, X, L1, L2, s)
        dX, dL1, dL2 = nf4.qlora_linear_bwd(w, dY, X, L1, L2, T, s)
        return Y, T, dX, dL1, dL2

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    torch.cuda.synchronize()
    for rep in range(3):
        X.copy_(_bf16(synth.normal_f32(1920 + rep, (M, K), 1.0)))
        dY.copy_(_bf16(synth.normal_f32(1930 + rep, (M, N), 1.0)))
        g.replay()
        torch.cuda.synchronize()
        refs = step()                                            # eager work between the replays
        torch.cuda.synchronize()
        for name, a, b in zip(("Y", "T", "dX", "dL1", "dL2"), outs, refs):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (M, rep, name)
