"""C-ABI contract on the host: the library loads, exports what include/nf4.h declares, builds the
same codebook as the oracle, and rejects bad arguments with the documented status before any HIP
call (so these run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

nf4 = pytest.importorskip("bit_nf4_quantized_codebook_amd")
lib = nf4.lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nf4.h")

OK, ENULL, ESHAPE, EALIGN, EUNSUP, EWS, EHIP, EARG = 0, -1, -2, -3, -4, -5, -6, -7


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    declared = _declared_functions()
    assert len(declared) >= 13
    assert set(declared) == set(nf4.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    for s in (OK, ENULL, ESHAPE, EALIGN, EUNSUP, EWS, EHIP, EARG):
        assert nf4.status_string(s)
    assert nf4.status_string(12345) == "unknown status"
    assert re.match(r"\d+\.\d+\.\d+", nf4.version())


@pytest.mark.parametrize("delta", [0.0, oracle.DELTA_DEFAULT, 16 / 17, 1 - 1 / 34, 0.99])
def test_codebook_bit_exact_with_oracle(delta):
    got = nf4.nf4_build_codebook(delta)
    ref = oracle.codebook(oracle.DELTA_DEFAULT if delta == 0.0 else delta)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_int4_and_fp4_codebooks_bit_exact_with_oracle():
    for got, ref in ((nf4.nf4_build_int4_codebook(), oracle.codebook_int4()),
                     (nf4.nf4_build_fp4_codebook(), oracle.codebook_fp4())):
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert lib.nf4_build_int4_codebook(None) == ENULL
    assert lib.nf4_build_fp4_codebook(None) == ENULL


def test_codebook_errors():
    out = np.zeros(16, np.float32)
    p = ctypes.c_void_p(out.ctypes.data)
    assert lib.nf4_build_codebook(None, 0.0) == ENULL
    assert lib.nf4_build_codebook(p, 0.3) == EARG
    assert lib.nf4_build_codebook(p, 1.0) == EARG
    assert b"delta" in lib.nf4_last_error()


def _cb():
    return nf4.nf4_build_codebook()


def test_quantize_argument_errors():
    cb = _cb()
    cbp = ctypes.c_void_p(cb.ctypes.data)
    fake = ctypes.c_void_p(0x100000)           # aligned, never dereferenced on these paths
    mis = ctypes.c_void_p(0x100004)
    assert lib.nf4_quantize(fake, 64, 64, None, fake, fake, None) == ENULL
    assert lib.nf4_quantize(fake, -1, 64, cbp, fake, fake, None) == ESHAPE
    assert lib.nf4_quantize(fake, 64, 32, cbp, fake, fake, None) == EUNSUP
    assert lib.nf4_quantize(None, 64, 64, cbp, fake, fake, None) == ENULL
    assert lib.nf4_quantize(mis, 64, 64, cbp, fake, fake, None) == EALIGN
    assert lib.nf4_quantize(None, 0, 64, cbp, None, None, None) == OK       # empty input
    eq = cb.copy()
    eq[5] = eq[6]                                # equal neighbours: accepted (the lower index wins)
    assert lib.nf4_quantize(None, 0, 64, ctypes.c_void_p(eq.ctypes.data), None, None, None) == OK
    bad = cb.copy()
    bad[3], bad[4] = bad[4], bad[3]
    assert lib.nf4_quantize(fake, 64, 64, ctypes.c_void_p(bad.ctypes.data), fake, fake, None) == EARG
    nozero = cb.copy()
    nozero[7] = 1e-3
    assert lib.nf4_quantize(fake, 64, 64, ctypes.c_void_p(nozero.ctypes.data), fake, fake, None) == EARG


def test_double_quant_argument_errors():
    fake = ctypes.c_void_p(0x100000)
    ws = lib.nf4_double_quant_workspace_size(1000, 256)
    assert ws > 0
    assert lib.nf4_double_quant(fake, 0, 256, fake, fake, fake, fake, ws, None) == ESHAPE
    assert lib.nf4_double_quant(fake, 1000, 128, fake, fake, fake, fake, ws, None) == EUNSUP
    assert lib.nf4_double_quant(fake, 1000, 256, None, fake, fake, fake, ws, None) == ENULL
    assert lib.nf4_double_quant(fake, 1000, 256, fake, fake, fake, fake, ws - 1, None) == EWS
    for fn in (lib.nf4_double_quant, lib.nf4_double_quant_int8):       # same checks, either format
        assert fn(fake, 0, 256, fake, fake, fake, fake, ws, None) == ESHAPE
        assert fn(fake, 1000, 128, fake, fake, fake, fake, ws, None) == EUNSUP
        assert fn(fake, 1000, 256, fake, fake, fake, fake, ws - 1, None) == EWS
    assert lib.nf4_double_quant(ctypes.c_void_p(0x100004), 1000, 256, fake, fake, fake, fake, ws, None) == EALIGN
    # workspace grows with the number of summation levels
    assert lib.nf4_double_quant_workspace_size(3670016, 256) >= 8 * (14336 + 56 + 1)


def _desc(rows=256, cols=256, block=64, dq_block=256, ptr=0x100000, cb=None):
    d = nf4._WeightDesc()
    d.packed = d.absmax_q = d.absmax_scale = d.absmax_mean = ptr
    d.rows, d.cols, d.block, d.dq_block = rows, cols, block, dq_block
    cb = _cb() if cb is None else cb
    for j in range(16):
        d.codebook[j] = float(cb[j])
    return d


def test_weight_dq_format_is_checked():
    out = ctypes.c_void_p(0x200000)
    d = _desc()
    d.dq_format = 7
    assert lib.nf4_dequant(ctypes.byref(d), out, None) == EARG
    assert b"dq_format" in lib.nf4_last_error()


def test_linear_argument_errors():
    fake = ctypes.c_void_p(0x100000)
    M, r = 8, 8
    wsb = lib.qlora_linear_workspace_size(M, 256, 256, r)
    assert wsb > 0
    fwd = lambda d, **kw: lib.qlora_linear_fwd(ctypes.byref(d), kw.get("X", fake), fake, fake,
                                                kw.get("scale", 2.0), kw.get("M", M), kw.get("r", r),
                                                fake, None, kw.get("ws", fake), kw.get("wsb", wsb), None)
    assert lib.qlora_linear_fwd(None, fake, fake, fake, 2.0, M, r, fake, None, fake, wsb, None) == ENULL
    assert fwd(_desc(), M=0) == ESHAPE
    assert fwd(_desc(), r=0) == EUNSUP
    assert fwd(_desc(), r=129) == EUNSUP
    assert fwd(_desc(), r=12) == EUNSUP
    assert fwd(_desc(block=128)) == EUNSUP
    assert fwd(_desc(dq_block=64)) == EUNSUP
    assert fwd(_desc(cols=200)) == EUNSUP
    assert fwd(_desc(rows=0)) == ESHAPE
    assert fwd(_desc(), scale=float("nan")) == EARG
    assert fwd(_desc(), X=None) == ENULL
    assert fwd(_desc(), X=ctypes.c_void_p(0x100002)) == EALIGN
    assert fwd(_desc(), wsb=wsb - 1) == EWS
    assert fwd(_desc(), ws=None) == EWS
    assert fwd(_desc(ptr=0x100008)) == EALIGN
    # 32-bit buffer offsets: each operand under 2 GiB (packed weight, X [M, K], Y [M, N])
    assert fwd(_desc(rows=65536, cols=65536)) == EUNSUP
    assert fwd(_desc(rows=65536, cols=65472)) == EWS          # just under: reaches the workspace check
    assert fwd(_desc(), M=1 << 22) == EUNSUP                  # X: 2^22 x 256 bf16 = 2 GiB
    assert fwd(_desc(rows=65536), M=1 << 14) == EUNSUP        # Y: 2^14 x 65536 bf16 = 2 GiB
    # backward: unknown flags, NULL gradient outputs
    d = _desc()
    assert lib.qlora_linear_bwd(ctypes.byref(d), fake, fake, fake, fake, None, 2.0, M, r, fake, fake,
                                fake, 2, fake, wsb, None) == EARG
    assert lib.qlora_linear_bwd(ctypes.byref(d), fake, fake, fake, fake, None, 2.0, M, r, fake, None,
                                fake, 0, fake, wsb, None) == ENULL
    assert lib.qlora_linear_bwd(ctypes.byref(d), fake, fake, fake, fake, None, 2.0, M, r, fake, fake,
                                fake, 0, fake, wsb - 1, None) == EWS


def test_static_forward_argument_errors():
    """The forward without a workspace checks its arguments like qlora_linear_fwd and rejects a
    shape whose forward needs more than the static scratch, all before any HIP call."""
    fake = ctypes.c_void_p(0x100000)
    st = lambda d, **kw: lib.qlora_linear_fwd_static(ctypes.byref(d), kw.get("X", fake), fake, fake,  # noqa: E731
                                                     2.0, kw.get("M", 8), kw.get("r", 8), fake, None, None)
    assert lib.qlora_linear_fwd_static(None, fake, fake, fake, 2.0, 8, 8, fake, None, None) == ENULL
    assert st(_desc(), M=0) == ESHAPE
    assert st(_desc(), r=12) == EUNSUP
    assert st(_desc(), X=None) == ENULL
    assert st(_desc(), X=ctypes.c_void_p(0x100002)) == EALIGN
    # from 1024 tokens an 8192 x 8192 weight is expanded to bf16 (128 MiB): with the rest, beyond the 128 MiB scratch
    assert st(_desc(rows=8192, cols=8192), M=4096, r=64) == EWS
    assert b"static scratch" in lib.nf4_last_error()
    assert nf4.QLORA_STATIC_SCRATCH_BYTES == 128 << 20
    hdr = open(HEADER).read()
    assert "#define QLORA_STATIC_SCRATCH_BYTES ((size_t)128 << 20)" in hdr


def test_multi_forward_argument_errors():
    """The forward of linears sharing X: n, the arrays, matching K and the workspace are checked
    before any HIP call; the workspace covers both the fused plan and each separate call."""
    fake = ctypes.c_void_p(0x100000)
    P = ctypes.c_void_p
    d = [_desc(rows=256, cols=256), _desc(rows=512, cols=256), _desc(rows=256, cols=128)]
    dp = (P * 3)(*[ctypes.addressof(x) for x in d])
    arr = (P * 3)(fake, fake, fake)
    N = (ctypes.c_int64 * 3)(256, 512, 256)
    wsb = lib.qlora_multi_workspace_size(3, ctypes.cast(N, P), 256, 1024, 16)
    assert wsb >= lib.qlora_linear_workspace_size(1024, 512, 256, 16)
    assert wsb >= lib.qlora_linear_workspace_size(1024, 1024, 256, 16)     # the fused plan
    assert lib.qlora_multi_workspace_size(4, ctypes.cast(N, P), 256, 1024, 16) == 0
    call = lambda n, **kw: lib.qlora_multi_fwd(n, kw.get("w", ctypes.cast(dp, P)), fake,  # noqa: E731
                                               ctypes.cast(arr, P), ctypes.cast(arr, P), 2.0, 1024, 16,
                                               kw.get("Y", ctypes.cast(arr, P)), None, fake, kw.get("wsb", wsb), None)
    assert call(0) == EARG and call(4) == EARG
    assert call(2, w=None) == ENULL and call(2, Y=None) == ENULL
    assert call(3) == ESHAPE                        # the third weight has another K
    assert call(2, wsb=16) == EWS


def test_dequant_and_swiglu_argument_errors():
    fake = ctypes.c_void_p(0x100000)
    d = _desc()
    assert lib.nf4_dequant(ctypes.byref(d), None, None) == ENULL
    assert lib.nf4_dequant(ctypes.byref(d), ctypes.c_void_p(0x100002), None) == EALIGN
    assert lib.nf4_dequant(None, fake, None) == ENULL
    assert lib.qlora_swiglu_fwd(fake, fake, fake, -1, None) == ESHAPE
    assert lib.qlora_swiglu_fwd(fake, fake, fake, 0, None) == OK
    assert lib.qlora_swiglu_fwd(None, fake, fake, 8, None) == ENULL
    assert lib.qlora_swiglu_bwd(fake, fake, fake, fake, ctypes.c_void_p(0x100001), 8, None) == EALIGN


def test_workspace_sizes_cover_all_configs():
    for M, N, K, r in [(8, 256, 256, 8), (4096, 4096, 4096, 64), (4096, 11008, 4096, 64),
                       (4096, 4096, 11008, 64), (2048, 22016, 8192, 64), (1, 28672, 8192, 64)]:
        ws = lib.qlora_linear_workspace_size(M, N, K, r)
        # at least T, sT, dT and the transposed adapters
        assert ws >= 2 * (3 * M * r + r * K + N * r)
        assert ws < 1 << 31


def test_route_by_token_count_and_tile_count():
    """qlora_linear_route: the documented path per token count, no split where the output tiles
    fill the 256 CUs (the 7B training shapes), splits where they do not; bad arguments rejected."""
    info = (ctypes.c_int32 * 4)()
    assert lib.qlora_linear_route(8, 256, 256, 8, None) == ENULL
    assert lib.qlora_linear_route(0, 256, 256, 8, info) == ESHAPE
    route = nf4.qlora_linear_route
    # decode sizes: GEMV forward, unsplit; the backward's dX product (32 tiles of 256 columns for
    # K = 8192, 448 reduction steps) splits 8 ways
    assert route(1, 28672, 8192, 64) == {"fwd": "gemv", "fwd_split": 1, "bwd": "fused", "bwd_split": 8}
    assert route(16, 28672, 8192, 64)["fwd"] == "gemv_wide"
    # the wide GEMV's 64 row blocks of 4096 rows split K four ways (one 1024-column window each);
    # 28672 rows make 256 blocks: no split
    assert route(32, 4096, 4096, 64) == {"fwd": "gemv_wide", "fwd_split": 4, "bwd": "fused", "bwd_split": 16}
    assert route(16, 28672, 8192, 64)["fwd_split"] == 1 and route(16, 4096, 11008, 64)["fwd_split"] == 4
    assert route(64, 4096, 4096, 64)["fwd"] == "gemv_wide" and route(65, 4096, 4096, 64)["fwd"] == "fused"
    assert route(1023, 4096, 4096, 64)["bwd"] == "fused"
    assert route(1024, 4096, 4096, 64)["fwd"] == "expanded"
    # 4096 x 4096 x 4096: 256 output tiles each way, no split; the 7B MLP shapes likewise
    for M, N, K in [(4096, 4096, 4096), (4096, 11008, 4096), (4096, 4096, 11008), (2048, 22016, 8192)]:
        rt = route(M, N, K, 64)
        assert rt["fwd_split"] == 1 and rt["bwd_split"] == 1, (M, N, K, rt)
    # 128 tokens: 16 tiles, 16 splits of 4 steps each way; 512 tokens: 32 tiles, 8 splits
    assert route(128, 4096, 4096, 64)["fwd_split"] == 16 and route(128, 4096, 4096, 64)["bwd_split"] == 16
    assert route(512, 4096, 4096, 64)["fwd_split"] == 8
    # never more splits than whole groups of 4 reduction steps
    assert route(100, 4096, 384, 64)["fwd_split"] == 1
    # the workspace grows by the partials: splits x M x N float32 at least
    assert lib.qlora_linear_workspace_size(128, 4096, 4096, 64) >= 16 * 128 * 4096 * 4


def test_flag_bits_are_distinct_and_match_the_binding():
    text = open(HEADER).read()
    vals = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (QLORA_\w+) (\d+)u", text)}
    assert vals["QLORA_GATED_FUSE"] & vals["QLORA_DX_ACCUMULATE"] == 0
    assert nf4.QLORA_GATED_FUSE == vals["QLORA_GATED_FUSE"]


def test_gated_argument_errors():
    d = _desc()
    fake = ctypes.c_void_p(0x100000)
    ws = lib.qlora_gated_workspace_size(64, 256, 256, 8)
    assert ws > 0
    # unknown flag bits
    assert lib.qlora_gated_fwd(ctypes.byref(d), ctypes.byref(d), fake, fake, fake, fake, fake, 1.0, 64, 8,
                               fake, fake, fake, None, None, 4, fake, ws, None) == EARG
    assert lib.qlora_gated_bwd(ctypes.byref(d), ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake,
                               None, None, 1.0, 64, 8, fake, fake, fake, fake, fake, 4, fake, ws, None) == EARG
    # shapes of gate and up must agree
    d2 = _desc(rows=512)
    assert lib.qlora_gated_fwd(ctypes.byref(d), ctypes.byref(d2), fake, fake, fake, fake, fake, 1.0, 64, 8,
                               fake, fake, fake, None, None, 0, fake, ws, None) == ESHAPE
    # workspace too small (the size query covers the larger, backward plan; 256 bytes fits neither)
    assert lib.qlora_gated_fwd(ctypes.byref(d), ctypes.byref(d), fake, fake, fake, fake, fake, 1.0, 64, 8,
                               fake, fake, fake, None, None, 0, fake, 256, None) == EWS
    assert lib.qlora_gated_bwd(ctypes.byref(d), ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake,
                               None, None, 1.0, 64, 8, fake, fake, fake, fake, fake, 0, fake, 256, None) == EWS
