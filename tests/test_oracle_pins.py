"""Pins for the CPU oracle: each function is checked against something other than itself --
the pages' printed numbers (tests/golden), closed forms, invariants the pages state, library
routines (scipy's normal quantile and CDF, torch's bf16 and float8_e4m3fn casts, torch autograd)
and exact rational brute force.  All CPU-only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special as sps
import scipy.stats as st
import torch

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "paper_values.json")))


# ------------------------------------------------------------------------------------------
# Codebook (notes section 3.2 eq. 4; section 5.1.2 Fig. 7 text)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("delta", [oracle.DELTA_DEFAULT, 16.0 / 17.0, 1.0 - 1.0 / 34.0, 0.99])
def test_codebook_structure(delta):
    g = GOLDEN["nf4_layout"]
    cb = oracle.codebook(delta)
    assert cb.dtype == np.float32 and cb.size == g["values"] == 2 ** g["bits"]
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == np.float32(g["range"][0]) and cb[-1] == np.float32(g["range"][1])
    assert np.count_nonzero(cb == 0) == g["zeros"]
    assert cb[7] == 0.0
    neg, pos = int(np.sum(cb < 0)), int(np.sum(cb > 0))
    assert sorted([neg, pos]) == sorted(g["halves"])
    # quantile counts per half, each counting the shared zero (section 3.2)
    assert neg + 1 == g["negative_quantiles"] and pos + 1 == g["positive_quantiles"]


@pytest.mark.parametrize("delta", [oracle.DELTA_DEFAULT, 16.0 / 17.0])
def test_codebook_equal_mass_per_half(delta):
    """Each code of a half covers the same probability under N(0,1) (equal expected counts per
    bin), measured with scipy's independent normal CDF."""
    cb = oracle.codebook(delta).astype(np.float64)
    zmax = sps.ndtri(delta)
    cdf = st.norm.cdf(cb * zmax)
    pos = np.diff(cdf[7:])
    neg = np.diff(cdf[:8])
    np.testing.assert_allclose(pos, (delta - 0.5) / 8, rtol=0, atol=2e-7)
    np.testing.assert_allclose(neg, (delta - 0.5) / 7, rtol=0, atol=2e-7)


def test_codebook_values_match_library_quantile():
    """The float32 codewords equal scipy's ndtri-based construction rounded to float32."""
    d = oracle.DELTA_DEFAULT
    z = sps.ndtri(d)
    ref = [-(sps.ndtri(0.5 + (d - 0.5) * (j / 7)) / z) for j in range(7, 0, -1)] + [0.0] + \
          [sps.ndtri(0.5 + (d - 0.5) * (j / 8)) / z for j in range(1, 9)]
    ref = np.array(ref, dtype=np.float64).astype(np.float32)
    assert np.array_equal(oracle.codebook(d), ref)


def test_norm_ppf_matches_scipy():
    ps = np.concatenate([np.linspace(1e-9, 1 - 1e-9, 2001), [0.5, 0.75, 0.9677083333333334]])
    for p in ps:
        a, b = oracle.norm_ppf(p), sps.ndtri(p)
        # p itself is only known to half an ulp; its quantile to that divided by the density
        cond = 2.0 ** -52 / st.norm.pdf(b)
        assert abs(a - b) <= 4e-15 * max(1.0, abs(b)) + 2 * cond, (p, a, b)


def test_codebook_rejects_bad_delta():
    with pytest.raises(ValueError):
        oracle.codebook(0.4)


# ------------------------------------------------------------------------------------------
# Number formats: bf16 and E4M3 against torch's casts
# ------------------------------------------------------------------------------------------

def _random_f32_bits(n, seed):
    u = (synth.uniform(seed, n) * 2.0 ** 32).astype(np.uint64).astype(np.uint32)
    exp = (u >> 23) & 0xFF
    u = np.where(exp == 0xFF, u & np.uint32(0xBFFFFFFF), u)       # finite only
    return u.view(np.float32)


def test_bf16_rne_matches_torch():
    x = _random_f32_bits(1 << 18, 7)
    sub = (x.view(np.uint32) & np.uint32(0x807FFFFF)).view(np.float32)        # subnormals
    ties = ((x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    big = np.array([3.3895e38, 3.3961e38, 3.4e38, -3.3962e38, 3.4028235e38], dtype=np.float32)
    for v in (x, sub, ties, big, np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32)):
        ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(oracle.bf16_rne(v), ref)


def _e4m3_torch(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.all(np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))))
    assert oracle.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0


def test_e4m3_encode_matches_torch():
    vals = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    nb = []
    for k in range(1, 4):
        nb += [np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(-np.inf))]
        pts = np.concatenate([pts] + nb)
    rnd = (synth.uniform(11, 200000) * 2 - 1) * 448
    tiny = (synth.uniform(12, 20000) * 2 - 1) * 2.0 ** -6
    x = np.concatenate([pts, -pts, rnd, tiny]).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert np.array_equal(oracle.e4m3_encode(x), _e4m3_torch(x))
    # signed zero is kept
    assert oracle.e4m3_encode(np.array([-0.0, -1e-30, 0.0], np.float32)).tolist() == [0x80, 0x80, 0x00]
    # saturation
    assert oracle.e4m3_encode(np.array([1e6, -470.0], np.float32)).tolist() == [0x7E, 0xFE]


def test_e4m3_round_trip_all_finite():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


# ------------------------------------------------------------------------------------------
# Level-1 quantization (notes section 3.1, section 3.2)
# ------------------------------------------------------------------------------------------

def _exact_codes(W, cb, block):
    """Exact rational argmin over the 16 codewords, ties to the lower index."""
    W = np.asarray(W, np.float32).reshape(-1)
    out = []
    cbf = [Fraction(float(c)) for c in cb]
    zc = next(j for j in range(16) if cb[j] == 0)
    for b0 in range(0, W.size, block):
        blk = W[b0:b0 + block]
        a = np.max(np.abs(blk))
        for x in blk:
            if a == 0:
                out.append(zc)
                continue
            n = Fraction(float(np.float32(x) / np.float32(a)))      # IEEE float32 division
            d = [abs(n - c) for c in cbf]
            out.append(min(range(16), key=lambda j: (d[j], j)))
    return np.array(out, dtype=np.uint8)


def test_quantize_golden_absmax_example():
    g = GOLDEN["absmax_example"]
    W = np.array(g["block"], dtype=np.float32)
    packed, absmax = oracle.quantize(W, block=len(g["block"]))
    assert absmax.tolist() == [g["absmax"]]
    codes = oracle.unpack(packed, W.size)
    assert codes[0] == 0                       # -absmax maps to the -1 endpoint
    assert np.array_equal(codes, _exact_codes(W, oracle.codebook(), 3))


def test_quantize_matches_exact_brute_force_adversarial():
    cb = oracle.codebook()
    mids = (cb[:-1].astype(np.float64) + cb[1:]) / 2
    vals = []
    for m in mids:
        f = np.float32(m)
        vals += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
    vals = np.array(vals, dtype=np.float32)
    blocks = []
    for scale in (1.0, 0.37, 3.0e-5, 1.7e3):
        blk = np.concatenate([[np.float32(scale)], vals * np.float32(scale)]).astype(np.float32)
        blk = np.resize(blk, 64)
        blocks.append(blk)
    rnd = synth.normal_f32(21, (8 * 64,), 0.02)
    W = np.concatenate(blocks + [rnd])
    packed, absmax = oracle.quantize(W, cb)
    assert np.array_equal(oracle.unpack(packed, W.size), _exact_codes(W, cb, 64))


def test_quantize_exact_zero_and_zero_block():
    W = synth.normal_f32(22, (4, 64), 1.0)
    W[1, :] = 0.0                  # an all-zero block
    W[2, ::3] = 0.0                # zeros inside a live block
    W[3, 5] = -0.0
    packed, absmax = oracle.quantize(W)
    codes = oracle.unpack(packed, W.size).reshape(4, 64)
    assert absmax[1] == 0.0
    assert np.all(codes[1] == 7) and np.all(codes[2, ::3] == 7) and codes[3, 5] == 7
    deq = oracle.bf16_to_f32(oracle.dequant_plain(packed, absmax, W.size)).reshape(4, 64)
    assert np.all(deq[W == 0] == 0.0)


def test_quantize_codebook_round_trip_is_lossless():
    cb = oracle.codebook()
    for e in (-20, -3, 0, 7):
        W = (np.tile(cb, 4) * np.float32(2.0 ** e)).astype(np.float32)
        packed, absmax = oracle.quantize(W, cb)
        assert np.all(absmax == np.float32(2.0 ** e))
        codes = oracle.unpack(packed, W.size)
        assert np.array_equal(codes, np.tile(np.arange(16, dtype=np.uint8), 4))
        assert np.array_equal(cb[codes] * absmax[0], W)


# ---- alternative 4-bit types (Int4, FP4): readings, pinned to eq. (1) and to torch's E2M1 ----

def _e2m1():
    """torch's reference E2M1 codec (its MX test helpers: encode rounds to nearest even and
    saturates, decode maps the 4-bit codes).  Those helpers import the test-only package
    ``expecttest``, absent from this image; a stand-in module supplies its one name."""
    import sys
    import types
    import unittest
    if "expecttest" not in sys.modules:
        try:
            import expecttest  # noqa: F401
        except ImportError:
            stub = types.ModuleType("expecttest")
            stub.TestCase = unittest.TestCase
            sys.modules["expecttest"] = stub
    try:
        from torch.testing._internal.common_quantized import _f32_to_floatx_unpacked, _floatx_unpacked_to_f32
    except Exception as e:  # pragma: no cover - depends on the torch build
        pytest.skip("torch's E2M1 reference codec is not importable: %s" % e)
    return (lambda x: _f32_to_floatx_unpacked(x, 2, 1)), (lambda c: _floatx_unpacked_to_f32(c, 2, 1))


def test_int4_codebook_quantize_is_eq1_at_4_bits():
    """Nearest Int4 codeword of n = x / absmax is eq. (1) with 2^3 - 1 = 7 levels per side."""
    cb = oracle.codebook_int4()
    assert np.all(np.diff(cb) > 0) and cb[8] == 0.0
    W = np.concatenate([synth.normal_f32(61, (64, 64), 0.02).reshape(-1),
                        (synth.uniform(62, 32 * 64) * 6.0 - 3.0).astype(np.float32)])
    packed, absmax = oracle.quantize(W, cb)
    codes = oracle.unpack(packed, W.size).astype(np.int64)
    n = (W.reshape(-1, 64) / absmax[:, None]).astype(np.float32).reshape(-1)   # fp32 division
    t = 7.0 * n.astype(np.float64)
    ref = np.rint(t)
    tie = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-6
    assert tie.sum() < 4
    assert np.array_equal((codes - 8)[~tie], ref[~tie].astype(np.int64))
    assert codes.min() >= 1                      # k = -8 is never produced
    assert set(np.unique(codes - 8)) <= set(range(-7, 8))
    # every block's absmax element maps to +-7 exactly
    blk = codes.reshape(-1, 64)
    assert np.all(np.max(np.abs(blk - 8), axis=1) == 7)


def test_int4_ties_go_to_the_lower_index():
    cb = oracle.codebook_int4()
    # 7 n = k + 1/2 exactly representable: n = (2k + 1) / 14 with absmax 1 in the block
    W = np.zeros(64, dtype=np.float32)
    W[0] = 1.0
    ks = np.arange(-7, 7)
    W[1:1 + ks.size] = ((2 * ks + 1) / 14.0).astype(np.float32)
    packed, _ = oracle.quantize(W, cb)
    codes = oracle.unpack(packed, W.size)
    assert np.array_equal(codes[1:1 + ks.size], _exact_codes(W, cb, 64)[1:1 + ks.size])


def test_fp4_codebook_is_e2m1_over_its_max():
    enc, dec = _e2m1()
    vals = dec(torch.arange(16, dtype=torch.uint8)).double().numpy()
    cb = oracle.codebook_fp4()
    assert cb.size == 16 and np.all(np.diff(cb) >= 0)
    assert np.count_nonzero(cb == 0.0) == 2 and not np.any(np.signbit(cb[cb == 0.0]))
    assert np.max(vals) == 6.0
    assert np.array_equal(np.unique(cb), np.unique((vals / 6.0).astype(np.float32)))
    assert np.array_equal(cb, -cb[::-1])


def test_fp4_quantize_is_e2m1_rounding_of_6n():
    """Nearest FP4 codeword of n is the E2M1 rounding of 6 n (away from the rounding ties)."""
    enc, dec = _e2m1()
    cb = oracle.codebook_fp4()
    W = np.concatenate([synth.normal_f32(63, (64, 64), 0.02).reshape(-1),
                        (synth.uniform(64, 32 * 64) * 2.0 - 1.0).astype(np.float32)])
    packed, absmax = oracle.quantize(W, cb)
    codes = oracle.unpack(packed, W.size)
    n = (W.reshape(-1, 64) / absmax[:, None]).astype(np.float32).reshape(-1)
    ref = dec(enc(torch.from_numpy(6.0 * n.astype(np.float64)).float())).double().numpy()
    grid = np.unique(np.abs(dec(torch.arange(8, dtype=torch.uint8)).double().numpy()))
    mids = (grid[:-1] + grid[1:]) / 2
    near_tie = np.min(np.abs(np.abs(6.0 * n.astype(np.float64))[:, None] - mids[None, :]), axis=1) < 1e-5
    assert near_tie.sum() < 8
    assert np.array_equal(cb[codes][~near_tie], (ref[~near_tie] / 6.0).astype(np.float32))
    assert np.array_equal(codes[~near_tie], _exact_codes(W, cb, 64)[~near_tie])
    assert not np.any(codes == 8)                # the second zero slot is never produced


def test_quantize_invariants_random():
    cb = oracle.codebook()
    W = synth.normal_f32(23, (64, 256), 0.02)
    packed, absmax = oracle.quantize(W, cb)
    codes = oracle.unpack(packed, W.size).reshape(-1, 64)
    blocks = W.reshape(-1, 64)
    assert np.array_equal(absmax, np.max(np.abs(blocks), axis=1))
    # the absmax element goes to an endpoint
    am = np.argmax(np.abs(blocks), axis=1)
    assert np.all(np.isin(codes[np.arange(blocks.shape[0]), am], [0, 15]))
    # monotone within a block
    for b in range(blocks.shape[0]):
        o = np.argsort(blocks[b], kind="stable")
        assert np.all(np.diff(codes[b][o].astype(int)) >= 0)
    # closed-form error bound: half the widest codeword gap times the block absmax
    gap = float(np.max(np.diff(cb.astype(np.float64))))
    rec = cb[codes].astype(np.float64) * absmax[:, None]
    err = np.abs(rec - blocks)
    assert np.all(err <= absmax[:, None] * (gap / 2) * (1 + 1e-6))
    # blocks run along the row-major flattening: permuting rows permutes blocks
    perm = np.random.default_rng(0).permutation(W.shape[0])
    p2, a2 = oracle.quantize(W[perm], cb)
    assert np.array_equal(a2.reshape(W.shape[0], -1), absmax.reshape(W.shape[0], -1)[perm])


def test_quantize_short_tail_and_odd_numel():
    W = synth.normal_f32(24, (131,), 1.0)
    packed, absmax = oracle.quantize(W)
    assert absmax.size == 3 and packed.size == 66
    assert absmax[2] == np.max(np.abs(W[128:]))
    assert packed[-1] >> 4 == 7                     # pad nibble is the zero code
    assert np.array_equal(oracle.unpack(packed, 131), _exact_codes(W, oracle.codebook(), 64))


def test_nibble_order():
    cb = oracle.codebook()
    W = np.zeros(64, np.float32)
    W[0], W[1] = -1.0, 1.0                          # codes 0 and 15
    packed, _ = oracle.quantize(W, cb)
    assert packed[0] == 0xF0
    assert np.all(packed[1:] == 0x77)


# ------------------------------------------------------------------------------------------
# Double quantization (notes section 3.3)
# ------------------------------------------------------------------------------------------

def test_grouped_sum_small_is_sequential_and_exact_cases():
    v = synth.normal(31, 200)
    seq = 0.0
    for x in v:
        seq += float(x)
    assert oracle.grouped_sum(v) == seq
    ints = np.floor(synth.uniform(32, 100000) * 1e6)
    assert oracle.grouped_sum(ints) == math.fsum(ints)
    # two levels: sum of the 256-group sequential sums, itself sequential
    w = synth.uniform(33, 256 * 40 + 17) * 1e-3
    gs = []
    for i in range(0, w.size, 256):
        s = 0.0
        for x in w[i:i + 256]:
            s += float(x)
        gs.append(s)
    tot = 0.0
    for s in gs:
        tot += s
    assert oracle.grouped_sum(w) == tot


def test_grouped_sum_three_levels_closed_form():
    """The order past two levels, on values whose float64 sum depends on it.

    131072 values form 512 groups of 256, then 2 groups, then 1: three levels.  Value 0 is 2^53
    and each later 256-group holds a single 1.0, the rest zero.
      level 1: group 0 sums to 2^53, groups 1 .. 511 to 1.0 each (exact);
      level 2: the first 256 sums are 2^53 followed by 255 ones; each one is added to 2^53 on its
               own, and 2^53 + 1 lies half-way between 2^53 and 2^53 + 2, so ties-to-even keeps
               2^53 every time.  The second 256 sums add up to 256 exactly;
      level 3: 2^53 + 256, exact.
    A plain sequential sum, and a sequential sum of the 256-group sums (two levels), both keep
    2^53; the exact sum is 2^53 + 511.  Each of these readings therefore gives a different value."""
    v = np.zeros(131072)
    v[0] = 2.0 ** 53
    v[256::256] = 1.0
    assert oracle.grouped_sum(v) == 2.0 ** 53 + 256
    assert math.fsum(v) == 2.0 ** 53 + 511
    seq = 0.0
    for x in v[v != 0]:
        seq += float(x)
    assert seq == 2.0 ** 53


@pytest.mark.parametrize("nb", [262144, 3670016])
def test_double_quant_mean_is_the_exact_mean_to_one_ulp(nb):
    """The stored mean against the exactly rounded sum (math.fsum) over n, on non-integer block
    constants at the 7B-projection and decode-weight block counts (three summation levels at the
    larger).  The float64 sum's rounding error is far below float32's, so the two agree within
    one unit in the last place of the float32 mean."""
    a = (synth.uniform(36 + nb % 7, nb) * 0.08 + 0.011).astype(np.float32)
    _, _, mean = oracle.double_quant(a)
    exact = np.float32(math.fsum(a.astype(np.float64)) / nb)
    assert abs(int(np.float32(mean).view(np.int32)) - int(exact.view(np.int32))) <= 1
    assert a.size == nb and not np.all(a == np.floor(a))


def test_memory_accounting_golden():
    g = GOLDEN["constant_overhead_bits"]
    gb = GOLDEN["block_sizes"]
    W = synth.normal_f32(34, (64, 1024), 0.02)
    packed, absmax = oracle.quantize(W, block=gb["weight_block"])
    codes, scales, mean = oracle.double_quant(absmax, dq_block=gb["dq_block"])
    n = W.size
    single = absmax.nbytes * 8 / n
    dq = (codes.nbytes + scales.nbytes) * 8 / n
    assert single == g["fp32_per_64"]
    assert round(dq, 3) == g["double_quant"]
    assert round(single - dq, 3) == g["saving"]
    assert packed.nbytes * 8 / n == 4
    s65 = GOLDEN["dq_saving_65b"]
    assert round(single - dq, 2) == s65["bits_per_param"]
    assert round((single - dq) * s65["params"] / 8 / 1e9) == s65["gigabytes"]


# ---- quantization-error statistics (NF4 against Int4 and FP4, with and without DQ) ----

def test_quant_error_bits_per_param_golden():
    g = GOLDEN["constant_overhead_bits"]
    assert oracle.bits_per_parameter(False) - 4 == g["fp32_per_64"]
    assert round(oracle.bits_per_parameter(True) - 4, 3) == g["double_quant"]
    assert round(oracle.bits_per_parameter(False) - oracle.bits_per_parameter(True), 3) == g["saving"]


def test_quant_error_exact_cases():
    # FP4 on its bf16-exact codewords (0, +-1/2, +-1) times powers of two: no error at all
    # (with DQ every block needs the same absmax: then the codes are 0 and a' is the mean exactly)
    base = np.float32([-1.0, -0.5, 0.0, 0.5, 1.0])
    for dq, exps in ((False, (-8, 0, 5)), (True, (5, 5, 5))):
        W = np.concatenate([np.resize(base, 64) * np.float32(2.0 ** e) for e in exps]).astype(np.float32)
        r = oracle.quant_error(W, oracle.codebook_fp4(), dq=dq)
        assert r["mse"] == 0.0 and r["max_abs"] == 0.0
        assert r["occupancy"].sum() == W.size
    # NF4 on its own codewords (absmax 1 in every block): each code once per 16 elements, 4 bits
    # of entropy, and the only error is bf16's rounding of the codewords (torch's cast)
    cb = oracle.codebook()
    W = np.tile(cb, 32).astype(np.float32)
    ref = torch.from_numpy(W).to(torch.bfloat16).double().numpy() - W.astype(np.float64)
    for dq in (False, True):
        r = oracle.quant_error(W, cb, dq=dq)
        assert np.all(r["occupancy"] == W.size // 16)
        assert abs(r["entropy_bits"] - 4.0) < 1e-12
        assert math.isclose(r["mse"], float(np.mean(ref * ref)), rel_tol=1e-12)
        assert r["max_abs"] == float(np.max(np.abs(ref)))


def test_quant_error_nf4_beats_int4_and_fp4_on_normal_weights():
    """[S] 5.1.2: NF4 is clearly better than the 4-bit float and integer types.  On normally
    distributed weights its error is the lowest and its codes are the most evenly used."""
    W = synth.normal_f32(71, (256, 1024), 0.02)
    res = {k: oracle.quant_error(W, cb, dq=True)
           for k, cb in (("nf4", oracle.codebook()), ("int4", oracle.codebook_int4()), ("fp4", oracle.codebook_fp4()))}
    assert res["nf4"]["mse"] < res["fp4"]["mse"] < res["int4"]["mse"]
    assert res["nf4"]["entropy_bits"] > res["fp4"]["entropy_bits"] > res["int4"]["entropy_bits"]
    # DQ saves 0.373 bits per weight for a small increase of the error
    plain = oracle.quant_error(W, oracle.codebook(), dq=False)
    assert plain["mse"] <= res["nf4"]["mse"] < 1.01 * plain["mse"]


def test_double_quant_int8_is_eq1_on_the_centred_constants():
    """Integer second level: eq. (1) at 8 bits, round(127 y / max|y|) per 256-block, y = a - mean."""
    a = np.abs(synth.normal_f32(81, (5000,), 0.05)).astype(np.float32)
    c, sc, m = oracle.double_quant(a, fmt="int8")
    _, _, m_e4 = oracle.double_quant(a)
    assert np.float32(m).view(np.uint32) == np.float32(m_e4).view(np.uint32)   # same mean
    codes = c.view(np.int8).astype(np.int64)
    y = (a - np.float32(m)).astype(np.float32)
    rebuilt = oracle.block_scales(c, sc, m, fmt="int8").astype(np.float64)
    for j in range(sc.size):
        blk = slice(256 * j, min(256 * (j + 1), a.size))
        yj = [Fraction(float(v)) for v in y[blk]]
        A = max(abs(v) for v in yj)
        assert abs(Fraction(float(sc[j])) * 127 - A) <= A * Fraction(1, 1 << 23)     # s = A / 127
        for code, v in zip(codes[blk], yj):
            assert abs(code - 127 * v / A) <= Fraction(1, 2) + Fraction(1, 1 << 20)
        k = int(np.argmax(np.abs(y[blk])))
        assert abs(codes[blk][k]) == 127
        # the rebuilt constant is within half a step of the original (plus float rounding)
        err = np.abs(rebuilt[blk] - a[blk].astype(np.float64))
        assert np.all(err <= float(sc[j]) * (0.5 + 1e-6) + 4 * np.spacing(np.float32(a.max())))


def test_double_quant_int8_constant_tensor():
    a = np.full(700, 0.0375, np.float32)
    c, sc, m = oracle.double_quant(a, fmt="int8")
    assert np.all(c == 0) and np.all(sc == 0.0) and m == np.float32(0.0375)
    assert np.all(oracle.block_scales(c, sc, m, fmt="int8") == np.float32(0.0375))


def test_double_quant_constant_and_single_block():
    a = np.full(1000, 0.0371, dtype=np.float32)
    codes, scales, mean = oracle.double_quant(a)
    assert mean == np.float32(0.0371)
    assert np.all(codes == 0) and np.all(scales == 0)
    assert np.all(oracle.block_scales(codes, scales, mean) == np.float32(0.0371))
    codes, scales, mean = oracle.double_quant(np.array([0.25], np.float32))
    assert mean == 0.25 and codes[0] == 0 and scales[0] == 0


def _round_f32_exact(fr: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational, ties to even (independent of fmaf)."""
    c = np.float32(float(fr))
    cands = [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))]
    def key(v):
        return (abs(Fraction(float(v)) - fr), int(np.array(v, np.float32).view(np.uint32)) & 1)
    return min(cands, key=key)


def test_double_quant_properties_and_fma():
    W = synth.normal_f32(35, (32, 4096), 0.02)
    _, absmax = oracle.quantize(W)
    codes, scales, mean = oracle.double_quant(absmax)
    nb = absmax.size
    # mean: float32 of the grouped float64 sum divided by n
    assert mean == np.float32(oracle.grouped_sum(absmax.astype(np.float64)) / nb)
    y = (absmax - mean).astype(np.float32)
    A = np.max(np.abs(y.reshape(-1, 256)), axis=1)
    assert np.array_equal(scales, (A / np.float32(448)).astype(np.float32))
    # the codes are E4M3 of the clamped scaled residuals, checked with torch's cast
    t = np.clip((y.reshape(-1, 256) / scales[:, None]).astype(np.float32), -448, 448).reshape(-1)
    assert np.array_equal(codes, _e4m3_torch(t))
    # centring by the mean gives codes of both signs
    neg = np.mean(codes >= 0x80)
    assert 0.2 < neg < 0.8
    # rebuilt constants: exact rational fma, then correct rounding to float32
    ap = oracle.block_scales(codes, scales, mean)
    dec = oracle.e4m3_decode(codes)
    for b in range(0, nb, 97):
        fr = Fraction(float(dec[b])) * Fraction(float(scales[b // 256])) + Fraction(float(mean))
        assert ap[b] == _round_f32_exact(fr)
    # error bound of the rebuilt constant: half an E4M3 step at |t| (relative 2^-4), or the
    # subnormal spacing 2^-9, in units of the 256-block multiplier
    s = np.repeat(scales, 256)[:nb]
    bound = np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10) * s + np.abs(absmax) * 2e-7
    assert np.all(np.abs(ap.astype(np.float64) - absmax) <= bound)


def test_double_quant_short_tail():
    a = np.abs(synth.normal_f32(36, (300,), 1.0))
    codes, scales, mean = oracle.double_quant(a)
    assert scales.size == 2
    assert scales[1] == np.float32(np.max(np.abs(a[256:] - mean)) / np.float32(448))


# ------------------------------------------------------------------------------------------
# Double dequantization (notes section 3.5, eq. 6)
# ------------------------------------------------------------------------------------------

def test_dequant_matches_torch_composition():
    cb = oracle.codebook()
    W = synth.normal_f32(41, (16, 512), 0.02)
    q = oracle.quantize_dq(W, cb)
    ap = oracle.block_scales(q["codes"], q["scales"], q["mean"])
    idx = oracle.unpack(q["packed"], W.size)
    prod = torch.from_numpy(cb[idx]) * torch.from_numpy(np.repeat(ap, 64))     # float32 multiply
    ref = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.dequant(q["packed"], q["codes"], q["scales"], q["mean"], W.size, cb), ref)


def test_dequant_zero_block_sign():
    W = synth.normal_f32(42, (8, 64), 0.02)
    W[3] = 0.0
    q = oracle.quantize_dq(W)
    ap = oracle.block_scales(q["codes"], q["scales"], q["mean"])
    d = oracle.dequant_weight(q)
    assert np.all(oracle.bf16_to_f32(d[3]) == 0.0)
    if ap[3] < 0:
        assert np.all(d[3] == 0x8000)
    else:
        assert np.all(d[3] == 0x0000)


def test_full_pipeline_error_bound():
    cb = oracle.codebook()
    W = synth.normal_f32(43, (64, 1024), 0.02)
    q = oracle.quantize_dq(W, cb)
    ap = oracle.block_scales(q["codes"], q["scales"], q["mean"]).astype(np.float64)
    deq = oracle.bf16_to_f32(oracle.dequant_weight(q, cb)).astype(np.float64).reshape(-1, 64)
    gap = float(np.max(np.diff(cb.astype(np.float64))))
    a = q["absmax"].astype(np.float64)[:, None]
    bound = np.abs(a) * gap / 2 + np.abs(ap[:, None] - a) + np.abs(deq) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(deq - W.reshape(-1, 64)) <= bound)


# ------------------------------------------------------------------------------------------
# QLoRA linear layer (notes section 3.5 eq. 5, section 4 eq. 3)
# ------------------------------------------------------------------------------------------

def _tiny():
    wl = synth.WORKLOADS["tiny"]
    lin = wl.linears[0]
    W = synth.weight_f32(wl, lin)
    Wd = oracle.dequant_weight(oracle.quantize_dq(W))
    l1, l2 = synth.lora_f32(wl, lin)
    X = synth.to_bf16_bits(synth.x_f32(wl))
    dY = synth.to_bf16_bits(synth.dy_f32(wl, wl.M, lin.N))
    return wl, Wd, synth.to_bf16_bits(l1), synth.to_bf16_bits(l2), X, dY


def _t64(bits):
    return torch.from_numpy(oracle.bf16_to_f32(bits).astype(np.float64))


def test_forward_special_cases():
    wl, Wd, L1, L2, X, _ = _tiny()
    s = wl.scale
    Y, T = oracle.forward(X, Wd, L1, L2, s)
    # L2 = 0: plain product with the dequantized weight (torch fp64 matmul)
    Y0, _ = oracle.forward(X, Wd, L1, np.zeros_like(L2), s)
    assert np.allclose(Y0, (_t64(X) @ _t64(Wd).T).numpy(), rtol=1e-13, atol=1e-13)
    # zero weight (quantized zeros dequantize exactly to 0): pure LoRA branch
    Wz = oracle.dequant_weight(oracle.quantize_dq(np.zeros((256, 256), np.float32)))
    assert np.all(oracle.bf16_to_f32(Wz) == 0)
    Yz, _ = oracle.forward(X, Wz, L1, L2, s)
    assert np.allclose(Yz, (s * (_t64(X) @ _t64(L1)) @ _t64(L2)).numpy(), rtol=1e-13, atol=1e-15)
    # identity input reproduces deq(W)^T + s L1 L2
    I = synth.to_bf16_bits(np.eye(256, dtype=np.float32))
    YI, _ = oracle.forward(I, Wd, L1, L2, s)
    ref = _t64(Wd).T + s * _t64(L1) @ _t64(L2)
    assert np.allclose(YI, ref.numpy(), rtol=1e-13, atol=1e-15)
    assert np.allclose(T, (_t64(X) @ _t64(L1)).numpy(), rtol=1e-13, atol=1e-15)


def test_backward_matches_torch_autograd():
    wl, Wd, L1, L2, X, dY = _tiny()
    s = wl.scale
    g = oracle.backward(dY, X, Wd, L1, L2, s)
    x = _t64(X).requires_grad_(True)
    l1 = _t64(L1).requires_grad_(True)
    l2 = _t64(L2).requires_grad_(True)
    w = _t64(Wd).requires_grad_(False)
    y = x @ w.T + s * (x @ l1) @ l2
    (y * _t64(dY)).sum().backward()
    for name, t in (("dX", x), ("dL1", l1), ("dL2", l2)):
        assert np.allclose(g[name], t.grad.numpy(), rtol=1e-12, atol=1e-13), name


def test_backward_rows_matches_autograd_on_a_row_subset():
    """The full-size spot-check form: adapter gradients over every token, dX on chosen rows only,
    against torch float64 autograd of the whole layer."""
    wl, Wd, L1, L2, X, dY = _tiny()
    s = wl.scale
    rows = np.array([0, 3, 7])
    g = oracle.backward_rows(dY, X, Wd, L1, L2, s, rows)
    x = _t64(X).requires_grad_(True)
    l1 = _t64(L1).requires_grad_(True)
    l2 = _t64(L2).requires_grad_(True)
    y = x @ _t64(Wd).T + s * (x @ l1) @ l2
    (y * _t64(dY)).sum().backward()
    assert np.allclose(g["dX"], x.grad.numpy()[rows], rtol=1e-12, atol=1e-13)
    assert np.allclose(g["dL1"], l1.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(g["dL2"], l2.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert g["dX"].shape == (rows.size, X.shape[1])


def test_backward_finite_differences():
    wl, Wd, L1, L2, X, dY = _tiny()
    s = wl.scale
    g = oracle.backward(dY, X, Wd, L1, L2, s)
    l1 = oracle.bf16_to_f32(L1).astype(np.float64)
    l2 = oracle.bf16_to_f32(L2).astype(np.float64)
    x = oracle.bf16_to_f32(X).astype(np.float64)
    dy = oracle.bf16_to_f32(dY).astype(np.float64)

    def E(x_, l1_, l2_):
        Y, _ = oracle.forward(x_, Wd, l1_, l2_, s)
        return float(np.sum(Y * dy))

    h = 1e-5
    for (i, j) in [(0, 0), (17, 3), (255, 7)]:
        e = np.zeros_like(l1); e[i, j] = h
        fd = (E(x, l1 + e, l2) - E(x, l1 - e, l2)) / (2 * h)
        assert abs(fd - g["dL1"][i, j]) <= 1e-7 * max(1.0, abs(fd))
    for (i, j) in [(0, 0), (5, 200)]:
        e = np.zeros_like(l2); e[i, j] = h
        fd = (E(x, l1, l2 + e) - E(x, l1, l2 - e)) / (2 * h)
        assert abs(fd - g["dL2"][i, j]) <= 1e-7 * max(1.0, abs(fd))
    for (i, j) in [(0, 0), (7, 100)]:
        e = np.zeros_like(x); e[i, j] = h
        fd = (E(x + e, l1, l2) - E(x - e, l1, l2)) / (2 * h)
        assert abs(fd - g["dX"][i, j]) <= 1e-7 * max(1.0, abs(fd))


def test_swiglu_matches_torch():
    g = synth.normal_f32(51, (16, 64), 1.0).astype(np.float64)
    u = synth.normal_f32(52, (16, 64), 1.0).astype(np.float64)
    dh = synth.normal_f32(53, (16, 64), 1.0).astype(np.float64)
    tg = torch.from_numpy(g).requires_grad_(True)
    tu = torch.from_numpy(u).requires_grad_(True)
    h = torch.nn.functional.silu(tg) * tu
    (h * torch.from_numpy(dh)).sum().backward()
    assert np.allclose(oracle.swiglu_fwd(g, u), h.detach().numpy(), rtol=1e-14, atol=1e-15)
    dg, du = oracle.swiglu_bwd(dh, g, u)
    assert np.allclose(dg, tg.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(du, tu.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_tolerance_measures():
    ref = np.array([[1.0, -2.0], [3.0, 0.5]])
    assert oracle.rel_fro(ref, ref) == 0 and oracle.max_abs_ratio(ref, ref) == 0
    assert not oracle.within_tolerance(ref * 1.01, ref)
    assert oracle.within_tolerance(ref * (1 + 1e-3), ref)
