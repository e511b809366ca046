"""Pins of the oracle's number codecs (CPU).

E4M3 is pinned to torch's float8_e4m3fn (an independent implementation of the
OCP format) and to a brute-force nearest-value search; INT8 to its closed-form
error bound.
"""
import numpy as np
import pytest
import torch

from oracle import codecs

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def brute_nearest(x):
    """Nearest finite E4M3 value by exhaustive search; ties go to the even code; saturating."""
    vals = codecs.e4m3_decode(np.array(FINITE, np.uint8))
    codes = np.array(FINITE)
    out = np.empty_like(x)
    for n, xv in enumerate(x):
        if abs(xv) > 448.0:
            out[n] = np.copysign(448.0, xv)
            continue
        dist = np.abs(vals - xv)
        best = dist.min()
        cand = codes[dist == best]
        cand_vals = vals[dist == best]
        if len(cand) > 1:
            even = cand_vals[(cand & 1) == 0]
            # +0 and -0 are both at distance |x| from x = 0-ish values: keep the sign of x
            same_sign = even[np.signbit(even) == np.signbit(xv)] if len(even) > 1 else even
            out[n] = same_sign[0]
        else:
            out[n] = cand_vals[0]
    return out


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.array_equal(ours[~nan], ref[~nan])
    # format landmarks of OCP E4M3
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def test_round_matches_brute_force_and_torch():
    rng = np.random.default_rng(0)
    vals = codecs.e4m3_decode(np.array(FINITE, np.uint8))
    pos = np.sort(np.unique(vals[vals > 0]))
    mids = (pos[1:] + pos[:-1]) / 2                       # exact ties
    x = np.concatenate([
        rng.standard_normal(4000) * 50,
        np.exp(rng.uniform(np.log(1e-4), np.log(600), 4000)),
        mids, -mids, pos, -pos, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        [0.0, 2.0 ** -10, 3 * 2.0 ** -11, 447.9, 448.0, 460.0, 464.0, 470.0, 1e6, -1e6],
    ])
    ours = codecs.e4m3_round(x)
    assert np.array_equal(ours, brute_nearest(x))
    inrange = np.abs(x) < 464.0
    ref = torch.from_numpy(x[inrange].astype(np.float32)).to(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    # torch converts from float32: compare on inputs that are exactly fp32
    exact32 = x[inrange].astype(np.float32).astype(np.float64) == x[inrange]
    assert np.array_equal(ours[inrange][exact32], ref[exact32])


def test_encode_decode_roundtrip():
    codes = np.array([c for c in FINITE if c != 0x80], np.uint8)
    assert np.array_equal(codecs.e4m3_encode(codecs.e4m3_decode(codes)), codes)
    x = np.random.default_rng(1).standard_normal(1000) * 100
    assert np.array_equal(codecs.e4m3_decode(codecs.e4m3_encode(x)), codecs.e4m3_round(x))


def test_int8_block_codec_bounds():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((256, 128)) * rng.uniform(0.1, 10, (256, 1))).astype(np.float32)
    x[128:192] = 0.0                                      # one all-zero block of 64 rows
    codes, s = codecs.int8_block_quant(x, 64)
    assert codes.dtype == np.int8 and s.dtype == np.float32
    assert s[2] == 0 and not codes[128:192].any()
    for b in (0, 1, 3):
        blk = x[b * 64:(b + 1) * 64].astype(np.float64)
        cb = codes[b * 64:(b + 1) * 64].astype(np.float64)
        amax = np.abs(blk).max()
        assert abs(s[b] - amax / 127) <= 1e-7 * amax
        # reconstruction within half a step (plus fp32 rounding of the scale)
        assert np.all(np.abs(blk - cb * s[b]) <= s[b] * (0.5 + 1e-5))
        # the element holding amax maps to +-127
        r, c = np.unravel_index(np.abs(blk).argmax(), blk.shape)
        assert abs(cb[r, c]) == 127 and np.sign(cb[r, c]) == np.sign(blk[r, c])
        assert np.abs(cb).max() <= 127


def test_fp8_block_codec_amax_maps_to_448():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((128, 128)).astype(np.float32)
    codes, s = codecs.fp8_block_quant(v, 64)
    dec = codecs.e4m3_decode(codes)
    for b in range(2):
        blk = v[b * 64:(b + 1) * 64].astype(np.float64)
        r, c = np.unravel_index(np.abs(blk).argmax(), blk.shape)
        assert abs(dec[b * 64 + r, c]) == 448.0
        rel = np.abs(dec[b * 64:(b + 1) * 64] * s[b] - blk)
        # E4M3 normal values carry 3 mantissa bits: error <= 2^-4 relative (+ subnormal floor)
        assert np.all(rel <= np.abs(blk) * 2.0 ** -4 + s[b] * 2.0 ** -10 + 1e-12)


@pytest.mark.parametrize("amax", [1e-30, 1e30])
def test_codecs_extreme_scales(amax):
    x = np.zeros((64, 128), np.float32)
    x[3, 7] = amax
    x[5, 9] = -amax / 2
    c8, s8 = codecs.int8_block_quant(x, 64)
    assert c8[3, 7] == 127 and c8[5, 9] in (-63, -64)
    cf, sf = codecs.fp8_block_quant(x, 64)
    d = codecs.e4m3_decode(cf)
    assert d[3, 7] == 448.0 and d[5, 9] == -224.0
