"""Pins of the oracle's encoders and of the quantising-append policy
(oracle/quantize.py) against references that are not the oracle itself:
torch's float8_e4m3fn cast, the OCP MX v1.0 rounding rule written out as a
table, closed forms of the block exponent, and invariants of the open-chunk
policy.  Mutation tests plant mistakes in copies of the policy and check that
a pin fails."""

import numpy as np
import pytest
import torch

from oracle import codecs as ocod
from oracle import quantize as oq


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encoder_matches_torch_cast():
    rng = np.random.default_rng(0)
    finite = ocod.FP8_E4M3[:0x7F]
    mids = (finite[:-1] + finite[1:]) / 2                      # every tie between neighbours
    vals = np.concatenate([
        finite, mids, -mids, -finite,
        rng.uniform(-448, 448, 20000),
        rng.normal(0, 1, 20000) * 2.0 ** rng.integers(-12, 8, 20000),
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        np.nextafter(mids.astype(np.float32), np.float32(-np.inf)),
        [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, -(2.0 ** -10), 1e-30, -1e-30],
    ]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    got = oq.encode_e4m3(vals)
    ref = _torch_e4m3(vals)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]


def test_e2m1_encoder_follows_the_ocp_rounding_table():
    # OCP MX v1.0: round to nearest, ties to even, saturate at the largest magnitude 6
    table = {
        0.0: 0, 0.1: 0, 0.25: 0, 0.26: 1, 0.5: 1, 0.74: 1, 0.75: 2, 1.0: 2, 1.25: 2, 1.3: 3, 1.5: 3,
        1.75: 4, 2.0: 4, 2.5: 4, 2.6: 5, 3.0: 5, 3.5: 6, 4.0: 6, 4.9: 6, 5.0: 6, 5.1: 7, 6.0: 7, 7.9: 7, 1e9: 7,
    }
    for v, code in table.items():
        assert oq.encode_e2m1(np.float32(v)) == code, v
        if code:
            assert oq.encode_e2m1(np.float32(-v)) == code | 8, -v
    assert oq.encode_e2m1(np.float32(-0.2)) == 0          # rounds to zero: the positive zero code
    assert oq.encode_e2m1(np.float32(-0.0)) == 0
    # decoding the code of a grid value gives it back
    for c in range(16):
        v = ocod.E2M1[c]
        assert ocod.E2M1[oq.encode_e2m1(np.float32(v))] == v


@pytest.mark.parametrize("k", range(-130, 129, 7))
def test_mxfp4_block_exponent_closed_form(k):
    for amax in (2.0 ** k, 1.5 * 2.0 ** k, np.nextafter(2.0 ** (k + 1), 0)):
        if not np.isfinite(amax) or amax == 0:
            continue
        E = int(oq.mxfp4_block_exponent(np.float64(amax)))
        assert E == min(max(k - 2, -127), 127) + 127
        if -125 <= k <= 129:
            assert 4.0 <= amax / 2.0 ** (E - 127) < 8.0
    assert int(oq.mxfp4_block_exponent(np.float64(0.0))) == 0


def test_mxfp4_rows_decode_within_half_a_grid_step_or_saturate():
    rng = np.random.default_rng(1)
    x = (rng.normal(0, 1, (64, 128)) * 2.0 ** rng.integers(-20, 20, (64, 1))).astype(np.float32)
    packed, E = oq.quantize_mxfp4_rows(x)
    back = ocod.dequant_mxfp4(packed, E)
    unit = np.repeat(2.0 ** (E.astype(np.float64) - 127), 32, axis=-1)
    # grid spacing is at most 2 units of 2^(E-127): error <= 1 unit, or < 2 where 6 < |x| < 8 units saturates
    err = np.abs(back - x)
    sat = np.abs(x) > 6 * unit
    assert np.all(err[~sat] <= unit[~sat]) and np.all(err[sat] < 2 * unit[sat])
    # the block maximum lands on 4 or 6 (times 2^(E-127)) after rounding
    bmax = np.abs(back).reshape(64, 4, 32).max(-1) / 2.0 ** (E.astype(np.float64) - 127)
    assert np.all(np.isin(bmax, [4.0, 6.0]))


def _bulk_fp8(x):
    """Reading for a whole chunk, evaluated with torch: scale = amax/448,
    codes = cast(clamp(x / scale))."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    amax = t.abs().max()
    scale = (amax / 448.0) if amax > 0 else torch.tensor(1.0)
    codes = (t / scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, np.float32(scale.item())


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def _run_policy(x, splits, policy=oq.append_fp8_chunk):
    codes = np.zeros((16, x.shape[1]), dtype=np.uint8)
    scale = np.float32(1.0)
    n = 0
    for k in splits:
        codes, scale = policy(codes, scale, n, x[n:n + k])
        n += k
    return codes, scale


def test_fp8_whole_chunk_equals_the_bulk_reading():
    rng = np.random.default_rng(2)
    for trial in range(50):
        x = _bf16(rng.normal(0, 1, (16, 128)) * 2.0 ** rng.integers(-8, 8))
        codes, scale = _run_policy(x, [16])
        rc, rs = _bulk_fp8(x)
        assert scale == rs and np.array_equal(codes, rc)
    zeros = np.zeros((16, 128), dtype=np.float32)
    codes, scale = _run_policy(zeros, [16])
    assert scale == 1.0 and not np.any(codes & 0x7F)


def test_fp8_open_chunk_invariants():
    rng = np.random.default_rng(3)
    for trial in range(200):
        x = _bf16(rng.normal(0, 1, (16, 64)) * np.exp2(rng.integers(-3, 4, (16, 1))))
        cuts = np.sort(rng.choice(np.arange(1, 16), rng.integers(0, 6), replace=False))
        splits = np.diff(np.concatenate([[0], cuts, [16]])).tolist()
        codes, scale = _run_policy(x, splits)
        # the scale is the running amax / 448 of all rows, as for the whole chunk
        assert scale == _bulk_fp8(x)[1]
        # every row decodes to its value within one rounding (half an e4m3 step: 2^-4 relative, 2^-10 * scale
        # among subnormals) per encoding it went through: at most one per append
        back = ocod.FP8_E4M3[codes].astype(np.float64) * np.float64(scale)
        tol = (np.abs(x) * 2.0 ** -4 + scale * 2.0 ** -10) * len(splits)
        assert np.all(np.abs(back - x) <= tol)
        # the rows appended last (after the final raise of the scale) are the bulk codes
        n_last = splits[-1]
        rc, _ = _bulk_fp8(x)
        if np.max(np.abs(x[16 - n_last:])) == np.max(np.abs(x)) or len(splits) == 1:
            assert np.array_equal(codes[16 - n_last:], rc[16 - n_last:])


def test_fp8_no_raise_keeps_stored_codes():
    rng = np.random.default_rng(4)
    x = _bf16(rng.normal(0, 1, (16, 128)))
    x[0, 0] = 50.0                                   # the first row holds the chunk maximum
    codes1, s1 = _run_policy(x, [1])
    codes, s = _run_policy(x, [1] * 16)
    assert s == s1 and np.array_equal(codes[:1], codes1[:1])
    assert np.array_equal(codes, _bulk_fp8(x)[0])   # nothing was ever re-encoded


def _policy_inverted_ratio(codes, scale, n_old, x_new):
    """Planted mistake: re-encodes the stored codes with new/old instead of old/new."""
    c, s = oq.append_fp8_chunk(codes, scale, n_old, x_new)
    if s != scale and n_old:
        r = np.float32(s / np.float32(scale))
        y = (ocod.FP8_E4M3[codes[:n_old]].astype(np.float32) * r).astype(np.float32)
        c[:n_old] = oq.encode_e4m3(np.clip(y, -448, 448))
    return c, s


def _policy_no_reencode(codes, scale, n_old, x_new):
    """Planted mistake: raises the scale but keeps the stored codes."""
    c, s = oq.append_fp8_chunk(codes, scale, n_old, x_new)
    c[:n_old] = np.asarray(codes, dtype=np.uint8)[:n_old]
    return c, s


def _policy_first_row_scale(codes, scale, n_old, x_new):
    """Planted mistake: the scale is fixed by the first append and never raised."""
    if n_old == 0:
        return oq.append_fp8_chunk(codes, scale, n_old, x_new)
    c = np.array(codes, dtype=np.uint8, copy=True)
    c[n_old:n_old + len(x_new)] = oq.quantize_fp8_rows(x_new, scale)
    return c, np.float32(scale)


@pytest.mark.parametrize("mutant", [_policy_inverted_ratio, _policy_no_reencode, _policy_first_row_scale])
def test_fp8_policy_mutations_are_caught(mutant):
    rng = np.random.default_rng(5)
    caught = False
    for trial in range(50):
        x = _bf16(rng.normal(0, 1, (16, 64)) * np.exp2(np.arange(16)[:, None] / 4.0))   # growing rows
        splits = [1] * 16
        codes, scale = _run_policy(x, splits, mutant)
        back = ocod.FP8_E4M3[codes].astype(np.float64) * np.float64(scale)
        tol = (np.abs(x) * 2.0 ** -4 + scale * 2.0 ** -10) * len(splits)
        ok = scale == _bulk_fp8(x)[1] and np.all(np.abs(back - x) <= tol)
        caught |= not ok
    assert caught
