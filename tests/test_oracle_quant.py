"""Pins of the oracle's quantizer against facts fixed outside the oracle itself:
hand-worked blocks, the published format tables, torch's independent E4M3
rounding, exact rational arithmetic for the tensor scale, and invariants of the
definition (QUADS explainer §1; TRACE post, "Fonctionnement, côté ingénierie")."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden
from qat_nvfp4_quantize_amd import inputs


def _golden_blocks():
    blocks = []
    for line in read_golden("nvfp4_blocks.txt"):
        name, vals, sc, packed, rsum = [f.strip() for f in line.split("|")]
        blocks.append((name, [float(v) for v in vals.split()], int(sc, 16),
                       bytes.fromhex(packed), float(rsum)))
    return blocks


def test_format_tables_match_published_values():
    for line in read_golden("format_tables.txt"):
        kind, key, val = line.split()
        if kind == "e2m1":
            assert oracle.e2m1_value(int(key)) == float(val)
        else:
            assert oracle.e4m3_value(int(key, 16)) == float(val)


def test_e4m3_table_matches_torch_decoding():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    assert np.array_equal(ref, mine)


def test_hand_worked_blocks():
    blocks = _golden_blocks()
    x = np.array([v for b in blocks for v in b[1]], np.float32).reshape(1, -1)
    codes, scales, st = oracle.quantize(x)
    assert st == 1.0  # anchor block fixes s_t = 1
    deq = oracle.dequantize(codes, scales, st)
    for i, (name, vals, sc, packed, rsum) in enumerate(blocks):
        assert scales[0, i] == sc, name
        assert bytes(codes[0, 8 * i:8 * i + 8]) == packed, name
        r = np.abs(x[0, 16 * i:16 * i + 16].astype(np.float64) - deq[0, 16 * i:16 * i + 16])
        assert r.sum() == pytest.approx(rsum, abs=0), name


def test_hand_worked_blocks_bf16_input_and_threshold_form():
    blocks = _golden_blocks()
    x = np.array([v for b in blocks for v in b[1]], np.float32).reshape(1, -1)
    xb = inputs.to_bf16_bits(x)  # every golden value is exact in bf16
    assert np.array_equal(inputs.bf16_bits_to_f32(xb), x)
    a = oracle.quantize(x)
    b = oracle.quantize(xb)
    c = oracle.quantize(x, threshold_form=True)
    for other in (b, c):
        assert np.array_equal(a[0], other[0]) and np.array_equal(a[1], other[1])
        assert a[2] == other[2]


def test_saturation_through_amax_override():
    # amax_in = 2688 gives s_t = 1; a block with amax 3000 targets 500 > 448.
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1] = 3000.0, -2700.0
    codes, scales, st = oracle.quantize(x, amax_in=2688.0)
    assert st == 1.0 and scales[0, 0] == 0x7E
    assert codes[0, 0] == (0x7 | (0xF << 4))  # both saturate to magnitude index 7


def test_tensor_scale_is_correctly_rounded_quotient():
    g = np.random.default_rng(1)
    amaxes = list(np.abs(g.standard_normal(2000).astype(np.float32) * 10.0 ** g.integers(-30, 30, 2000)).astype(np.float32))
    amaxes += [np.float32(2688.0), np.float32(1e-40), np.float32(3.4e38), np.float32(0.0)]
    for a in amaxes:
        a = np.float32(a)
        s = np.float32(oracle.tensor_scale(a))
        exact = Fraction(float(a)) / 2688
        lo = np.nextafter(s, np.float32(-np.inf), dtype=np.float32)
        hi = np.nextafter(s, np.float32(np.inf), dtype=np.float32)
        d = abs(Fraction(float(s)) - exact)
        for nb in (lo, hi):
            if np.isfinite(nb) and nb >= 0:
                dn = abs(Fraction(float(nb)) - exact)
                assert d < dn or (d == dn and (s.view(np.uint32) & 1) == 0), (a, s)


def test_e4m3_scale_rounding_matches_torch():
    # s_t = 1 (anchor 2688); block b has amax 6*q with q exact, so the target is q.
    g = np.random.default_rng(2)
    q = np.concatenate([
        g.uniform(0, 460, 3000), g.uniform(0, 0.02, 1000), g.uniform(0, 2, 1000),
    ]).astype(np.float32)
    # keep <= 21 significant bits so 6 q is exact in fp32
    q = (q.view(np.uint32) & np.uint32(0xFFFFFFF8)).view(np.float32)
    # add exact E4M3 midpoints (ties)
    mids = np.array([(oracle.e4m3_value(c) + oracle.e4m3_value(c + 1)) / 2 for c in range(126)],
                    np.float32)
    q = np.concatenate([q, mids])
    x = np.zeros((1, 16 * (len(q) + 1)), np.float32)
    x[0, 0] = 2688.0
    x[0, 16::16] = 6 * q
    assert np.array_equal(x[0, 16::16] / 6, q)
    _, scales, st = oracle.quantize(x, amax_in=2688.0)  # q up to 460 > 448: saturates
    assert st == 1.0
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales[0, 1:], ref)


def _random_tensor(seed, rows=64, K=256, dtype="f32"):
    g = np.random.default_rng(seed)
    x = (g.standard_t(3, (rows, K)) * np.exp(g.uniform(-3, 3, (rows, 1)))).astype(np.float32)
    x[g.random((rows, K)) < 0.02] = 0.0
    x[g.random((rows, K)) < 0.01] *= -0.0
    return inputs.to_bf16_bits(x) if dtype == "bf16" else x


def _near_tie_tensor(seed):
    """Values exactly on, and one ulp either side of, the E2M1 decision midpoints."""
    g = np.random.default_rng(seed)
    rows, K = 32, 128
    x = np.zeros((rows, K), np.float32)
    x[0, 0] = 2688.0  # s_t = 1
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    for r in range(rows):
        for b in range(K // 16):
            if r == 0 and b == 0:
                continue
            s_b = np.float32(oracle.e4m3_value(int(g.integers(1, 0x7F))))
            blk = np.zeros(16, np.float32)
            blk[0] = 6 * s_b
            m = mids[g.integers(0, 7, 15)] * s_b
            nudge = g.integers(-1, 2, 15)
            v = np.where(nudge < 0, np.nextafter(m, np.float32(0)),
                         np.where(nudge > 0, np.nextafter(m, np.float32(np.inf)), m))
            blk[1:] = v * np.where(g.random(15) < 0.5, -1, 1)
            x[r, 16 * b:16 * b + 16] = blk
    return x


def _e4m3_midpoints():
    """All 126 midpoints between consecutive finite non-negative E4M3 values."""
    v = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float64)
    return 0.5 * (v[:-1] + v[1:])


def _scale_tie_tensor(seed, s_t_amax=1.2345678e3):
    """A tensor scale with a full mantissa (amax = s_t_amax), block maxima at
    fl32(6 mid s_t) and one ulp either side of it for random E4M3 midpoints
    mid (so amax_b / (6 s_t) sits within an ulp or two of the midpoint), and
    other elements at fl32(m s_b s_t) -+ 1 ulp for E2M1 midpoints m under the
    scale the block will get."""
    g = np.random.default_rng(seed)
    rows, K = 32, 256
    x = np.zeros((rows, K), np.float32)
    x[0, 0] = np.float32(s_t_amax)
    s_t = np.float64(np.float32(np.float64(np.float32(s_t_amax)) / 2688.0))
    mids = _e4m3_midpoints()
    emids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for r in range(rows):
        for b in range(K // 16):
            if r == 0 and b == 0:
                continue
            mid = mids[g.integers(0, mids.size)]
            am = np.float32(6.0 * mid * s_t)
            am = [np.nextafter(am, np.float32(0)), am, np.nextafter(am, np.float32(np.inf))][g.integers(0, 3)]
            blk = np.zeros(16, np.float32)
            blk[g.integers(0, 16)] = am
            # the block scale is one of the two codes around mid; elements sit
            # near E2M1 midpoints under either
            s_b = np.float64(oracle.e4m3_value(int(np.searchsorted(mids, mid)) + int(g.integers(0, 2))))
            for j in range(16):
                if blk[j] != 0:
                    continue
                v = np.float32(emids[g.integers(0, 7)] * s_b * s_t)
                v = [np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))][g.integers(0, 3)]
                blk[j] = min(v, am) * (-1 if g.random() < 0.5 else 1)
            x[r, 16 * b:16 * b + 16] = blk
    return x


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_threshold_form_agrees_with_search(seed):
    for x in (_random_tensor(seed), _random_tensor(seed, dtype="bf16"), _near_tie_tensor(seed),
              _scale_tie_tensor(seed), _scale_tie_tensor(seed, 3.0e-3)):
        a = oracle.quantize(x)
        b = oracle.quantize(x, threshold_form=True)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def _normal_scale_mask(scales):
    # E4M3 codes 0x01..0x07 are subnormal scales; 0x00 and normal codes qualify.
    return (scales == 0) | (scales >= 0x08)


@pytest.mark.parametrize("seed", [3, 4])
def test_requantizing_dequantized_values_is_identity(seed):
    x = _random_tensor(seed)
    codes, scales, st = oracle.quantize(x)
    amax = float(np.abs(x).max())
    v = oracle.dequantize(codes, scales, st)
    c2, s2, st2 = oracle.quantize(v, amax_in=amax)
    assert st2 == st
    ok = _normal_scale_mask(scales)
    assert np.array_equal(s2[ok], scales[ok])
    okc = np.repeat(ok, 8, axis=1)
    assert np.array_equal(c2[okc], codes[okc])


def test_power_of_two_scaling_and_sign_symmetry_and_row_permutation():
    x = _random_tensor(5)
    codes, scales, st = oracle.quantize(x)
    for e in (-20, -3, 5, 40):
        c2, s2, st2 = oracle.quantize(x * np.float32(2.0 ** e))
        assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
        assert st2 == np.float32(st * 2.0 ** e)
    c3, s3, st3 = oracle.quantize(-x)
    assert st3 == st and np.array_equal(s3, scales)
    assert np.array_equal(c3, codes ^ np.uint8(0x88))
    perm = np.random.default_rng(0).permutation(x.shape[0])
    c4, s4, st4 = oracle.quantize(x[perm])
    assert st4 == st and np.array_equal(c4, codes[perm]) and np.array_equal(s4, scales[perm])


def test_all_zero_and_negative_zero_tensor():
    x = np.zeros((2, 32), np.float32)
    x[1] = -0.0
    codes, scales, st = oracle.quantize(x)
    assert st == 0.0 and not scales.any()
    assert (codes[0] == 0).all() and (codes[1] == 0x88).all()


def test_dequantize_matches_independent_decoding():
    x = _random_tensor(6)
    codes, scales, st = oracle.quantize(x)
    g = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # published E2M1 table
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    sb = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sb = np.repeat(sb, 16, axis=1)
    mag = (g[nib & 7] * sb * np.float64(st)).astype(np.float32)
    ref = np.where(nib & 8, -mag, mag)
    got = oracle.dequantize(codes, scales, st)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    gotb = oracle.dequantize(codes, scales, st, out="bf16")
    refb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gotb, refb)


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(7)
    x = (g.standard_normal(100000) * 10.0 ** g.integers(-20, 20, 100000)).astype(np.float32)
    x[:100] = (np.arange(100, dtype=np.uint32) << 16 | 0x8000).view(np.float32)  # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.to_bf16_bits(x), ref)
