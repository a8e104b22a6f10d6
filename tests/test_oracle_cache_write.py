"""Pins of the oracle's cache write path: rotary embedding, bf16 / e4m3 storage, cache append.

Rotary embedding: page "一文讀懂DeepSeek-V3.2核心技術DSA", "DSA 的四步工作流程", first step (the
projections carry rotary position information); page "DeepSeek 稀疏注意力路线", "DeepSeek-V3：MLA
基座", "核心机制（直觉）" (MLA's decoupled position channel).  The pages give no formula; the oracle
uses the standard rotation of pair i by position * base^(-2i/d).  fp8: e4m3fn with one scale per
128-wide row.

Every pin is independent of the oracle's code: round trips over every code, constructed ties,
torch's own casts, the complex-exponential form of the rotation, RoPE's relative-position property,
the mapping between the interleaved and split pair layouts, and an append followed by the already
pinned indexer.  A plausible slip (sin sign, pair layout, angle exponent, scale placement, a
dropped saturation, a wrong page lookup) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle


# ------------------------------------------------------------------------------ number formats

def test_e4m3_encode_round_trips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], dtype=np.uint8)   # all but NaN
    vals = oracle.decode(codes, "fp8")
    vals[codes == 0x80] = -0.0
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_encode_ties_go_to_even_code_and_saturate():
    codes = np.arange(0, 0x7e, dtype=np.uint8)                 # consecutive positive codes c, c+1
    lo = oracle.decode(codes, "fp8"); hi = oracle.decode(codes + 1, "fp8")
    mid = (lo + hi) / 2
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(oracle.e4m3_encode(mid), even)
    assert np.array_equal(oracle.e4m3_encode(-mid), even | 0x80)
    # just off the midpoint the nearer code wins
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mid, -np.inf)), codes)
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mid, np.inf)), codes + 1)
    assert oracle.e4m3_encode(np.array([1e6, -1e6, 449.0, 464.0, 479.0])).tolist() == [0x7e, 0xfe, 0x7e, 0x7e, 0x7e]


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.normal(0, 60, 4000), rng.normal(0, 0.01, 2000), rng.uniform(-448, 448, 2000)])
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


def test_bf16_encode_matches_torch_cast_and_ties():
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.normal(0, 1, 5000), rng.normal(0, 1e-30, 500), rng.normal(0, 1e30, 500)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_encode(x), ref)
    # exact midpoints between consecutive bf16 codes: ties to the even code
    codes = np.arange(0x3f80, 0x3f90, dtype=np.uint16)
    mid = ((codes.astype(np.uint32) << 16) | 0x8000).view(np.float32)
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint16)
    assert np.array_equal(oracle.bf16_encode(mid), even)


# ------------------------------------------------------------------------------ rotary embedding

def _complex_rope(x, pos, off, d, inter, base):
    """The rotation written as a complex product: pair (a, b) as a + ib times exp(i p theta_i)."""
    x = x.astype(np.float64).copy()
    i = np.arange(d // 2)
    a = off + (2 * i if inter else i)
    b = off + (2 * i + 1 if inter else i + d // 2)
    z = x[:, a] + 1j * x[:, b]
    z = z * np.exp(1j * np.outer(pos.astype(np.float64), base ** (-2.0 * i / d)))
    x[:, a] = z.real
    x[:, b] = z.imag
    return x


@pytest.mark.parametrize("inter", [1, 0])
def test_rope_matches_complex_product(inter):
    rng = np.random.default_rng(13)
    x = rng.normal(0, 1, (64, 128)).astype(np.float32)
    pos = rng.integers(0, 131072, 64).astype(np.int32)
    got = oracle.rope_rows(x, "f32", pos, (32, 64, inter, 10000.0))
    ref = _complex_rope(x, pos, 32, 64, inter, 10000.0)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6)
    # dims outside the span untouched, bit for bit
    assert np.array_equal(got[:, :32], x[:, :32]) and np.array_equal(got[:, 96:], x[:, 96:])


def test_rope_position_zero_is_identity_and_first_pair_turns_by_position():
    rng = np.random.default_rng(14)
    x = rng.normal(0, 1, (8, 64)).astype(np.float32)
    assert np.array_equal(oracle.rope_rows(x, "f32", np.zeros(8, np.int32), (0, 64, 1, 10000.0)), x)
    pos = np.arange(1, 9, dtype=np.int32) * 1000
    got = oracle.rope_rows(x, "f32", pos, (0, 64, 1, 10000.0))
    c, s = np.cos(pos), np.sin(pos)                       # theta_0 = base^0 = 1
    np.testing.assert_allclose(got[:, 0], x[:, 0] * c - x[:, 1] * s, atol=1e-6)
    np.testing.assert_allclose(got[:, 1], x[:, 0] * s + x[:, 1] * c, atol=1e-6)


def test_rope_quarter_turn():
    """base = 4/pi^2, width 4, split pairs: pair 1 turns by (pi^2/4)^(1/2) = pi/2 per position,
    so at position 1 (x1, x3) -> (-x3, x1) and at position 2 -> (-x1, -x3)."""
    x = np.array([[0.0, 3.0, 0.0, 5.0]], np.float32)
    base = 4.0 / math.pi ** 2
    one = oracle.rope_rows(x, "f32", np.array([1], np.int32), (0, 4, 0, base))
    two = oracle.rope_rows(x, "f32", np.array([2], np.int32), (0, 4, 0, base))
    np.testing.assert_allclose(one[0, [1, 3]], [-5.0, 3.0], atol=1e-6)
    np.testing.assert_allclose(two[0, [1, 3]], [-3.0, -5.0], atol=1e-6)


def test_rope_relative_position_and_norm():
    """<R(m) q, R(n) k> depends only on m - n, and every pair keeps its length."""
    rng = np.random.default_rng(15)
    q = rng.normal(0, 1, (1, 64)).astype(np.float32)
    k = rng.normal(0, 1, (1, 64)).astype(np.float32)
    rope = (0, 64, 1, 10000.0)
    dots = []
    for m, n in [(7, 3), (107, 103), (5004, 5000), (4, 0)]:
        a = oracle.rope_rows(q, "f32", np.array([m], np.int32), rope).astype(np.float64)
        b = oracle.rope_rows(k, "f32", np.array([n], np.int32), rope).astype(np.float64)
        dots.append(float((a @ b.T)[0, 0]))
    np.testing.assert_allclose(dots, dots[0], rtol=0, atol=2e-5)
    r = oracle.rope_rows(q, "f32", np.array([12345], np.int32), rope).astype(np.float64)
    np.testing.assert_allclose(np.hypot(r[0, 0::2], r[0, 1::2]), np.hypot(q[0, 0::2], q[0, 1::2]), rtol=1e-6)


def test_rope_split_layout_is_interleaved_layout_of_permuted_row():
    rng = np.random.default_rng(16)
    x = rng.normal(0, 1, (16, 64)).astype(np.float32)
    pos = rng.integers(0, 70000, 16).astype(np.int32)
    perm = np.ravel(np.column_stack([np.arange(32), np.arange(32) + 32]))   # split pair i -> slots 2i, 2i+1
    split = oracle.rope_rows(x, "f32", pos, (0, 64, 0, 10000.0))
    inter = oracle.rope_rows(x[:, perm], "f32", pos, (0, 64, 1, 10000.0))
    assert np.array_equal(split[:, perm], inter)


def test_rope_store_bf16_is_rounding_of_rope_rows():
    rng = np.random.default_rng(17)
    x = rng.normal(0, 1, (4, 3, 576)).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pos = np.array([0, 9, 70000, 131071], np.int32)
    rope = (512, 64, 1, 10000.0)
    out, scale = oracle.rope_store(bits, "bf16", pos, rope, "bf16")
    assert scale is None
    rot = oracle.rope_rows(bits.reshape(12, 576), "bf16", np.repeat(pos, 3), rope)
    ref = torch.from_numpy(rot).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out.reshape(12, 576), ref)
    assert np.array_equal(out[..., :512], bits[..., :512])     # unrotated dims copied exactly


def test_fp8_row_quantisation():
    """Per-row scale = amax / 448: the largest element becomes +-448, every element is recovered
    within half a code step, and an all-zero row stays zero."""
    rng = np.random.default_rng(18)
    x = rng.normal(0, 3, (5, 2, 128)).astype(np.float32)
    x[4, 1] = 0.0
    out, scale = oracle.rope_store(x, "f32", np.zeros(5, np.int32), None, "fp8")
    dec = oracle.decode(out, "fp8")
    for t in range(5):
        for h in range(2):
            row = x[t, h].astype(np.float64)
            amax = np.abs(row).max()
            if amax == 0:
                assert np.all(dec[t, h] == 0) and scale[t, h] == np.float32(1e-12) / np.float32(448)
                continue
            assert scale[t, h] == np.float32(np.float32(amax) / np.float32(448))
            j = np.abs(row).argmax()
            assert abs(dec[t, h, j]) == 448.0
            rec = dec[t, h] * scale[t, h]
            step = np.maximum(np.abs(row) * 2.0 ** -4, 2.0 ** -10 * scale[t, h])   # half an e4m3 step
            assert np.all(np.abs(rec - row) <= step * 1.0001)


# ------------------------------------------------------------------------------ cache append

def test_paged_append_equals_contiguous_append_and_skips_bad_tokens():
    rng = np.random.default_rng(19)
    B, S, W, ps = 3, 256, 128, 64
    T = 200
    seq = rng.integers(0, B, T).astype(np.int32)
    pos = rng.integers(0, S, T).astype(np.int32)
    _, first = np.unique(np.stack([seq, pos], 1), axis=0, return_index=True)   # distinct (seq, pos)
    seq, pos = seq[np.sort(first)], pos[np.sort(first)]
    T = len(seq)
    x = rng.normal(0, 1, (T, W)).astype(np.float32)
    rope = (0, 64, 0, 10000.0)
    contig = np.zeros((B * S, W), np.uint8); cs = np.zeros(B * S, np.float32)
    oracle.cache_append(x, "f32", seq, pos, B, rope, contig, "fp8", cs, seq_stride=S)
    pt = rng.permutation(B * S // ps).astype(np.int32).reshape(B, S // ps)
    paged = np.zeros((B * S, W), np.uint8); pscale = np.zeros(B * S, np.float32)
    oracle.cache_append(x, "f32", seq, pos, B, rope, paged, "fp8", pscale, page_table=pt, page_size=ps)
    logical = (pt[:, :, None] * ps + np.arange(ps)).reshape(B, S)             # row of (b, s)
    assert np.array_equal(paged[logical.ravel()], contig) and np.array_equal(pscale[logical.ravel()], cs)
    written = np.zeros(B * S, bool); written[seq * S + pos] = True
    assert np.all(contig[~written] == 0) and np.all(cs[~written] == 0)
    # bad tokens: sequence out of range, negative position, position past the rows, page -1
    pt2 = pt.copy(); pt2[1, 2] = -1
    bad_seq = np.array([B, -1, 0, 0, 1], np.int32)
    bad_pos = np.array([0, 0, -5, S, 2 * ps + 3], np.int32)
    before = paged.copy()
    oracle.cache_append(rng.normal(0, 1, (5, W)).astype(np.float32), "f32", bad_seq, bad_pos, B, rope, paged, "fp8",
                        pscale, page_table=pt2, page_size=ps)
    assert np.array_equal(paged, before)


def test_append_then_indexer_equals_indexer_on_the_rows():
    """Keys appended without rotation into an f32 cache score exactly like the same keys placed
    directly: the append puts token (b, s) where the (pinned) indexer looks for it."""
    rng = np.random.default_rng(20)
    B, S, W = 2, 128, 128
    keys = rng.normal(0, 1, (B, S, W)).astype(np.float32)
    order = rng.permutation(B * S)
    seq = (order // S).astype(np.int32); pos = (order % S).astype(np.int32)
    pt = rng.permutation(B * S // 64).astype(np.int32).reshape(B, S // 64)
    cache = np.zeros((B * S, W), np.float32)
    oracle.cache_append(keys[seq, pos], "f32", seq, pos, B, None, cache, "f32", page_table=pt, page_size=64)
    q = rng.normal(0, 1, (2, 4, W)).astype(np.float32)
    w = rng.uniform(0, 1, (2, 4)).astype(np.float32)
    q_seq = np.array([0, 1], np.int32); q_len = np.array([S, 77], np.int32)
    got = oracle.indexer(q, "f32", None, w, cache, "f32", None, q_seq, q_len, page_table=pt, page_size=64)
    ref = oracle.indexer(q, "f32", None, w, keys.reshape(B * S, W), "f32", None, q_seq, q_len, seq_stride=S)
    assert np.array_equal(got, ref)
