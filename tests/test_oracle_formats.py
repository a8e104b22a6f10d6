"""Pins of the oracle's number decoders: against the format definitions (golden points) and
against torch's independent CPU casts over every bit pattern."""
import os

import numpy as np
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _points(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 16), float(val)))
    return rows


def _same(a, b):
    if np.isnan(b):
        return np.isnan(a)
    return a == b and np.signbit(a) == np.signbit(b)


def test_e4m3_golden_points():
    pts = _points("e4m3fn_points.txt")
    raw = np.array([c for c, _ in pts], dtype=np.uint8)
    got = oracle.decode(raw, "fp8")
    for (code, want), g in zip(pts, got):
        assert _same(g, want), (hex(code), g, want)


def test_bf16_golden_points():
    pts = _points("bf16_points.txt")
    raw = np.array([c for c, _ in pts], dtype=np.uint16)
    got = oracle.decode(raw, "bf16")
    for (code, want), g in zip(pts, got):
        assert _same(g, want), (hex(code), g, want)


def test_e4m3_all_codes_match_torch():
    raw = np.arange(256, dtype=np.uint8)
    got = oracle.decode(raw, "fp8")
    ref = torch.from_numpy(raw).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for g, r in zip(got, ref):
        assert _same(g, r)


def test_bf16_all_codes_match_torch():
    raw = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(raw, "bf16")
    ref = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f32_passthrough():
    x = np.array([0.0, -0.0, 1.5, -2.25e-30, 3.4e38], dtype=np.float32)
    got = oracle.decode(x, "f32")
    assert np.array_equal(got, x.astype(np.float64))
