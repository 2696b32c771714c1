"""Pins for the oracle's codecs (OCP E4M3FN and bf16), against things other
than the oracle itself: torch's float8_e4m3fn / bfloat16 conversions, values
the format definition fixes, and an independent bitwise encoder run over every
binary32 input."""
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _torch_e4m3_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def test_e4m3_decode_all_codes_match_torch():
    ours = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_e4m3_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    # sign of zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3_decode_format_anchors():
    # OCP 8-bit FP spec, E4M3: max normal S.1111.110 = 448, min normal 2^-6,
    # min subnormal 2^-9, max subnormal 0.875 * 2^-6, one = S.0111.000.
    d = oracle.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x07, 0x38, 0xB8, 0xFE], dtype=np.uint8))
    assert d.tolist() == [448.0, 2.0 ** -6, 2.0 ** -9, 0.875 * 2.0 ** -6, 1.0, -1.0, -448.0]


def test_bf16_decode_all_codes_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _encode_with_torch(x: np.ndarray) -> np.ndarray:
    """torch's float8_e4m3fn rounding (RNE) after saturating to +-448; torch
    itself turns out-of-range values into NaN, so saturation is applied first."""
    t = torch.from_numpy(x.astype(np.float32))
    t = torch.where(torch.isnan(t), t, t.clamp(-448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_on_ties_and_neighbours():
    vals = np.concatenate([[0.0], _torch_e4m3_values()[:0x7F]])
    vals = np.unique(vals[np.isfinite(vals)])
    mids = (vals[:-1] + vals[1:]) / 2  # exact in float32: ties
    cand = np.concatenate([vals, mids, [448.0, 464.0, 500.0, 1e30, np.inf]]).astype(np.float32)
    # one ulp either side of every candidate
    up = np.nextafter(cand, np.float32(np.inf))
    dn = np.nextafter(cand, np.float32(-np.inf))
    x = np.concatenate([cand, up, dn])
    x = np.concatenate([x, -x]).astype(np.float32)
    ours = oracle.e4m3_encode(x)
    assert np.array_equal(ours, _encode_with_torch(x))


def test_e4m3_encode_matches_torch_on_random_and_all_bf16():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(2_000_000) * np.exp(rng.uniform(-12, 7, 2_000_000))).astype(np.float32)
    bf16 = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    bf16 = bf16[~np.isnan(bf16)]
    x = np.concatenate([x, bf16])
    assert np.array_equal(oracle.e4m3_encode(x), _encode_with_torch(x))


def test_e4m3_encode_special_values():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 448.0, 449.0, 1e9, -1e9],
                 dtype=np.float32)
    out = oracle.e4m3_encode(x).tolist()
    assert out[0] & 0x7F == 0x7F and out[1] & 0x7F == 0x7F       # NaN stays NaN
    assert out[2:] == [0x7E, 0xFE, 0x00, 0x80, 0x7E, 0x7E, 0x7E, 0xFE]


@pytest.mark.slow
def test_e4m3_encode_exhaustive_against_bitwise_encoder():
    lib = oracle_build.ensure_built()
    src = os.path.join(ROOT, "tests", "c", "e4m3_exhaustive.c")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "e4m3_exhaustive")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-o", exe, src, lib,
                        "-Wl,-rpath," + os.path.dirname(lib)], check=True)
        res = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().splitlines()[-1] == "0"
