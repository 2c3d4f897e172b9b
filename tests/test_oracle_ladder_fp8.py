"""Pins for the oracle's ladder and element decoding (CPU only)."""
import numpy as np
import pytest
import torch

import oracle


def test_ladder_closed_form_and_steps():
    # [PR3] MSA verify commit: token t attends kv_len - qo_len + t + 1 positions.
    for kv in (1, 2, 7, 127, 128, 129, 300, 517, 4096):
        for qo in range(1, min(kv, 8) + 1):
            b = oracle.ladder_bounds(kv, qo)
            assert len(b) == qo
            assert b[-1] == kv                      # the last verify token sees everything
            assert b[0] == kv - qo + 1
            assert np.all(np.diff(b) == 1)          # one more position per token


def test_ladder_qo1_is_decode():
    # At qo_len = 1 the ladder is ordinary decode: the single token sees all kv_len.
    for kv in (1, 5, 300, 131072):
        assert list(oracle.ladder_bounds(kv, 1)) == [kv]


def test_ladder_rejects_bad_lengths():
    with pytest.raises(ValueError):
        oracle.ladder_bounds(3, 4)
    with pytest.raises(ValueError):
        oracle.ladder_bounds(3, 0)


def test_n_valid_pages_brute_force():
    # Number of 128-token pages holding at least one attended position.
    for bound in range(1, 700):
        brute = sum(1 for p in range(10) if 128 * p < bound)
        assert oracle.n_valid_pages(bound) == brute
        brute32 = sum(1 for p in range(40) if 32 * p < bound)
        assert oracle.n_valid_pages(bound, 32) == brute32


def test_e4m3fn_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                                  # 0x7F and 0xFF only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[~nan].max() == 448.0                       # largest finite value
    assert ours[1] == 2.0 ** -9                            # smallest subnormal


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
