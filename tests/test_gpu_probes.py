"""The measurement helpers read what they are given: the XOR fold of the streaming-read
probes equals the XOR of every 32-bit word of the bytes they should read (whole buffer,
or a list of units with out-of-range entries skipped)."""
import functools

import numpy as np
import pytest
import torch

import speculative_decode_verify_p128_amd as sdv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _fold(words: np.ndarray) -> int:
    return int(functools.reduce(np.bitwise_xor, words.astype(np.uint32).ravel(), np.uint32(0)))


def test_read_probe_folds_every_word():
    print("\n[gpu] read_probe fold", flush=True)
    rng = np.random.default_rng(5)
    host = rng.integers(0, 2**32, size=(1 << 18) + 36, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.zeros(64, dtype=torch.int32, device=DEV)
    sdv.read_probe(buf, sink, 64)
    torch.cuda.synchronize()
    assert _fold(sink.cpu().numpy().view(np.uint32)) == _fold(host)


@pytest.mark.parametrize("unit_bytes", [4096, 8192, 16384])
def test_read_units_probe_folds_listed_units(unit_bytes):
    print(f"\n[gpu] read_units_probe fold {unit_bytes}", flush=True)
    rng = np.random.default_rng(unit_bytes)
    n_units_buf = 40
    host = rng.integers(0, 2**32, size=n_units_buf * unit_bytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    units = rng.integers(0, n_units_buf, size=23).astype(np.int64)
    units = np.concatenate([units, [n_units_buf, -1, n_units_buf + 7]])   # skipped
    sink = torch.zeros(8, dtype=torch.int32, device=DEV)
    sdv.read_units_probe(buf, torch.from_numpy(units).to(DEV), unit_bytes, sink, 8)
    torch.cuda.synchronize()
    per = unit_bytes // 4
    want = 0
    for u in units:
        if 0 <= u < n_units_buf:
            want ^= _fold(host[u * per:(u + 1) * per])
    assert _fold(sink.cpu().numpy().view(np.uint32)) == want
