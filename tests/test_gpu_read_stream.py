"""The read-stream reference kernel (gdn_read_stream) reads every word exactly once: its
per-workgroup XOR folds equal the same folds computed on the host from the documented
mapping (workgroup b reads the 32 KiB from byte 32768 b on), bit for bit, on a ragged size
and at a whole number of 32 KiB workgroups; and a single non-zero word lands in the one
workgroup that owns it."""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_decode_amd import abi
from tests.gpu_util import note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PER = 256 * 8  # 16-byte words per workgroup: 256 threads x 8 loads


def _expected(buf: np.ndarray) -> np.ndarray:
    """Workgroup b folds the 32-bit words of the 32 KiB from byte 32768 b on that exist."""
    w = buf.view(np.uint32)
    g = (len(w) // 4 + PER - 1) // PER
    padded = np.zeros(g * PER * 4, np.uint32)
    padded[:len(w)] = w
    return np.bitwise_xor.reduce(padded.reshape(g, PER * 4), axis=1)


def _run(buf: np.ndarray) -> np.ndarray:
    g = (buf.nbytes // 16 + PER - 1) // PER
    src = torch.from_numpy(buf.copy()).to(DEV)
    sink = torch.full((g + 4,), -1, dtype=torch.int32, device=DEV)  # 4 guard words past the end
    abi.gdn_read_stream(src.data_ptr(), buf.nbytes, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = sink.cpu().numpy().view(np.uint32)
    assert np.all(out[g:] == 0xFFFFFFFF), "a word past the sink was written"
    return out[:g]


@pytest.mark.parametrize("nbytes", [16, 16 * 123457, 32768 * 40])
def test_read_stream_folds_every_word_once(nbytes):
    note(f"read stream: {nbytes} bytes")
    rng = np.random.Generator(np.random.PCG64(nbytes))
    buf = rng.integers(0, 256, nbytes, dtype=np.uint8)
    got = _run(buf)
    np.testing.assert_array_equal(got, _expected(buf))
    total = np.bitwise_xor.reduce(buf.view(np.uint32))
    assert np.bitwise_xor.reduce(got) == total


def test_read_stream_one_word():
    nbytes = 16 * 100003
    for pos in (0, nbytes // 4 - 1, 12345):
        note(f"read stream: one non-zero word at {pos}")
        buf = np.zeros(nbytes, np.uint8)
        buf.view(np.uint32)[pos] = 0x9E3779B9
        got = _run(buf)
        exp = _expected(buf)
        np.testing.assert_array_equal(got, exp)
        assert np.count_nonzero(got) == 1 and got[np.flatnonzero(got)[0]] == 0x9E3779B9
