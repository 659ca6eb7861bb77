"""Zero-run decoding of fp16 activations on the device (page
"Openai/692db884-... (section 28)", zero-run encoding of ReLU outputs): the
expanded tensor equals the encoder's input bit for bit and the oracle's
decode of the same stream; inconsistent blocks fail alone and write nothing.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_dequantization_amd as lt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def host_u16(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()


def status_tensor(n):
    return torch.full((max(n, 1),), -1, dtype=torch.int32, device=DEV)


def test_relu_4096x14336_activation_round_trip():
    """The 4096x14336 ReLU activation workload (about 90% zeros, with
    random-byte and 0xAB stress chunks): bit-exact against the input and the
    oracle's decode."""
    a = synth.relu_4096x14336()
    x = a.data.view(np.uint16)
    bitmap, val_off, vals = lt.encode_zero_runs(x)
    z = lt.ZeroRunTensor.from_host(bitmap, val_off, vals, x.size, DEV)
    st = status_tensor(val_off.size - 1)
    out = lt.decode_zero_runs(z, status=st)
    got = host_u16(out)
    assert np.all(st.cpu().numpy()[:val_off.size - 1] == 0)
    assert np.array_equal(got, x)
    ref, rst = O.zr_decode(bitmap, val_off, vals, x.size)
    assert np.all(rst == 0) and np.array_equal(got, ref)


@pytest.mark.parametrize("n", [1, 7, 8, 31, 511, 512, 513, 1023, 1024, 1025, 4097, 100001])
def test_lengths_and_guards(n):
    """Every length near the block and half-block sizes, with -0.0 and
    subnormals among the values; nothing written past n."""
    rng = np.random.default_rng(n)
    x = np.maximum(0, rng.standard_normal(n) - 1.0).astype(np.float16).view(np.uint16).copy()
    x[rng.integers(0, n, max(1, n // 50))] = 0x8000
    x[rng.integers(0, n, max(1, n // 50))] = 0x0001
    z = lt.ZeroRunTensor.build(x, DEV)
    guard = 64
    buf = torch.full((n + 2 * guard,), 0x5A5A, dtype=torch.int16, device=DEV)
    out = buf[guard:guard + n].view(torch.float16)
    lt.decode_zero_runs(z, out=out)
    b = host_u16(buf)
    assert np.all(b[:guard] == 0x5A5A) and np.all(b[guard + n:] == 0x5A5A)
    assert np.array_equal(b[guard:guard + n], x)


@pytest.mark.parametrize("shift", [1, 3, 7])
def test_unaligned_values(shift):
    """The values array starting 2, 6 or 14 bytes past a 16-byte boundary."""
    rng = np.random.default_rng(40 + shift)
    x = np.maximum(0, rng.standard_normal(50000) - 1.3).astype(np.float16).view(np.uint16)
    bitmap, val_off, vals = lt.encode_zero_runs(x)
    store = torch.zeros(vals.size + 16, dtype=torch.int16, device=DEV)
    store[shift:shift + vals.size] = torch.from_numpy(vals.view(np.int16)).to(DEV)
    z = lt.ZeroRunTensor.from_host(bitmap, val_off, vals, x.size, DEV)
    z.vals = store[shift:shift + vals.size]
    assert np.array_equal(host_u16(lt.decode_zero_runs(z)), x)


def test_inconsistent_blocks_fail_alone():
    """A bitmap bit flipped, a val_off entry moved, and a bit set past the
    end: the statuses equal the oracle's, failed blocks keep the buffer's
    previous contents, and every other block decodes."""
    rng = np.random.default_rng(9)
    n = 10 * 1024 + 300
    x = np.maximum(0, rng.standard_normal(n) - 1.0).astype(np.float16).view(np.uint16)
    bitmap, val_off, vals = lt.encode_zero_runs(x)
    bitmap = bitmap.copy()
    val_off = val_off.copy()
    bitmap[32 * 2 + 5] ^= 1 << 9                 # block 2
    val_off[6] += np.uint64(3)                   # blocks 5 and 6
    bitmap[32 * 10 + 31] |= 1 << 31              # block 10: element 11263 >= n
    z = lt.ZeroRunTensor.from_host(bitmap, val_off, vals, n, DEV)
    out = torch.full((n,), 0x7777, dtype=torch.int16, device=DEV)
    st = status_tensor(11)
    lt.decode_zero_runs(z, out=out.view(torch.float16), status=st)
    got = host_u16(out)
    s = st.cpu().numpy()[:11]
    ref = np.full(n, 0x7777, np.uint16)
    ref, rst = O.zr_decode(bitmap, val_off, vals, n, ref)
    assert np.array_equal(s, rst), (s, rst)
    assert sorted(np.nonzero(s)[0].tolist()) == [2, 5, 6, 10]
    assert np.array_equal(got, ref)
