"""The one-direction ceiling kernels: a2av_device_fill writes exactly its
pattern over exactly its range, and a2av_device_read loads every 16-byte
vector once (the XOR of its sink words equals the fold of the source computed
on the host). Both at sizes that take each launch shape (8 KiB pieces, and
4 KiB pieces with the occupancy cap from 64 MiB)."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from gpu_util import GuardedBuffer

pytestmark = pytest.mark.gpu

SIZES = [16, 4096 + 16, (1 << 20) + 48, (64 << 20) + 16, 256 << 20]


def _say(*a):
    print(*a, flush=True)


def host_fold(buf: np.ndarray) -> int:
    """((x ^ z) << 32) | (y ^ w) for the XOR (x, y, z, w) of every 16-byte
    vector of buf, read as four little-endian 32-bit words."""
    v = buf.view(np.uint32).reshape(-1, 4)
    x, y, z, w = (int(np.bitwise_xor.reduce(v[:, i])) for i in range(4))
    return ((x ^ z) << 32) | (y ^ w)


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("nt", [True, False], ids=["nt", "temporal"])
def test_fill_writes_its_pattern_and_nothing_else(nbytes, nt):
    _say("fill", nbytes, nt)
    b = GuardedBuffer(nbytes)
    B.a2av_device_fill(b.view, nbytes, 0x3C5A7E81, nontemporal=nt)
    torch.cuda.synchronize()
    assert b.guards_intact()
    want = int(np.array([0x3C5A7E81], dtype=np.uint32).view(np.int32)[0])
    assert bool((b.view.view(torch.int32) == want).all())


@pytest.mark.parametrize("nbytes", SIZES)
def test_read_loads_every_vector(nbytes):
    _say("read", nbytes)
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes % 1000003)
    src = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(B.SINK_WORDS, dtype=torch.int64, device="cuda")
    B.a2av_device_read(src, nbytes, sink)
    torch.cuda.synchronize()
    got = 0
    for word in sink.cpu().numpy().view(np.uint64):
        got ^= int(word)
    assert got == host_fold(src.cpu().numpy())


def test_bad_sizes_are_refused():
    t = torch.zeros(64, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(B.SINK_WORDS, dtype=torch.int64, device="cuda")
    for fn in (lambda: B.a2av_device_read(t, 24, sink),
               lambda: B.a2av_device_read(t[4:], 16, sink),
               lambda: B.a2av_device_fill(t, 8, 1),
               lambda: B.a2av_device_fill(t[8:], 16, 1)):
        with pytest.raises(B.A2avError) as e:
            fn()
        assert e.value.code == B.EARG
