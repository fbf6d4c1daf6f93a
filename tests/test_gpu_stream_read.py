"""uno_stream_read (the measurement helper behind bench.py's stream-floor leg): every
16-byte word of the range is read once, by thread (word mod T) of a grid of T
threads, so each workgroup's xor of its words matches the host's; windows rotate
through the region; bad arguments are refused."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import uno
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wg,threads,loads,nwords", [(3, 64, 1, 1000), (7, 192, 2, 4099),
                                                     (16, 256, 4, 65536), (5, 1024, 8, 70001)])
def test_stream_read_covers_every_word(wg, threads, loads, nwords):
    import torch
    log(f"stream_read {wg} x {threads}, {loads} loads, {nwords} words")
    r = np.random.default_rng(nwords)
    data = r.integers(-2**31, 2**31 - 1, size=(nwords + 3, 4), dtype=np.int64).astype(np.int32)
    src = dev(data.ravel())
    sink = torch.full((wg,), 12345, dtype=torch.int32, device="cuda")
    uno.stream_read(src, nwords * 16, wg, threads, loads, sink, reps=3)  # windows 0, 0, 0
    word = np.bitwise_xor.reduce(data[:nwords], axis=1)
    owner = (np.arange(nwords) % (wg * threads)) // threads
    want = np.zeros(wg, dtype=np.int32)
    for b in range(wg):
        want[b] = np.bitwise_xor.reduce(word[owner == b]) if np.any(owner == b) else 0
    assert np.array_equal(host(sink), want)


def test_stream_read_rotates_windows():
    import torch
    nb, nwin = 4096, 3
    data = (np.arange(nwin * nb // 4 + 8, dtype=np.int64) * 2654435761 % (2**31 - 1)).astype(np.int32)
    src = dev(data)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    words = np.bitwise_xor.reduce(data[: nwin * nb // 4].reshape(nwin, nb // 16, 4), axis=2)
    for reps in (1, 2, 3, 4, 5):           # the last launch reads window (reps - 1) mod 3
        uno.stream_read(src[: nwin * nb // 4], nb, 1, 64, 2, sink, reps=reps)
        assert host(sink)[0] == np.bitwise_xor.reduce(words[(reps - 1) % nwin])


def test_stream_read_refuses_bad_arguments():
    import torch
    src = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for args in ((1000, 4, 64, 1), (1024, 4, 96, 1), (1024, 4, 64, 3), (1024, 4, 2048, 1)):
        with pytest.raises(uno.UnoError):
            uno.stream_read(src, args[0], args[1], args[2], args[3], sink)
    with pytest.raises(uno.UnoError):
        uno.stream_read(src, 1024, 4, 64, 1, sink, reps=0)
