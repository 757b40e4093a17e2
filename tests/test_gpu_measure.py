"""The measurement helpers on the GPU: the plain read reads every byte, and
every hand-off mode gives the merge's exact sums (in split order, the same
bits in all three modes) on two calls in a row."""
import numpy as np
import pytest
import torch

from decode_kv_amd import csa2
from test_gpu_parity import DEV

pytestmark = pytest.mark.gpu


def test_stream_read_covers_every_byte():
    x = torch.randint(0, 1 << 30, ((3 << 20) // 4,), dtype=torch.int32, device=DEV)
    nbytes = x.numel() * 4
    sink = torch.zeros(csa2.stream_read_sink_words(nbytes), dtype=torch.int32, device=DEV)
    csa2.stream_read(x, sink)
    torch.cuda.synchronize()
    assert int(sink.ne(0).sum()) > 0


@pytest.mark.parametrize("groups,splits", [(4, 20), (8, 16), (3, 7)])
def test_handoff_modes_agree(groups, splits):
    scratch = torch.zeros(csa2.handoff_scratch_bytes(groups, splits), dtype=torch.uint8, device=DEV)
    ref = None
    for value in (1.0, 3.5):
        want = np.zeros((groups, 8192), np.float32)
        i = np.arange(8192, dtype=np.float32)
        for s in range(splits):                      # the merge adds the splits in order
            want += (np.float32(value) + np.float32(s) + i * np.float32(1e-6)).astype(np.float32)
        for mode in (0, 1, 2):
            out = torch.full((groups, 8192), float("nan"), dtype=torch.float32, device=DEV)
            csa2.handoff(mode, groups, splits, value, scratch, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            np.testing.assert_allclose(got, want, rtol=1e-6)
            if mode == 0:
                ref = got
            else:
                assert np.array_equal(got, ref), mode
    tail = scratch[-8 * groups:].cpu().numpy()       # the counters end at zero
    assert (tail == 0).all()
