"""GPU checks of the measurement helpers (not part of the attention path):
the MFMA loop computes what it claims (exact sums on operands of ones and
zeros), and the streaming read launches over a buffer that is not a
multiple of its chunk size."""

import pytest

pytestmark = pytest.mark.gpu


def _rswa():
    from kv_cache_management_amd import rswa

    rswa.load()
    return rswa


@pytest.mark.parametrize("value,iters", [(1.0, 3), (0.0, 5), (2.0, 1)])
def test_measure_mfma_exact_on_constant_operands(value, iters):
    """Every 32x32x16 product of constant operands v adds 16 v^2 to each of
    its 16 accumulators per lane; four chains, summed over the 64 lanes of
    the block's first wave: 65536 v^2 iters, exact in fp32."""
    import torch

    R = _rswa()
    ops = torch.full((R.RSWA_MEASURE_MFMA_FRAGMENTS, 8), value, device="cuda", dtype=torch.bfloat16)
    sink = torch.full((512,), float("nan"), device="cuda", dtype=torch.float32)
    st = R.rswa_measure_mfma(ops.data_ptr(), iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, R.load().rswa_status_string(st)
    torch.cuda.synchronize()
    want = 65536.0 * value * value * iters
    assert torch.all(sink == want), (sink[:4].tolist(), want)


@pytest.mark.parametrize("nbytes", [(3 << 20) + 48, 16, (64 << 20) + 8192 * 3 + 16])
def test_measure_read_reads_every_byte_once(nbytes):
    """The sink words (one wrapping 32-bit sum per wavefront, untouched words
    left at zero) sum to the buffer's 32-bit word sum: every byte of a
    buffer whose size is no multiple of the 8 KB slab is read exactly once."""
    import numpy as np
    import torch

    R = _rswa()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).to("cuda")
    sink = torch.zeros(R.RSWA_MEASURE_SINK_WORDS, device="cuda", dtype=torch.int32)
    st = R.rswa_measure_read(buf.data_ptr(), nbytes, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, R.load().rswa_status_string(st)
    torch.cuda.synchronize()
    got = int(sink.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
    want = int(host.view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
    assert got == want
