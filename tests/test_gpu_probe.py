"""The read-only streaming kernel (int4vh_stream_read), the bench's
achievable-bandwidth reference: it must read every byte of the buffer once
(the xor of its per-wave words equals the xor of the buffer's 32-bit words in
mode 0) and finish in both modes, including buffers smaller than one wave's
share of the grid.  Needs an MI355X and the built library."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [1024, 64 * 1024, 3 * 1024 * 1024 + 7 * 1024, 64 << 20])
def test_stream_read_reads_every_byte(nbytes):
    from int4_output_head_amd import binding
    print(f"[gpu-probe] stream {nbytes} B", flush=True)
    sys.stdout.flush()
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
    want = int(np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32)))
    out = binding.stream_read(buf, 0)
    torch.cuda.synchronize()
    assert int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))) == want
    out1 = binding.stream_read(buf, 1)
    torch.cuda.synchronize()
    assert int(out1.abs().sum().item()) == 0


def test_stream_read_rejects_bad_sizes():
    from int4_output_head_amd import binding
    buf = torch.zeros(1000, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        binding.stream_read(buf, 0)
