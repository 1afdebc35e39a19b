"""The read-only streaming probe reads exactly the regions it is given
(needs an MI355X).

Each lane XORs the dwords it loads and writes the sink only when the result
equals the probe's key, so planting the key in one dword of a region that is
otherwise zero shows whether that dword was read, for every launch shape.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

KEY = 0x9E3779B9 - (1 << 32)          # as int32


def _run(regions, variant):
    import bit_block_quantized_amd as q
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    q.qmv_probe_stream_read(regions, variant, sink)
    torch.cuda.synchronize()
    return int(sink.item())


@pytest.mark.parametrize("variant", range(6))
def test_probe_reads_every_region_and_nothing_past_it(variant):
    buf = torch.zeros(1 << 22, dtype=torch.int32, device="cuda")     # 16 MiB
    base = buf.data_ptr()
    regions = [(base, 4096), (base + 65536, 300000), (base + (1 << 21), 1 << 20),
               (base + (3 << 21), 48)]
    assert _run(regions, variant) == 0
    # a key at the last dword inside region 1 is read ...
    buf.zero_()
    buf[(65536 + 300000 - 4) // 4] = KEY
    assert _run(regions, variant) == KEY, "last dword of region 1 not read"
    # ... one just past a region is not
    buf.zero_()
    buf[(65536 + 300000) // 4] = KEY
    assert _run(regions, variant) == 0, "read past the end of region 1"
    # the first dword of the last, tiny region is read
    buf.zero_()
    buf[(3 << 21) // 4] = KEY
    assert _run(regions, variant) == KEY, "first dword of region 3 not read"


def test_probe_many_regions():
    buf = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    base = buf.data_ptr()
    regions = [(base + r * 16384, 8192) for r in range(64)]
    buf[(63 * 16384 + 8192 - 16) // 4] = KEY
    assert _run(regions, 0) == KEY
