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


def test_clock_stamps_advance_at_100_mhz():
    """Two stamps around a sleep on the host: the counter advances, at the
    rate bench.py divides by (100 MHz, within 5% of the host's clock over
    ~0.2 s), and each stamp writes only its own word."""
    import time

    import bit_block_quantized_amd as q
    st = torch.full((4,), -1, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream()
    q.qmv_probe_clock(st[1:2], stream=s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    time.sleep(0.2)
    q.qmv_probe_clock(st[2:3], stream=s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    v = st.cpu().tolist()
    assert v[0] == -1 and v[3] == -1
    ticks = v[2] - v[1]
    assert ticks > 0
    rate = ticks / (t1 - t0)
    assert 0.95e8 < rate < 1.05e8, rate
    # a misaligned word is refused on the host, before any launch
    assert q.lib().qmv_probe_clock(st.data_ptr() + 4, None) == 1
