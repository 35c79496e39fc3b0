"""The read-bandwidth probe (pa_read_bandwidth_probe) that bench.py reports
the practical HBM ceiling with: it reads every word of the buffer."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words,grid", [(1 << 22, 64), (1 << 22, 4096), (12345 * 4, 7)])
def test_read_probe_reads_every_word(words, grid):
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import say
    say(f"read probe words={words} grid={grid}")
    buf = torch.zeros(words, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    pa.read_bandwidth_probe(buf, grid, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 0  # an all-zero buffer folds to 0: nothing written
    # one planted word, anywhere (here the last), reaches the thread that
    # reads it: its folded value is the pattern, and it writes the sink
    buf[-1] = 0x9E3779B9 - (1 << 32)
    pa.read_bandwidth_probe(buf, grid, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) & 0xFFFFFFFF == 0x9E3779B9
