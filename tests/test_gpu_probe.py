"""The read probe (gqa_hbm_read_probe) reads every 16-byte vector of its two
buffers: a buffer that is zero but for one vector holding the probe's fixed
word makes exactly the wavefront that reads that vector store the word to
the sink, wherever the vector lies (full rounds, ragged ends, either buffer,
any launch shape); all-zero buffers leave the sink untouched."""
import pytest
import torch

import gqa_mqa_kv_amd as gqa

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MAGIC = 0x9e3779b9   # the word the probe compares each wavefront's fold with


def probe(a, b, wpc):
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    gqa.hbm_read_probe(a, wpc, sink, b=b)
    torch.cuda.synchronize()
    return int(sink.view(torch.int32)[0]) & 0xffffffff


@pytest.mark.parametrize("a_vecs,b_vecs", [(64, 0), (4096 + 1, 0), (65536 + 3, 777), (1, 5), (0, 70001),
                                           (1 << 20, (1 << 18) + 5)])
@pytest.mark.parametrize("wpc", [1, 2, 8])
def test_probe_reads_every_vector(a_vecs, b_vecs, wpc):
    print("[gpu-case] probe", a_vecs, b_vecs, wpc, flush=True)
    a = torch.zeros(max(a_vecs, 1), 4, dtype=torch.int32, device=DEV)[:a_vecs]
    b = torch.zeros(max(b_vecs, 1), 4, dtype=torch.int32, device=DEV)[:b_vecs] if b_vecs else None
    assert probe(a, b, wpc) == 0
    g = torch.Generator().manual_seed(a_vecs + 7 * b_vecs + wpc)
    total = a_vecs + b_vecs
    picks = {0, total - 1} | {int(i) for i in torch.randint(total, (6,), generator=g)}
    for i in sorted(picks):
        buf, j = (a, i) if i < a_vecs else (b, i - a_vecs)
        buf[j, 1] = torch.tensor(MAGIC, dtype=torch.int64).to(torch.int32)
        assert probe(a, b, wpc) == MAGIC, "vector %d of %d not read" % (i, total)
        buf[j, 1] = 0
