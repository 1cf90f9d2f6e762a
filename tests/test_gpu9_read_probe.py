"""pa_debug_read_probe (measurement support for the K/V load layouts).

The probe's output is fully defined by include/pa.h: wave w of the grid (one
workgroup of `waves` waves per CU) reads blocks[w * per + k] for k < per =
num_blocks / (CUs * waves) rounded down to even, each index clamped to the
buffer's blocks; lane l of a wave folds every 16-byte word it loads into one
value by XOR, and writes the XOR of that value's four 32-bit words, converted
to float, to sink[w * 64 + l]. In the linear layout load i of lane l covers
bytes [1024 i + 16 l, +16) of a block; in the rows layout lane (c, j) = (l %
16, l / 16) covers bytes [64 i + 16 j, +16) of row c. A NumPy model of that
definition must match the device bit for bit, which pins the two lane layouts
the partition pass loads with and the clamping of the block indices.
"""
import numpy as np
import pytest
import torch

import paged_attention_decode_block_amd as pa
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _model(buf, blocks, row_bytes, linear, cus, waves):
    blk = 16 * row_bytes
    nbuf = buf.size // blk
    lpb = row_bytes // 64
    nw = cus * waves
    per = len(blocks) // nw // 2 * 2
    words = buf[: nbuf * blk].view(np.uint32).reshape(nbuf, blk // 4)
    lanes = np.arange(64)
    if linear:
        offs = [1024 * i + 16 * lanes for i in range(lpb)]
    else:
        offs = [(lanes % 16) * row_bytes + 16 * (lanes // 16) + 64 * i for i in range(lpb)]
    sink = np.zeros((nw, 64), dtype=np.uint32)
    for w in range(nw):
        acc = np.zeros((64, 4), dtype=np.uint32)
        for k in range(per):
            b = min(max(int(blocks[w * per + k]), 0), nbuf - 1)
            for o in offs:
                idx = (o // 4)[:, None] + np.arange(4)[None, :]
                acc ^= words[b][idx]
        sink[w] = acc[:, 0] ^ acc[:, 1] ^ acc[:, 2] ^ acc[:, 3]
    return sink.reshape(-1).astype(np.float32)


@pytest.mark.parametrize("row_bytes", [128, 256, 512])
@pytest.mark.parametrize("linear", [True, False])
def test_read_probe_matches_its_definition(row_bytes, linear):
    cus = pa.pa_query_device(0)
    waves = 2
    rng = np.random.default_rng(2026 + row_bytes + int(linear))
    nbuf = 40
    buf = rng.integers(0, 256, size=nbuf * 16 * row_bytes + 300, dtype=np.uint8)
    # four blocks per wave, some indices outside the buffer (clamped)
    blocks = rng.integers(-5, nbuf + 5, size=cus * waves * 4 + 3, dtype=np.int32)
    sink = torch.full((cus * waves * 64,), float("nan"), device=DEV)
    say(f"[probe] row_bytes {row_bytes} linear {linear}")
    pa.pa_debug_read_probe(torch.from_numpy(buf).to(DEV), torch.from_numpy(blocks).to(DEV),
                           row_bytes, linear, waves, sink)
    torch.cuda.synchronize()
    want = _model(buf, blocks, row_bytes, linear, cus, waves)
    got = sink.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_read_probe_rejects_a_short_sink():
    cus = pa.pa_query_device(0)
    buf = torch.zeros(16 * 256, dtype=torch.uint8, device=DEV)
    blocks = torch.zeros(8, dtype=torch.int32, device=DEV)
    sink = torch.zeros(cus * 4 * 64 - 1, device=DEV)
    with pytest.raises(pa.PaError):
        pa.pa_debug_read_probe(buf, blocks, 256, True, 4, sink)
