"""GPU check of pa_read_probe, the read-bandwidth probe the bench measures its
ceilings with: every listed tile is read exactly once (the XOR of what the
wavefronts store equals the XOR of the tiles' 16-byte pieces)."""
import numpy as np
import pytest
import torch

import paged_kv_decode_slot_amd as pa
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _xor16(a: np.ndarray) -> np.ndarray:
    return np.bitwise_xor.reduce(a.view(np.uint32).reshape(-1, 4), axis=0)


@pytest.mark.parametrize("tile_bytes,ordered,waves", [(4096, False, 256), (4096, True, 64), (8192, False, 1024),
                                                      (1024, True, 4)])
def test_read_probe_reads_every_listed_tile_once(tile_bytes, ordered, waves):
    g = torch.Generator().manual_seed(tile_bytes + waves)
    n_tiles = 3000
    src = torch.randint(-2**31, 2**31 - 1, (n_tiles * tile_bytes // 4,), dtype=torch.int32, generator=g)
    host = src.numpy().view(np.uint32).reshape(n_tiles, -1)
    if ordered:
        ids = None
        expect = _xor16(host)
        call, sink = pa.prepare_read_probe(src.to(DEV), tile_bytes, None, num_waves=waves)
    else:
        pick = torch.randperm(n_tiles, generator=g)[:1700].to(torch.int32)
        expect = _xor16(host[pick.numpy()])
        ids = pick.to(DEV)
        call, sink = pa.prepare_read_probe(src.to(DEV), tile_bytes, ids, num_waves=waves)
    log(f"[probe] tile {tile_bytes} B, {'address order' if ordered else 'listed tiles'}, {waves} waves")
    call()
    torch.cuda.synchronize()
    got = _xor16(sink.cpu().numpy())
    assert np.array_equal(got, expect)
