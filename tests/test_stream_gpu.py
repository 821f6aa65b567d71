"""The read-only streaming kernel (fp_stream_read) behind the bench's
ceiling: it reads the buffer the way the fused call reads W_cat and writes
a workgroup's word only when a lane's xor of its data hits a fixed value.
Checked: a planted word is found by exactly the workgroup whose 1/256 of
the buffer holds it (so every part of the buffer is read, by the right
workgroup), and nothing else is written."""
import pytest
import torch

import projection_gemm_sparse_amd as P

pytestmark = pytest.mark.gpu

MAGIC = 0x9e3779b9


@pytest.mark.parametrize("nbytes", [18350080, 4096 * 256, 16 * 1000])
def test_stream_read_visits_each_part_once(nbytes):
    n_words = nbytes // 4
    per_wg = -(-(nbytes // 16) // 256)          # 16-byte vectors per workgroup
    for wg in (0, 3, 255):
        v = wg * per_wg + per_wg // 2           # a vector inside workgroup wg's range
        if v * 16 >= nbytes:
            continue
        buf = torch.zeros(n_words, dtype=torch.int32, device="cuda")
        buf[v * 4 + 1] = torch.tensor(MAGIC, dtype=torch.int64).to(torch.int32)
        sink = torch.full((256,), 7, dtype=torch.int32, device="cuda")
        assert P.fp_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), 0) == P.FP_OK
        torch.cuda.synchronize()
        got = sink.cpu().numpy().astype("uint32")
        for b in range(256):
            want = MAGIC if b == wg else 7
            assert got[b] == want, (nbytes, wg, b, hex(int(got[b])))
