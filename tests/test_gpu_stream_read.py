"""The read-ceiling measurement hook reads every 16-byte word it is given:
a buffer of zeros with one word 0x9e3779b9 makes the block that reads it
write the sink; without it the sink stays untouched.  Sizes cover whole
8-load chunks and a remainder."""
import ctypes

import pytest
import torch

import gated_gqa_decode_amd as ga
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("n_words", [4, 4 * 2048, 4 * 2048 * 8192 + 4 * 37])
@pytest.mark.parametrize("where", ["first", "last", "none"])
def test_stream_read_touches_every_word(n_words, where):
    buf = torch.zeros(n_words, dtype=torch.int32, device=DEV)
    if where == "first":
        buf[0] = torch.tensor(MAGIC, dtype=torch.int64).to(torch.int32)
    elif where == "last":
        buf[-1] = torch.tensor(MAGIC, dtype=torch.int64).to(torch.int32)
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    st = ga.lib.gated_attn_stream_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(4 * n_words),
                                       ctypes.c_void_p(sink.data_ptr()),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ga.GA_OK
    torch.cuda.synchronize()
    got = int(sink.item()) & 0xFFFFFFFF
    assert got == (MAGIC if where != "none" else 7)
