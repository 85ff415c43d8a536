import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


import pytest  # noqa: E402


@pytest.fixture(params=["offset32", "wide"])
def page1_copies(request):
    """Runs a page-size-1 decode test through both forms of the stage-1
    copies: 32-bit offsets from the pool's start (what small pools get) and
    64-bit addresses (what pools of more than 4 GiB of rows get; the library
    reads GATED_ATTN_DECODE_WIDE at every launch)."""
    old = os.environ.get("GATED_ATTN_DECODE_WIDE")
    os.environ["GATED_ATTN_DECODE_WIDE"] = "1" if request.param == "wide" else "0"
    yield request.param
    if old is None:
        os.environ.pop("GATED_ATTN_DECODE_WIDE", None)
    else:
        os.environ["GATED_ATTN_DECODE_WIDE"] = old
