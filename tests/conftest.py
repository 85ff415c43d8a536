import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


import pytest  # noqa: E402


@pytest.fixture(params=["mma", "valu"])
def decode_stage1(request):
    """Runs a decode test through each stage-1 body (the library reads
    GATED_ATTN_DECODE_STAGE1 at every launch; e4m3 pools and groups above 8
    always take the MFMA body)."""
    old = os.environ.get("GATED_ATTN_DECODE_STAGE1")
    os.environ["GATED_ATTN_DECODE_STAGE1"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("GATED_ATTN_DECODE_STAGE1", None)
    else:
        os.environ["GATED_ATTN_DECODE_STAGE1"] = old
