import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def library_asm(tmp_path_factory):
    """{source: (kernels checked, violations, assembly text)} for every
    library source that loads memory straight into LDS, compiled once per
    session for gfx950 with the library's own flags."""
    from concurrent.futures import ThreadPoolExecutor

    from blockwise_attention_ffn_amd import build as B

    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not installed")
    d = str(tmp_path_factory.mktemp("asm"))
    srcs = [s for s in B.SOURCES if s.endswith(".hip") and B.uses_lds_dma(s)]
    with ThreadPoolExecutor(max_workers=4) as ex:
        res = list(ex.map(lambda s: B.check_source(s, out_dir=d), srcs))
    out = {}
    for s, (checked, errs) in zip(srcs, res):
        with open(os.path.join(d, os.path.splitext(s)[0] + ".gfx950.s")) as fh:
            out[s] = (checked, errs, fh.read())
    return out
