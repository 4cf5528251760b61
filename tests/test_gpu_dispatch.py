"""The dispatch probe through the C ABI: one launch of one-wave workgroups
reports the XCD each ran on.  The decode kernels' column layout is tuned for
the hardware's round robin over the eight XCDs (their results do not depend
on it: every layout is a fixed permutation, checked by the parity tests)."""
import pytest

from paged_kv_cache_50_amd import pagedkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pagedkv.lib()
    yield
    torch.cuda.synchronize()


def test_xcd_probe_reports_every_xcd():
    xcds = pagedkv.xcd_probe(16)
    print(f"[gpu-test] XCDs of 16 consecutive workgroups: {xcds}", flush=True)
    assert all(0 <= x < 8 for x in xcds)
    assert set(xcds) == set(range(8))


def test_xcd_probe_rejects_bad_sizes():
    torch = pytest.importorskip("torch")
    out = torch.empty(4, dtype=torch.int32, device="cuda")
    lib = pagedkv.lib()
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.pkv_xcd_probe(out.data_ptr(), 0, stream) == 2
    assert lib.pkv_xcd_probe(out.data_ptr(), 2000, stream) == 2
