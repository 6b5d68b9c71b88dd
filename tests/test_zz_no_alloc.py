"""tq2_gemm_noalloc (the allocation-free variant of tq2_gemm_ws) against
tq2_gemm_ws with a caller workspace: the same kernels on the same inputs, so
the results must match bit for bit.  Two calls in a row, the second with a
smaller problem (the scratch array keeps the first call's contents), and the
smaller one also against the oracle within path 2's tolerance."""

import numpy as np
import pytest

import oracle
import tq2_inputs as G
from tests.parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq2():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    from gemv_tq2_g128_amd import tq2 as mod
    return mod


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_noalloc_matches_workspace_entry(tq2):
    for (m, n, k, res) in ((100, 200, 4096, True), (40, 96, 1152, False)):
        print("noalloc case", m, n, k, res, flush=True)
        c = G.random_case(3100 + m, m, n, k, residual=res)
        soa = tq2.reformat_aos_to_soa(_dev(c["aos"]), n, k)
        x = _dev(c["x"].reshape(m, k))
        r = _dev(c["residual"].reshape(m, n)) if res else None
        need = tq2.gemm_workspace_bytes(m, n, k)
        assert 0 < need <= tq2.NOALLOC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        a = torch.full((m, n), float("nan"), device="cuda")
        b = torch.full((m, n), float("nan"), device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        rp = r.data_ptr() if r is not None else 0
        st = tq2.gemm_ws_ptr(soa.data_ptr(), x.data_ptr(), rp, a.data_ptr(), m, n, k,
                             ws.data_ptr(), need, stream)
        assert st == tq2.TQ2_OK, tq2.status_string(st)
        st = tq2.gemm_noalloc_ptr(soa.data_ptr(), x.data_ptr(), rp, b.data_ptr(), m, n, k, stream)
        assert st == tq2.TQ2_OK, tq2.status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(a, b), "tq2_gemm_noalloc differs from tq2_gemm_ws at %s" % ((m, n, k),)
        ref = oracle.matmul(c["aos"], c["x"], n, k, c["residual"])
        s = oracle.error_scale(c["aos"], c["x"], n, k, c["residual"])
        ok, msg = check(b.cpu().numpy(), ref, s, 2, c["name"] + "_noalloc")
        print(msg, flush=True)
        assert ok, msg


def test_noalloc_rejects_more_than_its_scratch(tq2):
    m, n, k = 128, 16, 16640                       # needs 4.26 MB > 4 MiB
    assert tq2.gemm_workspace_bytes(m, n, k) > tq2.NOALLOC_SCRATCH_BYTES
    soa = torch.zeros(tq2.soa_bytes(n, k), dtype=torch.uint8, device="cuda")
    x = torch.zeros((m, k), device="cuda")
    out = torch.full((m, n), 7.0, device="cuda")
    st = tq2.gemm_noalloc_ptr(soa.data_ptr(), x.data_ptr(), 0, out.data_ptr(), m, n, k,
                              torch.cuda.current_stream().cuda_stream)
    assert st == tq2.TQ2_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)                   # nothing was enqueued
