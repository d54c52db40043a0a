"""The issue probe of include/gdn_bench.h on the GPU: each mode runs, every
thread writes its float, and the values are the chains' results (a
measurement helper; its timings are the bench's, not asserted here)."""
import pytest
import torch

from speculative_decode_amd import ops

pytestmark = pytest.mark.gpu


def test_issue_probe_modes_write_their_results():
    dev = torch.device("cuda:0")
    blocks, n_mfma, n_valu = 4, 3, 5
    lane = torch.arange(64, dtype=torch.float64)
    for mode in (1, 2, 3):
        out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device=dev)
        ops.issue_probe(out, mode, n_mfma, n_valu)
        torch.cuda.synchronize()
        got = out.view(blocks, 8, 64).double().cpu()
        # matrix waves: lane l supplies A[l % 32][l / 32] = l * 0.001 and
        # B = 0.5; a lane's 16 elements sum its rows 8(r/4) + 4(l/32) + r%4 of
        # column l % 32, over both chains
        if mode & 1:
            a = (torch.arange(64) * 0.001).double()
            col = a.view(2, 32)              # k = lane / 32, m = lane % 32
            c = (col.sum(0) * 0.5) * n_mfma * 2  # two chains; C[m][n] = sum_k A[m][k] B[k][n]
            rows = torch.tensor([[8 * (r // 4) + 4 * (l // 32) + r % 4 for r in range(16)]
                                 for l in range(64)])
            want = c[rows].sum(1)
            assert torch.allclose(got[:, :4], want.expand(blocks, 4, 64), rtol=1e-5)
        else:
            assert (got[:, :4] == 0).all()
        if mode & 2:
            x = torch.stack([lane + i for i in range(8)])
            for _ in range(n_valu):
                x = x * 1.0001 + 0.9999
            want = x.sum(0)
            assert torch.allclose(got[:, 4:], want.expand(blocks, 4, 64), rtol=1e-5)
        else:
            assert (got[:, 4:] == 0).all()
