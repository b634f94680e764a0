"""The allocation-free device packer against the one with a workspace argument.

tq_pack_tq2_dev_noalloc runs the kernels of tq_pack_tq2_dev with the
workspace in the library's fixed per-device array.  Two calls in a row, the
second on a smaller matrix (so a stale total from the first call would show),
each through the raw C ABI, must give exactly the bytes, scales and gamma of
tq_pack_tq2_dev on the same latents (and of the host packer).
"""

import sys

import numpy as np
import pytest

from synth import latent_weights_f32, seed_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("bit_mixed_precision_amd.binding")


def _noalloc(W):
    N, K = W.shape
    qs = torch.full((N, K // 4), 0xAB, dtype=torch.uint8, device="cuda")
    sc = torch.full((N, K // 256), 7.0, dtype=torch.float16, device="cuda")
    g = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    st = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    rc = tq.lib.tq_pack_tq2_dev_noalloc(W.data_ptr(), N, K, 1e-5, qs.data_ptr(), sc.data_ptr(),
                                       g.data_ptr(), st.data_ptr(), s)
    assert rc == tq.TQ_OK, tq.tq_status_string(rc)
    torch.cuda.synchronize()
    return qs, sc, g, st


def test_noalloc_pack_matches_workspace_pack_twice():
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    for i, (N, K, sigma) in enumerate([(1024, 4096, 0.02), (96, 512, 3.0)]):
        print(f"[noalloc] call {i}: N={N} K={K}", file=sys.stderr, flush=True)
        Wh = latent_weights_f32(seed_for(910, i, N, K), N, K, sigma)
        W = torch.from_numpy(Wh).cuda()
        qs, sc, g, st = _noalloc(W)
        q_ref, s_ref, g_ref, st_ref = tq.tq_pack_dev(2, W)
        torch.cuda.synchronize()
        assert int(st.item()) == tq.TQ_OK == int(st_ref.item())
        assert torch.equal(qs, q_ref)
        assert torch.equal(sc.view(torch.int16), s_ref.view(torch.int16))
        assert float(g.item()) == float(g_ref.item())
        qh, shh, gh = tq.tq_pack_tq2(Wh, eps=1e-5)
        np.testing.assert_array_equal(qs.cpu().numpy(), qh)
        assert float(g.item()) == gh


def test_noalloc_pack_argument_errors():
    """Argument errors before any device work: null, shape, alignment."""
    A = 0x10000
    call = lambda W=A, N=64, K=512, q=A, s=A: tq.raw_call(
        "tq_pack_tq2_dev_noalloc", W, N, K, 1e-5, q, s, None, None, None)
    assert call(W=None) == tq.TQ_ERR_NULL
    assert call(q=None) == tq.TQ_ERR_NULL
    assert call(K=300) == tq.TQ_ERR_SHAPE
    assert call(N=0) == tq.TQ_ERR_SHAPE
    assert call(K=(1 << 20) + 256) == tq.TQ_ERR_SHAPE
    assert call(W=A + 4) == tq.TQ_ERR_ALIGN
