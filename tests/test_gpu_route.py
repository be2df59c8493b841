"""moe_route on the GPU vs the routing oracle: ids bit-exact, weights within 1e-6."""
import numpy as np
import pytest

from oracle.route import route

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,k,seed", [(1, 16, 2, 0), (64, 256, 8, 1), (37, 256, 6, 2), (8192, 256, 8, 3),
                                        (5, 4096, 32, 4), (3, 7, 7, 5), (0, 256, 8, 6)])
def test_route_parity(T, E, k, seed):
    import torch
    import expert_cached_decode_amd as EC
    rng = np.random.default_rng(seed)
    logits = rng.normal(size=(T, E)).astype(np.float32)
    if T > 2:
        logits[1] = np.round(logits[1] * 2) / 2  # many ties
        logits[2] = 0.0
    lg = torch.from_numpy(logits).cuda()
    ids = torch.full((max(T, 1), k), -7, dtype=torch.int32, device="cuda")
    w = torch.zeros((max(T, 1), k), dtype=torch.float32, device="cuda")
    EC.moe_route(lg, T, E, k, ids, w)
    torch.cuda.synchronize()
    if T == 0:
        assert (ids.cpu() == -7).all()
        return
    sample = range(T) if T <= 64 else rng.choice(T, 64, replace=False)
    ri, rw = route([logits[t] for t in sample], k)
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    for n, t in enumerate(sample):
        assert list(gi[t]) == ri[n], t
        np.testing.assert_allclose(gw[t], rw[n], rtol=0, atol=1e-6)
    assert np.allclose(gw.sum(axis=1), 1.0, atol=1e-6)
