"""apex_attn_decode_noalloc (the decode entry point that allocates nothing and
keeps its split-K partials in the library's own scratch) against
apex_attn_decode with a caller workspace, on two calls in a row, the second
smaller than the first, both splitting the keys so the scratch is used; then
a call whose split needs no scratch."""
import numpy as np
import pytest
import torch

import apex_inputs
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def taa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_attention_amd as t
    t.lib()
    return t


CASES = [
    # B, Sk, Hq, Hkv, d, W, m, seed: the first two need the scratch (several
    # key splits per (b, KV head)); the last merges its two parts in-kernel
    (2, 20000, 16, 1, 128, 0, 19999, 71),
    (1, 5000, 8, 1, 64, 300, 4100, 72),
    (256, 256, 16, 8, 128, 0, 255, 73),
]


def test_noalloc_decode_matches_workspace_decode(taa):
    for B, Sk, Hq, Hkv, d, W, m, seed in CASES:
        print("[no-alloc] case", (B, Sk, Hq, Hkv, d, W, m), flush=True)
        need = taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d)
        assert 0 < need <= 16 << 20
        q, kc, vc, kn, vn = apex_inputs.decode_inputs(B, Sk, Hq, Hkv, d, "bf16", seed=seed,
                                                      device="cuda")
        kc0, vc0 = kc.cpu(), vc.cpu()
        kc2, vc2 = kc.clone(), vc.clone()
        o_ws, o_na = torch.empty_like(q), torch.full_like(q, float("nan"))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        taa.apex_attn_decode(q, kc, vc, kn, vn, o_ws, m=m, W=W, workspace=ws)
        taa.apex_attn_decode_noalloc(q, kc2, vc2, kn, vn, o_na, m=m, W=W)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: identical bits, caches included
        assert torch.equal(o_na, o_ws)
        assert torch.equal(kc2, kc) and torch.equal(vc2, vc)
        ref = oracle.decode(q.cpu(), kc0, vc0, kn.cpu(), vn.cpu(), m=m, W=W)
        err = np.abs(o_na.cpu().double().numpy() - ref)
        print("[no-alloc] vs oracle: max_abs %.3g mean_abs %.3g" % (err.max(), err.mean()),
              flush=True)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3
