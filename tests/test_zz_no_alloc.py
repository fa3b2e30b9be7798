"""mmdit_joint_attention_noalloc (the entry point for callers that cannot allocate) against
mmdit_joint_attention with a caller workspace, through the C ABI: two calls in a row, the
second on a smaller input, both with a split tail in the static scratch (the second call
reads a scratch that still holds the first call's key-range results).  The two entry points
run the same kernels with the same split, so the outputs must agree bit for bit; each is also
held to the 16-bit bar against the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_mmdit_amd as mm
from tests.util import assert_close, log, to_host64

pytestmark = pytest.mark.gpu


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).cuda()


# (B, n_vis, n_cond): 288 (batch x head, query tile) items leave 32 for the last round (8 key
# ranges each), then 264 items leave 8 (32 ranges each) on a smaller input
CASES = [(2, 1400, 77, 11), (1, 2700, 77, 21)]


def test_noalloc_matches_workspace_entry_point_twice():
    H, D = 24, 128
    ws = torch.empty(mm.ATTN_SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    for B, nv, nc, seed in CASES:
        log(f"  noalloc: B={B} n_vis={nv} n_cond={nc}")
        qv, kv, vv = (_rand((B, nv, H, D), seed + i) for i in range(3))
        qc, kc, vc = (_rand((B, nc, H, D), seed + 3 + i) for i in range(3))
        ov = torch.empty((B, nv, H, D), dtype=torch.float32, device="cuda")
        oc = torch.empty((B, nc, H, D), dtype=torch.float32, device="cuda")
        mm.joint_attention_noalloc(qv, kv, vv, qc, kc, vc, o_vis=ov, o_cond=oc)
        rv, rc = mm.joint_attention(qv, kv, vv, qc, kc, vc, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ov, rv) and torch.equal(oc, rc), "noalloc and workspace entry points differ"
        for b in range(B):
            f = lambda t: to_host64(t[b:b + 1])  # noqa: E731
            ev, ec = oracle.joint_attention(f(qv), f(kv), f(vv), f(qc), f(kc), f(vc))
            assert_close(f"o_vis[b={b}]", f(ov), ev, 2e-2)
            assert_close(f"o_cond[b={b}]", f(oc), ec, 2e-2)


def test_noalloc_lse_and_errors():
    """With lse the call does not split (same as the workspace entry point); bad arguments are
    refused before launch."""
    H, D, nv, nc = 2, 128, 300, 20
    qv, kv, vv = (_rand((1, nv, H, D), 31 + i) for i in range(3))
    qc, kc, vc = (_rand((1, nc, H, D), 34 + i) for i in range(3))
    ov = torch.empty((1, nv, H, D), dtype=torch.float32, device="cuda")
    oc = torch.empty((1, nc, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, H, nv + nc), dtype=torch.float32, device="cuda")
    mm.joint_attention_noalloc(qv, kv, vv, qc, kc, vc, o_vis=ov, o_cond=oc, lse=lse)
    rv, rc, rl = mm.joint_attention(qv, kv, vv, qc, kc, vc, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(ov, rv) and torch.equal(oc, rc) and torch.equal(lse, rl)
    with pytest.raises(mm.MmditError, match="overlap"):
        mm.joint_attention_noalloc(qv, kv, vv, qc, kc, vc, o_vis=qv, o_cond=oc)   # output on top of an input
    torch.cuda.synchronize()
    assert np.isfinite(to_host64(ov)).all()
