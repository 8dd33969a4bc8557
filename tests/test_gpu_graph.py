"""attn_fwd captured in a HIP graph (through torch.cuda.graph) and replayed:
every replay, with eager work and synchronisations in between, must equal
the eager call on the same inputs bit for bit (needs an MI355X)."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("f32", False), ("f16", True)])
def test_graph_replays_match_eager(dtype, causal):
    import transformer_attention_04_amd as A
    w = W.Workload("graph", 2, 8, 640, 700, 64, causal, (dtype,), seed=81)
    q, k, v = (x.to(DEV) for x in W.make_inputs(w, dtype))
    q2, k2, v2 = (x.to(DEV) for x in W.make_inputs(w, dtype, seed=82))
    out = torch.empty_like(q)
    A.attn_fwd(q, k, v, causal=causal, out=out)          # warm-up outside capture
    torch.cuda.synchronize()
    eager = A.attn_fwd(q, k, v, causal=causal).clone()
    eager2 = A.attn_fwd(q2, k2, v2, causal=causal).clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_fwd(q, k, v, causal=causal, out=out)
    for rep in range(6):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from eager"
        # eager work of the program between replays
        junk = A.attn_fwd(q2, k2, v2, causal=causal)
        junk.mul_(2).add_(1)
        torch.cuda.synchronize()
    # new data in the captured input buffers
    q.copy_(q2), k.copy_(k2), v.copy_(v2)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager2), f"replay {rep} on new inputs differs from eager"
