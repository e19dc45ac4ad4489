"""A whole training step (fused id check, transpose hoisted into the forward call on the
library's second stream, pretransposed backward) captured into a HIP graph and replayed: every
replay equals the same step run eagerly, bit for bit, with unrelated eager work and host
synchronisations between the replays."""
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import oracle
import tbe_inputs as ti
from test_gpu_forward import small_spec

pytestmark = pytest.mark.gpu


class Step:
    """Device buffers of one batch and the calls of one step on them."""

    def __init__(self, bt, weights, momentum, cfg_kw=None):
        cfg_kw = cfg_kw or {}
        self.bt = bt
        self.t = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device="cuda", pooling_hint=bt.spec.pooling_hint)
        self.W, self.mom = weights, momentum
        self.idx, self.off = bt.indices.cuda(), bt.offsets.cuda()
        self.psw = None if bt.psw is None else bt.psw.cuda()
        self.grad = bt.grad_out.cuda()
        self.out = torch.zeros(bt.B, sum(bt.D), device="cuda")
        self.counts = torch.zeros(2, dtype=torch.int64, device="cuda")
        self.bws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(self.t))
        self.cfg = tbe.make_config(long_threshold=16, chunk=8, **cfg_kw)
        self.bcfg = tbe.make_config(long_threshold=16, chunk=8, pretransposed=1, **cfg_kw)
        self.ws = tbe.workspace(tbe.tbe_backward_workspace_bytes(self.t, self.idx.numel(),
                                                                 self.psw is not None, self.cfg))

    def __call__(self):
        spec = self.bt.spec
        tbe.tbe_forward_hoisted(self.t, self.W, self.idx, self.off, self.psw, self.out, self.counts,
                                self.bws, self.ws, self.cfg)
        lr = oracle.f32_literal(spec.lr)
        if spec.optimizer == "sgd":
            tbe.tbe_backward_sgd(self.t, self.W, self.idx, self.off, self.psw, self.grad, lr, self.ws,
                                 self.bcfg)
        else:
            tbe.tbe_backward_rowwise_adagrad(self.t, self.W, self.mom, self.idx, self.off, self.psw,
                                             self.grad, lr, oracle.f32_literal(spec.eps), self.ws,
                                             self.bcfg)


# dense rows picked before the sort: the backward runs them, the long runs and a second short-run
# grid on the second stream beside the first, both grids taking work from a shared counter
PRESORT = dict(dense_min=64, dense_presort=1)


@pytest.mark.parametrize("name,cfg_kw", [("skewed", None), ("mixed", None), ("histogram", None),
                                         ("skewed", PRESORT)])
def test_step_graph_replays_match_eager(name, cfg_kw):
    bt = ti.make_batch(small_spec(name), 95)
    mom0 = (bt.momentum if bt.momentum is not None else torch.zeros(sum(bt.E))).cuda()
    eager = Step(bt, bt.weights.cuda(), mom0.clone(), cfg_kw)
    graphed = Step(bt, bt.weights.cuda(), mom0.clone(), cfg_kw)
    # warm-up outside the capture (makes the library's second stream), then reset the state
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graphed()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphed.W.copy_(bt.weights.cuda())
    graphed.mom.copy_(mom0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for k in range(3):
        g.replay()
        eager()
        scratch.mul_(1.5).add_(float(k))   # unrelated eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(graphed.out.view(torch.int32), eager.out.view(torch.int32)), k
        assert torch.equal(graphed.W.view(torch.uint8), eager.W.view(torch.uint8)), k
        assert torch.equal(graphed.mom.view(torch.int32), eager.mom.view(torch.int32)), k
        assert torch.equal(graphed.counts, eager.counts), k
