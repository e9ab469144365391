"""The Muon step captured in a HIP graph and replayed: every launch of the
hot path is a kernel (buffers that must start at zero are cleared by kernels,
never by memset nodes), so a captured step replays to bitwise the results of
the same step run eagerly.  Each replay runs from the same momentum buffers
as an eager step between the replays, with unrelated eager work and
synchronisations in between, and is checked against that eager step; this
covers the caller-workspace entry (muon_momentum_ns5_batched; the mixed set
below runs as several launch groups on the caller's stream) and the entry
that allocates nothing (muon_momentum_ns5_batched_static).  The GPT-2 124M step, which the
benchmark times as graph replays, is checked the same way at its full size
(it runs as three parts on three streams, so the capture takes in the
library's side streams), and its first replay against the oracle on one
matrix of each shape."""

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_09_amd import step, workloads

from . import parity

pytestmark = pytest.mark.gpu

# (tile-64 and tile-128 shapes: several launch groups, one stream)
SHAPES = [(768, 768), (768, 2304), (3072, 768), (64, 128), (128, 64), (200, 520), (33, 17), (768, 2304)] + \
    [(768, 3072)] * 10


@pytest.fixture(scope="module")
def muon():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from newton_schulz_09_amd import muon as m
    return m


def _inputs(seed):
    rng = np.random.default_rng(seed)
    gs = [torch.from_numpy(rng.standard_normal(s).astype(np.float32)).cuda() for s in SHAPES]
    bs = [torch.from_numpy((0.1 * rng.standard_normal(s)).astype(np.float32)).cuda() for s in SHAPES]
    return gs, bs


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture (library set-up, first-use work)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match_eager(run_eager, replay, bufs, bufs0, outs, name):
    a = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        print(f"{name}: replay {rep}", flush=True)
        for b, b0 in zip(bufs, bufs0):
            b.copy_(b0)
        run_eager()
        torch.cuda.synchronize()
        want_o = [o.clone() for o in outs]
        want_b = [b.clone() for b in bufs]
        for b, b0 in zip(bufs, bufs0):
            b.copy_(b0)
        _ = a @ a  # unrelated eager work between the eager step and the replay
        torch.cuda.synchronize()
        replay()
        torch.cuda.synchronize()
        for k in range(len(outs)):
            assert torch.equal(outs[k], want_o[k]), f"{name}: replay {rep}, update {k} {tuple(outs[k].shape)}"
            assert torch.equal(bufs[k], want_b[k]), f"{name}: replay {rep}, buffer {k} {tuple(bufs[k].shape)}"
        assert all(torch.isfinite(o).all().item() for o in outs)


def test_fused_step_replays_from_a_graph(muon):
    st = step.MuonStep(SHAPES)
    gs, bs = _inputs(5)
    for k in range(len(SHAPES)):
        st.grads[k].copy_(gs[k])
        st.bufs[k].copy_(bs[k])
    bufs0 = [b.clone() for b in st.bufs]
    graph = _capture(st.fused_step)
    _replays_match_eager(st.fused_step, graph.replay, st.bufs, bufs0, st.outs, "caller workspace")


def test_static_entry_replays_from_a_graph(muon):
    gs, bs = _inputs(6)
    outs = [torch.empty_like(g) for g in gs]
    bufs0 = [b.clone() for b in bs]

    def run():
        muon.momentum_ns5_batched_static(gs, bs, outs=outs, mu=0.95)

    graph = _capture(run)
    _replays_match_eager(run, graph.replay, bs, bufs0, outs, "static workspace")
    # and the same as the caller-workspace entry
    ref_b = [b.clone() for b in bufs0]
    want = muon.ns5_batched(gs, bufs=ref_b, mu=0.95)
    for b, b0 in zip(bs, bufs0):
        b.copy_(b0)
    graph.replay()
    torch.cuda.synchronize()
    for k in range(len(gs)):
        assert torch.equal(outs[k], want[k]), k
        assert torch.equal(bs[k], ref_b[k]), k


@pytest.mark.timeout(600)
def test_gpt2_124m_step_replays_from_a_graph(muon):
    """The benchmark's configuration: the 48-matrix GPT-2 124M step captured
    once and replayed; every replay bitwise equals the eager step from the
    same buffers, and the first replay's updates of one matrix per shape
    match the oracle (momentum within 1 float32 ulp)."""
    items = workloads.gpt2_124m()
    st = step.MuonStep([it[2].shape for it in items])
    for k, (_, _, G, buf) in enumerate(items):
        st.grads[k].copy_(torch.from_numpy(G))
        st.bufs[k].copy_(torch.from_numpy(buf))
    bufs0 = [b.clone() for b in st.bufs]
    graph = _capture(st.fused_step)
    for b, b0 in zip(st.bufs, bufs0):
        b.copy_(b0)
    graph.replay()
    torch.cuda.synchronize()
    for k in range(4):  # one matrix of each shape (the layer-0 block)
        _, _, G, buf = items[k]
        want_b, want_u = oracle.momentum_nesterov(G, buf, 0.95)
        assert parity.ulp_diff32(parity.to_np(st.bufs[k]), want_b).max() <= 1
        r = parity.assert_ns5_parity(parity.to_np(st.outs[k]), oracle.ns5(want_u), f"replay, {G.shape}")
        print(f"gpt2-124m replay {G.shape}: relative Frobenius {r:.3g}", flush=True)
    _replays_match_eager(st.fused_step, graph.replay, st.bufs, bufs0, st.outs, "gpt2-124m")
