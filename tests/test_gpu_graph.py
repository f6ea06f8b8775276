"""The whole tower captured as one HIP graph (torch.cuda.CUDAGraph around
vit_encoder_forward, which allocates nothing and never synchronises) and
replayed: every replay must equal the eager forward bit for bit, with eager
work and synchronisations of the program between the replays."""

import pytest
import torch

import synth
import vision_transformer_encoder_amd as vit
from gpu_util import announce

pytestmark = pytest.mark.gpu


def test_encoder_graph_replays_match_eager(gpu):
    ep = synth.encoder_params(0)
    W = vit.EncoderWeights(ep.patch, ep.blocks, ep.mergers, gpu)
    grids = [(18, 54), (12, 20)]  # two windows, 972 + 240 tokens
    T = sum(h * w for h, w in grids)
    px = torch.from_numpy(synth.pixels(1, T)).to(gpu)
    px_other = torch.from_numpy(synth.pixels(2, T)).to(gpu)
    grid_dev = torch.tensor(grids, dtype=torch.int32, device=gpu)
    ws = torch.empty(vit.vit_encoder_workspace_size(T, len(grids)), dtype=torch.uint8, device=gpu)
    out = torch.empty((4, T // 4, 4096), dtype=torch.bfloat16, device=gpu)
    announce(f"vit_encoder_forward eager reference T={T}")
    ref, _ = vit.vit_encoder_forward(W, px, grids, grid_dev=grid_dev)
    torch.cuda.synchronize()

    announce("capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vit.vit_encoder_forward(W, px, grids, workspace=ws, out=out, grid_dev=grid_dev)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work on the same buffers between the replays
        out.fill_(0)
        vit.vit_encoder_forward(W, px_other, grids, workspace=ws, out=out, grid_dev=grid_dev)
        torch.cuda.synchronize()
        announce(f"replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep} differs from eager"


def test_encoder_graph_replay_matches_oracle(gpu):
    """A replay of the captured tower against the fp64 oracle itself (not
    only against the eager forward): the four merger outputs and the last
    hidden state of two small images (8 x 8 and 4 x 6), held to the stated
    tolerance or twice the oracle's drift under implementation-size noise,
    whichever is wider (the free-running rule)."""
    import numpy as np

    import oracle as O
    from oracle import inputs as OI
    from gpu_util import check_within, host_f64, implementation_noise, metrics

    ep = synth.encoder_params(0)
    W = vit.EncoderWeights(ep.patch, ep.blocks, ep.mergers, gpu)
    grids = [(8, 8), (4, 6)]
    T = sum(h * w for h, w in grids)
    pxh = synth.pixels(0, T)
    px = torch.from_numpy(pxh).to(gpu)
    grid_dev = torch.tensor(grids, dtype=torch.int32, device=gpu)
    ws = torch.empty(vit.vit_encoder_workspace_size(T, len(grids)), dtype=torch.uint8, device=gpu)
    out = torch.empty((4, T // 4, 4096), dtype=torch.bfloat16, device=gpu)
    last = torch.empty((T, 1152), dtype=torch.bfloat16, device=gpu)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vit.vit_encoder_forward(W, px, grids, workspace=ws, out=out, grid_dev=grid_dev, last_hidden=last)
    torch.cuda.synchronize()
    out.fill_(0)
    last.fill_(0)
    announce(f"graph replay T={T}")
    graph.replay()
    torch.cuda.synchronize()
    ow = OI.encoder_weights(ep)
    ref_out, ref_last = O.encoder_forward(pxh.astype(np.float64), ow, grids)
    with implementation_noise(100):
        n_out, n_last = O.encoder_forward(pxh.astype(np.float64), ow, grids)
    got = host_f64(out)
    for i, name in enumerate(("deepstack8", "deepstack16", "deepstack24", "final")):
        check_within(got[i], ref_out[i], metrics(n_out[i], ref_out[i]), f"graph replay {name}")
    check_within(host_f64(last), ref_last, metrics(n_last, ref_last), "graph replay last hidden")
