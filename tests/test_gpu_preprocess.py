"""GPU parity of the input preparation (vit_preprocess_frames) against the
oracle, bit for bit (the same f32 operations in the same order), for a still
image at the page's full and capped resolutions, a video with an odd frame
count and an identity-size resize; then a short video through the whole
tower, within the oracle's noise envelope."""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import preprocess as P
import synth
import vision_transformer_encoder_amd as vit
from gpu_util import announce, check_within, host_f64, implementation_noise, metrics

pytestmark = pytest.mark.gpu

MEAN, STD = (0.48145466, 0.4578275, 0.40821073), (0.26862954, 0.26130258, 0.27577711)


@pytest.mark.parametrize("case", [
    ("image 724x2172 -> 736x2176", (1, 724, 2172), None),
    ("image 724x2172, max_pixels 1e6", (1, 724, 2172), 1_000_000),
    ("video 3 frames 90x130", (3, 90, 130), None),
    ("4 frames, identity size 64x96", (4, 64, 96), None),
], ids=lambda c: c[0] if isinstance(c, tuple) else str(c))
def test_preprocess_bit_exact(gpu, case):
    name, (F_, H, W), max_pixels = case
    frames = synth.frames_u8(3, F_, (F_, H, W, 3))
    oh, ow = vit.vit_smart_resize(H, W, max_pixels=max_pixels)
    announce(f"vit_preprocess_frames {name}: {F_} x {H} x {W} -> {oh} x {ow}")
    px, grids = vit.vit_preprocess_frames(torch.from_numpy(frames).to(gpu), (oh, ow), MEAN, STD)
    ref, rgrids = P.preprocess_frames(frames, oh, ow, MEAN, STD)
    got = px.cpu().numpy().astype(np.float64)
    assert grids == rgrids
    assert got.shape == ref.shape
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} of {ref.size} values differ"


def test_video_through_the_tower(gpu):
    frames = synth.frames_u8(3, 7, (3, 100, 70, 3))
    oh, ow = vit.vit_smart_resize(100, 70)
    px, grids = vit.vit_preprocess_frames(torch.from_numpy(frames).to(gpu), (oh, ow), MEAN, STD)
    assert len(grids) == 2  # frames (0, 1) and (2, 2)
    ep = synth.encoder_params(0)
    W = vit.EncoderWeights(ep.patch, ep.blocks, ep.mergers, gpu)
    T = px.shape[0]
    announce(f"vit_encoder_forward on a preprocessed 3-frame video, grids {grids}, T={T}")
    out, last = vit.vit_encoder_forward(W, px, grids, want_last_hidden=True)
    torch.cuda.synchronize()
    import oracle.inputs as OI
    ow_ = OI.encoder_weights(ep)
    ref_px, _ = P.preprocess_frames(frames, oh, ow, MEAN, STD)
    ref_out, ref_last = O.encoder_forward(ref_px, ow_, grids)
    with implementation_noise(300):
        eo, el = O.encoder_forward(ref_px, ow_, grids)
    got = host_f64(out)
    for i, name in enumerate(("deepstack8", "deepstack16", "deepstack24", "final")):
        check_within(got[i], ref_out[i], metrics(eo[i], ref_out[i]), f"video tower {name}")
    check_within(host_f64(last), ref_last, metrics(el, ref_last), "video tower last hidden")
