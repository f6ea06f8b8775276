"""Image / video preprocessing of the vision tower's input (test
infrastructure only, like the rest of this package).

Sources: FlashRT doc "Qwen3-VL-8B on RTX 5090", section 1 (image
preprocessing runs on the GPU; ``max_pixels`` applies the processor's
smart_resize, which rounds to the patch grid; the "TTFT vs resolution"
table), section 3 (per-prompt geometry) and section 5 (each image, or each
video frame group, is an independent attention window); spark_model page
"layers/vision_encoder.rs", PATCH_DIM doc (a patch is C x temporal_patch_size
x patch_size^2 = 3 x 2 x 16 x 16 = 1536 values).

Readings where the pages are silent (each fixed once):

* smart_resize with factor 32 (patch 16 x merge 2): each side rounded to the
  nearest multiple of 32 (ties to even, at least 32); if the area exceeds
  max_pixels, both sides are scaled by beta = sqrt(h w / max_pixels) and
  floored to multiples of 32; below min_pixels, scaled up by
  sqrt(min_pixels / (h w)) and ceiled.  This reproduces every row of the
  "TTFT vs resolution" table for the 2172 x 724 image.
* resize: bilinear with half-pixel centres (source = (dst + 0.5) H/H' - 0.5,
  clamped at 0, upper neighbour clamped to the last row / column), in f32
  with every operation rounded in a fixed order;
* normalisation: y = v a_c + b_c with a_c = 1/(255 std_c) and
  b_c = -mean_c/std_c rounded to f32 (mean and std are f32 inputs);
* patchify: frames 2g and 2g+1 form temporal group g (a missing last frame
  repeats the one before; a still image is one frame), each group is one
  window of (h'/16) x (w'/16) patches in raster order, and a patch vector is
  laid out [channel][frame of the pair][row 0..15][col 0..15].
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

PATCH = 16
TEMPORAL = 2
MERGE_FACTOR = 32  # patch 16 x spatial merge 2


def smart_resize(height: int, width: int, factor: int = MERGE_FACTOR, min_pixels: int = 0,
                 max_pixels: Optional[int] = None) -> Tuple[int, int]:
    """(height', width'), multiples of ``factor``, per the reading above."""
    h_bar = max(factor, int(round(height / factor)) * factor)
    w_bar = max(factor, int(round(width / factor)) * factor)
    if max_pixels is not None and h_bar * w_bar > max_pixels:
        beta = math.sqrt(height * width / max_pixels)
        h_bar = max(factor, math.floor(height / beta / factor) * factor)
        w_bar = max(factor, math.floor(width / beta / factor) * factor)
    elif min_pixels and h_bar * w_bar < min_pixels:
        beta = math.sqrt(min_pixels / (height * width))
        h_bar = math.ceil(height * beta / factor) * factor
        w_bar = math.ceil(width * beta / factor) * factor
    return h_bar, w_bar


def _axis(n_in: int, n_out: int):
    f = np.float32
    scale = f(n_in) / f(n_out)
    s = (np.arange(n_out, dtype=np.float32) + f(0.5)) * scale - f(0.5)
    s = np.maximum(s, f(0.0))
    i0 = np.floor(s).astype(np.int64)
    i1 = np.minimum(i0 + 1, n_in - 1)
    lam = (s - i0.astype(np.float32)).astype(np.float32)
    return i0, i1, lam, (f(1.0) - lam).astype(np.float32)


def resize_bilinear(frame, out_h: int, out_w: int) -> np.ndarray:
    """[H, W, C] uint8 (or values on the u8 grid) -> [out_h, out_w, C] f32
    values:  v = (hy (hx P00 + lx P01)) + (ly (hx P10 + lx P11)), each
    product and sum rounded to f32."""
    img = np.asarray(frame, dtype=np.float32)
    H, W = img.shape[:2]
    y0, y1, ly, hy = _axis(H, out_h)
    x0, x1, lx, hx = _axis(W, out_w)
    p00 = img[y0][:, x0]
    p01 = img[y0][:, x1]
    p10 = img[y1][:, x0]
    p11 = img[y1][:, x1]
    hx_, lx_ = hx[None, :, None], lx[None, :, None]
    hy_, ly_ = hy[:, None, None], ly[:, None, None]
    top = hx_ * p00 + lx_ * p01
    bot = hx_ * p10 + lx_ * p11
    v = hy_ * top + ly_ * bot
    assert v.dtype == np.float32
    return v


def normalize_coefficients(mean: Sequence[float], std: Sequence[float]):
    """a_c = 1/(255 std_c), b_c = -mean_c/std_c, rounded to f32, from mean
    and std taken as f32 values (the precision the per-channel constants
    are given in)."""
    m32 = [float(np.float32(m)) for m in mean]
    s32 = [float(np.float32(s)) for s in std]
    a = np.array([1.0 / (255.0 * s) for s in s32], dtype=np.float64).astype(np.float32)
    b = np.array([-m / s for m, s in zip(m32, s32)], dtype=np.float64).astype(np.float32)
    return a, b


def preprocess_frames(frames, out_h: int, out_w: int, mean: Sequence[float], std: Sequence[float]):
    """[F, H, W, 3] uint8 frames -> (pixels [G * (out_h/16) * (out_w/16), 1536]
    f32 values as float64, grids [(out_h/16, out_w/16)] * G), G = ceil(F/2)."""
    fr = np.asarray(frames)
    if fr.ndim != 4 or fr.shape[3] != 3:
        raise ValueError("frames must be [F, H, W, 3]")
    if out_h % PATCH or out_w % PATCH:
        raise ValueError("the resized size must be a multiple of the patch size")
    F = fr.shape[0]
    a, b = normalize_coefficients(mean, std)
    norm = [(resize_bilinear(fr[i], out_h, out_w) * a + b).astype(np.float32) for i in range(F)]
    gh, gw = out_h // PATCH, out_w // PATCH
    rows = []
    for g in range((F + 1) // 2):
        pair = [norm[2 * g], norm[min(2 * g + 1, F - 1)]]
        # [t, gh, 16, gw, 16, c] -> [gh, gw, c, t, 16, 16]
        st = np.stack(pair).reshape(TEMPORAL, gh, PATCH, gw, PATCH, 3)
        rows.append(st.transpose(1, 3, 5, 0, 2, 4).reshape(gh * gw, 3 * TEMPORAL * PATCH * PATCH))
    return np.concatenate(rows).astype(np.float64), [(gh, gw)] * ((F + 1) // 2)
