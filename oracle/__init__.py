"""CPU oracle for the Qwen3-VL-style ViT vision-tower forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It is plain numpy in float64,
shares no code, headers, tables or helpers with the HIP library, and is
written directly from the definitions on the source pages:

* FlashRT doc "Qwen3-VL-8B on RTX 5090 (NVFP4 language stack + FP8 ViT)",
  sections 1 (Headline performance), 3 (Inference architecture),
  4 (Correctness) and 5 (Notes & limitations);
* the spark_model source page "layers/vision_encoder.rs" (struct ViTBlock,
  MergerLayer, VisionEncoder: dimensions, weight list, DeepStack indexes);
* the same FlashRT doc, sections 1 and 5, for the image / video
  preprocessing in ``preprocess.py`` (smart_resize, temporal frame pairs);
* TensorRT-Model-Connect PR #2106 "docs(qwen3_omni): record why FP8 is not
  shipped", section Implementation (FP8 scale = amax / 448).

Every function says which passage it follows.  Points the pages leave open
are taken with one fixed reading each; the list of readings lives with the
design notes of the repository.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, brute force or an independent library
routine.  One result is *parity unpinned*: agreement with the trained
Qwen3-VL model (the cosines of section 4 of the FlashRT page) cannot be
checked, because neither the weights nor the reference model are available.
"""

from .vit_oracle import *  # noqa: F401,F403
from . import preprocess  # noqa: F401  (image / video input preparation)
