"""Seeded synthetic inputs for the InternVL visual-token connector.

This module only draws numbers and lays out shapes; it holds none of the
connector's arithmetic.  Both the CPU oracle (``oracle/``) and the GPU path
(tests, ``bench.py``) take their inputs from here, so the two sides always see
the same bytes.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    IMG_START,
    IMG_END,
    IMG_CONTEXT,
    TEXT_VOCAB,
    config,
    make_weights,
    make_vit_tiles,
    make_vit,
    make_sequence,
    make_batch_sequences,
    make_valid_tokens,
    make_tiles_per_image,
    to_bf16_exact,
    sample_tiles,
)
