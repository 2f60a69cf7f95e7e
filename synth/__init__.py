"""Seeded synthetic input generators shared by the oracle tests, the GPU
parity tests and the benchmark.  Holds no arithmetic of the method."""
from .gen import (FORMATS, LARGE_SHAPES, PROJECTION_SHAPES, QmvInputs, default_variant,
                  draw_biases, draw_scales, draw_t5_bytes, draw_words, draw_x, make_inputs,
                  packed_row_bytes, seed_for, t5_bytes_per_group)

__all__ = [
    "FORMATS", "LARGE_SHAPES", "PROJECTION_SHAPES", "QmvInputs", "default_variant",
    "draw_biases", "draw_scales", "draw_t5_bytes", "draw_words", "draw_x", "make_inputs",
    "packed_row_bytes", "seed_for", "t5_bytes_per_group",
]
from .spec import QWEN_VOCAB, SpecInputs, make_spec_inputs
