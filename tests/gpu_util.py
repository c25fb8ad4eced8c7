"""Helpers for the GPU parity tests: upload at an element offset, compare
(re-exported from the shared ``harness`` module)."""
from harness import (DEV, ELEM, NP_DTYPE, TORCH_DTYPE, bf16_nan, download, f16_nan,  # noqa: F401
                     mismatches, nan_mask, ulp_f32, upload)
