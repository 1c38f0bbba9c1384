"""Seeded synthetic inputs for the KV-vector quantizer.

This package holds random-number recipes only: Gaussian key/value/query
tensors with scaled outlier channels, and a unit-normalised Gaussian mixture
for inner-product search.  It contains none of the quantizer's arithmetic, so
both the CPU oracle and the GPU library's tests and benchmark may draw their
inputs from it.
"""
from .inputs import (  # noqa: F401
    kv_gaussian,
    tiny_case,
    outlier_channels,
    mixture_db,
    queries_gaussian,
)
