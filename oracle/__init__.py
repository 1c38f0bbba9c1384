"""CPU oracle for online KV-vector quantization — TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, float64 statement of what the GPU library
computes.  It exists to check the library and nothing else: only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it.
The GPU product path never imports, links or calls anything in here, and this
package never imports the GPU library.  The two share no code; the only
common module is ``synth`` (seeded random inputs, none of the method's
arithmetic).
"""
from .tq_oracle import *  # noqa: F401,F403
from . import polar_oracle as polar  # noqa: F401
