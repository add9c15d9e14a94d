"""CPU oracle for large-beam decode attention (fp64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call anything in this package.
The library under ``shared_prefix_beam_amd`` never imports it, and this
package imports nothing from the library: the two share no code.  Inputs
come from the seeded generator module, which holds no attention arithmetic.
"""
from .oracle import build, decode_attn, lib_path  # noqa: F401
