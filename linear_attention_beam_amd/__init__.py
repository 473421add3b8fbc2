"""Large-beam Gated DeltaNet decoding on AMD Instinct MI355X (gfx950).

The decode runs in hand-written HIP kernels behind the C ABI of
include/gdn_beam.h (libgdnbeam.so).  `binding` mirrors that ABI name for name;
`decoder.BeamDecoder` owns a torch-allocated workspace and one context.
Importing the package without the built library raises ImportError.
"""
from . import binding  # noqa: F401  (loads libgdnbeam.so or raises)
from .binding import GdnBeamError  # noqa: F401

__all__ = ["binding", "GdnBeamError"]
