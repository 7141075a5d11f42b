"""MI355X-native W4A4G4 triple-branch linear (FourTune, arXiv 2607.05711).

The compute lives in libfourtune.so (HIP for gfx950, plain C ABI declared in
include/fourtune.h).  `bit_quantized_amd.ops` is the thin ctypes binding;
`bit_quantized_amd.synth` makes seeded synthetic inputs.  Importing the
package does not load the library; the first call through `ops` does, and
fails loudly if it is not built.
"""
__all__ = ["ops", "synth"]
