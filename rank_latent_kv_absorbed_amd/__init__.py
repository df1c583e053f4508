"""MI355X-native latent KV cache with absorbed multi-head latent attention.

The hot path (fused cache write, absorbed attention, window eviction) lives in
libmla.so, built from csrc/ for gfx950; ``mla`` is its ctypes binding.
"""

from .mla import (  # noqa: F401
    LatentCache, DenseCache, MlaError, LibraryMissing, lib, make_config, attend_flops,
    attend_bytes, mha_attend_flops,
)
