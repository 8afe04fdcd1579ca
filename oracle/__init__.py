"""fp64 CPU oracle for Transformer-FSQ latent decode (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the bench's CPU-baseline leg may use this
package. The HIP library and its Python binding never import it.
"""
from .fsq_oracle import (  # noqa: F401
    BITS, CODE_OFFSET, DELTA, H_BOUND, LEVELS,
    bytes_per_token, decode_attn, decode_attn_materialised, decode_partials,
    decoder_blocks, encode, fsq_bound, fsq_codes, fsq_levels, full_cache_bytes,
    levels_of_codes, pack_codes, projection, unpack_codes,
)
