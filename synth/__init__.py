"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package only draws random inputs (catalogs of token-id strings, byte-string
catalogs and vocabularies, embedding tables, hidden states).  It holds none of the decode method's arithmetic: no
trie, no mask, no dot product, no argmax.
"""
from .configs import (  # noqa: F401
    CONFIGS,
    Config,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    catalog,
    embedding,
    hidden_states,
    pack_catalog,
    random_catalog,
    stress_rows,
)
from .charsets import (  # noqa: F401
    CHAR_CONFIGS,
    CharConfig,
    byte_vocab,
    char_catalog,
    char_hidden,
    char_vocab,
    hex_strings,
    tool_strings,
)
