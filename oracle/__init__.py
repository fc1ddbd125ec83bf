"""CPU oracle (plain numpy, float64) for absorbed MLA attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, calls or links anything here.
"""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import (absorbed_query, bf16_bits_to_f64, cache_bytes_per_token, dense_visible_positions,
                         expanded_scores, indexed_visible_positions, latent_attention, mla_reference,
                         query_position, softmax_attention, up_project, visible_sets)
from . import kpool_indexer  # noqa: F401  (the k-pooled indexer that produces position lists)
from . import latent_append  # noqa: F401  (down-projection of new tokens into the cache)
from . import naive_form  # noqa: F401  (the expanded form, stage by stage)
