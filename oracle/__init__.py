"""fp64 CPU oracle for paged decode attention and its append step.

TEST INFRASTRUCTURE. Only the tests under ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product library never calls it,
and nothing here imports the product library (``paged_kv_cache_177_amd``).

Every function is a plain, slow, literal statement of what the pages define; see
``oracle/reference.py`` for the citations and for the functions whose parity is pinned.
"""

from .reference import (  # noqa: F401
    BLOCK,
    storage_to_f64,
    f32_to_storage,
    rope_tables,
    rope_rotate_f32,
    rms_norm_head_f32,
    append_kv,
    gather_paged,
    gather_padded_columns,
    attend_two_pass,
    attend_brute_force,
    attend_online_tiled,
    attend_split_merge,
    attend_block_sparse,
    attend_block_mask_additive,
    merge_partials,
    decode_paged,
    decode_padded,
    decode_paged_block_sparse,
    decode_padded_additive_mask,
    padded_valid_columns,
    extract_row_padded,
    assemble_padded,
    spike_embed_f32,
    tokenize_kv,
)
