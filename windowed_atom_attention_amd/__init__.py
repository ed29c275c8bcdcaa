"""windowed_atom_attention_amd -- the windowed atom-attention block on AMD
Instinct MI355X (gfx950): hand-written HIP kernels behind a C-ABI library
(libatomattn.so, declared in include/atom_attn.h) with a thin ctypes
binding. Importing the package does not load the library; the first call
does, and fails loudly if it has not been built."""
from .api import (backward_workspace_bytes, block_backward, masks, noalloc_max_bytes,
                  pack_params, packed_bytes, slot_attention_backward,
                  pair_bias_split, profile_enable, profile_read, single_to_pair, slot_attention,
                  tied_row_attention, tied_workspace_bytes, window_table,
                  windowed_atom_attention, workspace_bytes)

__all__ = ["windowed_atom_attention", "masks", "slot_attention",
           "workspace_bytes", "pair_bias_split", "profile_enable", "profile_read",
           "noalloc_max_bytes", "pack_params", "packed_bytes", "window_table",
           "single_to_pair", "tied_row_attention", "tied_workspace_bytes", "block_backward",
           "backward_workspace_bytes", "slot_attention_backward"]
