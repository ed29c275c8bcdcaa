"""windowed_atom_attention_amd -- the windowed atom-attention block on AMD
Instinct MI355X (gfx950): hand-written HIP kernels behind a C-ABI library
(libatomattn.so), with a thin ctypes binding."""
