"""Gated DeltaNet decode block for MI355X (gfx950).

One call runs a GDN layer's decode front for 1-16 rows: residual add + Gemma
RMSNorm, in_proj_qkvz / in_proj_ba, the causal conv update with SiLU, the
gated delta rule on the cached SSM state, and the gated RMSNorm. The work runs
in hand-written HIP kernels behind a C ABI (include/gdn_block.h); this package
holds the shapes, the seeded input generator and a thin ctypes binding.
"""
