"""MI355X-native Multi-head Latent Attention (absorbed-weight decode over a
paged latent cache), behind a C-ABI HIP library.

Importing the package is cheap; the HIP library is loaded on first use by
``mla_latent_kv_15_amd.lib``.
"""
__all__ = ["inputs", "lib"]
