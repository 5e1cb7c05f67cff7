"""Weight-absorbed Multi-head Latent Attention (MLA) decode for AMD MI355X (gfx950).

The compute lives in ``libmla.so`` (HIP kernels behind a C ABI, declared in
``include/mla.h``); ``mla_latent_kv_lat_amd.capi`` is the thin Python binding.
"""
