"""fp8_mla_latent_amd: absorbed MLA decode over an fp8-e4m3 latent KV cache on
MI355X (gfx950).  The product is the C-ABI library ``libmla8.so`` (header
``include/mla8.h``); ``fp8_mla_latent_amd.mla8`` is its thin Python binding."""

__all__ = ["mla8", "workloads"]
