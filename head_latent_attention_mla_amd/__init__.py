"""MI355X-native absorbed MLA decode attention.

The compute path is the HIP library ``libmla.so`` (C ABI declared in
``include/mla.h``); ``head_latent_attention_mla_amd.mla`` is its thin ctypes
binding.  ``workloads`` draws seeded synthetic inputs.
"""
