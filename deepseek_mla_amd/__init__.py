"""MI355X-native absorbed Multi-head Latent Attention.

The compute path lives in the HIP library built from csrc/ (C-ABI declared in
include/mla.h); ``deepseek_mla_amd.mla`` is its thin Python binding.
"""
