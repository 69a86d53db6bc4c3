"""MI355X-native CSA sparse-attention decode step (HIP kernels behind a C ABI).

The compute entry points live in ``sparse_attention_decode_csa_amd.csa`` and
load the in-tree HIP library on first use; importing the package itself loads
nothing, so the seeded-input module can be used on machines without a GPU.
"""
