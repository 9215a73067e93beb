"""Top-k sparse MLA decode for AMD MI355X (gfx950).

The compute path is the HIP library libsparse_mla.so (C ABI in include/sparse_mla.h);
`sparse_mla_decode_03_amd.binding` marshals torch tensors into it.
"""
