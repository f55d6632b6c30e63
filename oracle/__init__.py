"""CPU oracle and tolerance checker -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The product (``compressed_attention_fwht_amd``)
never imports it, and it never imports the product.
"""
from .kvq_oracle import (hadamard_matrix, fwht, nearest, rvq_encode, reconstruct_rot,
                         reconstruct, attend, attend_dense, lse_merge, window_append,
                         window_flush, smooth_factors, smooth_rows, smooth_keys, smooth_query,
                         smooth_encode, reconstruct_smooth, lloyd_update, fit_codebooks,
                         lloyd_max_levels, lloyd_max_distortion, scalar_nearest, boundary_sum,
                         scalar_rvq_encode, pack_bits, unpack_bits, scalar_reconstruct,
                         scalar_product_codebook, attend_scalar,
                         code_bytes_per_vector,
                         compression_ratio_vs_fp16)
from .check import (check_codes, check_scalar_codes, check_recon, check_attn, CODE_REL_TOL,
                    RECON_ATOL, ATTN_ATOL, ATTN_REL_L2)
