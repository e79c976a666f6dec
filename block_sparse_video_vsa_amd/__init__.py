"""MI355X (gfx950) Video Sparse Attention fine block-sparse forward.

The computation lives in the HIP library libvsa.so (C ABI: include/vsa.h);
`native` is its Python binding and `workloads` makes seeded synthetic inputs.
"""
from .native import (VSAError, cube_vbs, fwd_workspace_size,  # noqa: F401
                     load_library, proxy_workspace_size,
                     vsa_fwd, vsa_fwd_lse, vsa_fwd_noalloc, vsa_fwd_prepacked, vsa_fwd_proxy,
                     vsa_fwd_proxy_bitmask, vsa_fwd_proxy_bsr, vsa_merge,
                     vsa_kc_stats, vsa_pack_values, vsa_preprocess, route_workspace_size,
                     vsa_route_topk,
                     vsa_tile, vsa_untile)
