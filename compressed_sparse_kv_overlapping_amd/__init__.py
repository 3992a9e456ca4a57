"""MI355X (gfx950) token-axis compressed attention: CSA and HCA.

A thin binding over the C-ABI library libcskv.so (include/cskv.h): every
function checks and marshals torch tensors (device memory and the current
stream) and calls the library; all arithmetic runs in the HIP kernels.  If the
library is not built, every call raises.
"""
from .binding import (compress, compress2, compress2_workspace_size, index_topk, index_topk_noalloc, index_topk_mxfp4, sparse_attend_mxfp4, hca_attend_mxfp4, sparse_attend_mxfp8, hca_attend_mxfp8, sparse_attend, csa_attend, hca_attend, merge,
                      index_topk_workspace_size, attend_workspace_size, csa_workspace_size,
                      hca_workspace_size, library, CskvError, DT_F32, DT_BF16, DT_E4M3)

__all__ = ["compress", "compress2", "compress2_workspace_size", "index_topk", "index_topk_noalloc", "index_topk_mxfp4", "sparse_attend_mxfp4", "hca_attend_mxfp4", "sparse_attend_mxfp8", "hca_attend_mxfp8", "sparse_attend", "csa_attend", "hca_attend", "merge",
           "index_topk_workspace_size", "attend_workspace_size", "csa_workspace_size",
           "hca_workspace_size", "library", "CskvError", "DT_F32", "DT_BF16", "DT_E4M3"]
