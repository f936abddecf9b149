"""CPU oracle for N:M / V:N:M structured-sparse products and dynamic N:M attention.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the
package's smoke check and the benchmark's CPU-baseline leg may import or run
anything in this package. The product path (the HIP library and its binding)
never calls it, and this package imports nothing from the product.

Plain NumPy, float64 wherever arithmetic happens (fp16 -> fp64 is exact). Each
function names the passage of the pages it follows:

* "2:4 sparsity on sparse tensor cores" (lecture notes): the definition, the
  compressed format, how the tensor core uses it, the worked 2 x 8 example.
* "VENOM: A vectorized N:M format for unleashing the power of sparse tensor
  cores" (SC'23): Sec. 3 The V:N:M format, Fig. 2-4.
* "Dynamic N:M fine-grained structured sparse attention mechanism on GPUs"
  (PPoPP'23, Chinese text): Sec. 3.2, Listing 1, Sec. 4.2 Fig. 6(b), Sec. 4.3.
* VENOM Sec. 5 and Fig. 11: the energy (magnitude preservation) metric
  (oracle/energy.py).
* "Coruscant: Co-Designing GPU Kernel and Sparse Tensor Core ...", Sec. 3.1,
  Fig. 7 and Sec. 3.2: the bitmap sparse format (oracle/bitmap.py).
* The attention page's data-type variants, Sec. 1, Fig. 1-3 and Sec. 4.2:
  bf16 scores with 2:4 and fp32 scores with 1:2 (oracle/variants.py).

Every function here is pinned by at least one CPU test against a printed
worked example, a closed form, an invariant, a reduction to a textbook case or
brute force; no function is "parity unpinned".
"""
from .nm import (magnitude_key, select_top_n, prune_encode_nm, decode_nm, spmm_nm,
                 NM_LEGAL_CODES)
from .vnm import column_scores, prune_encode_vnm, decode_vnm, spmm_vnm
from .attention import sddmm_prune_nm, softmax_nm_rows, attention_nm, full_attention
from . import energy
from . import bitmap
from . import variants

__all__ = [
    "magnitude_key", "select_top_n", "prune_encode_nm", "decode_nm", "spmm_nm", "NM_LEGAL_CODES",
    "column_scores", "prune_encode_vnm", "decode_vnm", "spmm_vnm",
    "sddmm_prune_nm", "softmax_nm_rows", "attention_nm", "full_attention",
]
