"""MSA index-branch block scores on AMD Instinct MI355X (gfx950).

The operator lives in the HIP library ``libmsa_index_score.so`` (C ABI in
``include/msa_index_score.h``), with the top-k block selection over its
output (``msa_block_topk``); this package holds its sources (``csrc/``), the
hipcc build step (``build.py``) and a ctypes binding with the same names.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MsaError,
    MsaLayoutError,
    MsaTensor,
    block_topk,
    describe,
    index_score,
    load_library,
    msa_block_topk,
    msa_index_score,
    msa_index_score_kernel_family,
    msa_index_score_mxfp4,
    msa_index_score_out_width,
    msa_status_str,
)
