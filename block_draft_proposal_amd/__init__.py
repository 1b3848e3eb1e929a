"""DFlash2 draft-block hot path for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``libdflash.so`` (declared in ``include/dflash.h``); this package holds that
library's sources (``csrc/``), its build script and a thin ctypes binding.
"""
from .binding import (  # noqa: F401
    DraftConfig,
    BlockArgs,
    DFlashError,
    LIB_PATH,
    EXPORTED,
    lib,
    last_error,
    make_config,
    dflash_validate_config,
    dflash_conv,
    dflash_conv_prepare,
    dflash_topk,
    dflash_lattice,
    dflash_walk,
    dflash_verify,
    dflash_lm_head,
    dflash_lm_head_topk,
    dflash_propose_block,
    dflash_propose_block_noalloc,
    ProposeBlock,
    ProposeGraph,
    dflash_philox_uniforms,
    dflash_hbm_ceiling,
    CEILING_READ,
    CEILING_COPY,
    propose_block_workspace_size,
    propose_block_schedule,
    SCHEDULE_ONE_LAUNCH,
    SCHEDULE_AUX_STREAM,
)
