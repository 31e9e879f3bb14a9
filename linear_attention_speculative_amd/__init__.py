"""MI355X-native KDA RecoverSSM speculative verify and commit.

The compute path is the HIP library `libkda_recoverssm.so` (C ABI in
include/kda_recoverssm.h); this package is its thin torch binding.
"""
from ._abi import LIB_PATH, load  # noqa: F401
from .ops import (  # noqa: F401
    CommitContext,
    KdaError,
    KdaUnaligned,
    abi_version,
    check_verify,
    check_verify_qkv,
    conv_update_verify,
    conv_update_verify_noalloc,
    describe,
    reset_counter,
    set_launch_events,
    verify_args,
    verify_qkv,
)
