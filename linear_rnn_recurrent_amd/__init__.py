"""Selective state update (Mamba-style SSM decode, prefill, MTP replay and tree
verify) over a paged recurrent-state pool, as hand-written HIP kernels for AMD
Instinct MI355X.

The compute lives in libssu.so (C ABI declared in include/ssu.h); this package
only marshals torch GPU tensors into those calls.
"""
from .ssu import (SsuError, SsuPool, DeviceArray, ReplayLayerTable, StateLayerTable,
                  load_library, ssu_decode, ssu_prefill, ssu_replay, ssu_tree_verify,
                  ssu_tree_verify_noalloc, TREE_SCRATCH_BYTES,
                  ssu_replay_layers, ssu_state_clear_layers, ssu_state_gather,
                  ssu_state_scatter, ssu_state_pack, ssu_state_unpack, pack_workspace_bytes,
                  ssu_gdn_decode, gdn_workspace_bytes, tree_workspace_bytes,
                  LIB_PATH, EXPORTS)

__all__ = ["SsuError", "SsuPool", "DeviceArray", "ReplayLayerTable", "StateLayerTable",
           "load_library", "ssu_decode", "ssu_prefill", "ssu_replay", "ssu_tree_verify",
           "ssu_tree_verify_noalloc", "TREE_SCRATCH_BYTES",
           "ssu_replay_layers", "ssu_state_clear_layers", "ssu_state_gather", "ssu_state_scatter",
           "ssu_state_pack", "ssu_state_unpack", "pack_workspace_bytes", "ssu_gdn_decode", "gdn_workspace_bytes",
           "tree_workspace_bytes",
           "LIB_PATH", "EXPORTS"]
