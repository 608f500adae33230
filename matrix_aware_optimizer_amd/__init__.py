"""Muon optimizer step with SignMuon's 1-bit sign / majority-vote tail on MI355X.

The compute path is libmuon.so (hand-written HIP kernels for gfx950 behind a
C ABI, declared in ``include/muon.h``); this package is its ctypes binding
plus host-side orchestration.  PyTorch provides device memory and streams.
"""
from ._abi import (  # noqa: F401
    MUON_BF16, MUON_F32, MUON_MAX_NUMEL, MUON_MAX_VOTERS, MUON_NS_PAD, MuonError, PreparedNS, apply_update, lib,
    majority_vote, muon_momentum, muon_momentum_workspace_bytes, muon_version, ns_apply,
    ns_gram, ns_normalize, ns_orthogonalize, ns_poly, ns_workspace_bytes, packed_words,
    sign_pack, status_string, vote_and_update,
)
from ._abi import MUON_INT8_MAX_VOTERS, sign_int8, sum_int8, threshold_pack  # noqa: F401
from ._abi import apply_update_dense, unpack_signs  # noqa: F401
from ._abi import new_stage_workspace, ns_apply_signs, ns_stage_workspace_bytes  # noqa: F401
from ._abi import MUON_DION_MAX_RANK, dion_step, dion_workspace_bytes  # noqa: F401
from ._abi import ns_bf16_min_side, ns_residual_iterations, ns_workspace_status, set_split_wait_limit  # noqa: F401
from ._abi import muon_momentum_noalloc, time_next_launch  # noqa: F401
from .signmuon import SignMuonStep  # noqa: F401
