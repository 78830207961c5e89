"""MI355X-native paged Q8_0-K / Q4_0-V attention: Python binding of libkvattn.

The hot path (split-KV matrix-core attention, log-sum-exp merge, ring
streaming scheduler) is HIP/C++ in ``csrc/`` behind the C-ABI of
``include/kvattn.h``; this package only marshals arguments to it.
"""
from .kvattn import (E_ARG, E_HIP, E_NOSPACE, E_PLAN, E_RANGE, E_STATE, E_UNSUPPORTED, OK, PT_HOST,  # noqa: F401
                     PT_RING, PT_RING_FLAG, TYPE_F16, TYPE_Q4_0, TYPE_Q8_0, Handle, KVAttnError, Params, allocate,
                     default_scale, global_error, lib, make_params, page_bytes, sched_simulate, supported,
                     validate_page_table, workspace_bytes, POLICY_CONTEXT, POLICY_FITS, POLICY_GROW_RING,
                     POLICY_HOLD, POLICY_SHRINK_RING, PolicyConfig, PolicyDecision, PolicyObservation, PolicyState,
                     policy_config, policy_step)
