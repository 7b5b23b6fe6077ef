"""MI355X (gfx950) KV-cache append + causal GQA attention step.

The computation lives in the HIP library ``libkvc.so`` (C ABI in
``include/kvc.h``); this package is its ctypes binding plus seeded synthetic
workloads.
"""
from .kvc import (KVC_BF16, KVC_F32, KvcDims, KvcError, kv_cache_attention_step,
                  kv_cache_attention_step_, kvc_plan_step, kvc_status_string,
                  kvc_step_inplace, kvc_step_out_of_place, kvc_workspace_bytes, load)

__all__ = ["KVC_BF16", "KVC_F32", "KvcDims", "KvcError", "kv_cache_attention_step",
           "kv_cache_attention_step_", "kvc_plan_step", "kvc_status_string", "kvc_step_inplace",
           "kvc_step_out_of_place", "kvc_workspace_bytes", "load"]
