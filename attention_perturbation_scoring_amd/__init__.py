"""MI355X-native DropKV KV-cache scoring, selection and compaction.

The compute path is the HIP library ``libdropkv.so`` (C-ABI in include/dropkv.h);
``attention_perturbation_scoring_amd.dropkv`` is its thin ctypes binding and
``attention_perturbation_scoring_amd.workload`` draws seeded synthetic inputs.
"""
__all__ = ["dropkv", "workload"]
