"""libkvc: MI355X-native (gfx950) KV-cache token scoring, eviction/compaction and
hybrid low-rank compression.

The compute lives in the HIP library ``libkvc.so`` behind the C ABI declared in
``include/kvc.h``; ``token_scoring_eviction_amd.kvc`` binds it with ctypes and
``token_scoring_eviction_amd.pipeline`` chains the calls into the ManifoldKV
eviction step and the OjaKV prefill/decode loop.
"""
from . import kvc  # noqa: F401

__all__ = ["kvc"]
