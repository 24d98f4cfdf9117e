"""MI355X-native decode-step MQA/GQA attention against a KV cache.

The compute path is a HIP library for gfx950 behind a C ABI
(``include/mqa_decode.h``); :mod:`.binding` marshals torch tensors into it.
Importing the package does not load the native library; the first call does,
and it raises if the library has not been built.
"""
from .workloads import WORKLOADS, Workload, make_inputs, make_prefill_inputs  # noqa: F401


def decode(*args, **kwargs):
    from .binding import decode as _decode
    return _decode(*args, **kwargs)


def prefill(*args, **kwargs):
    from .binding import prefill as _prefill
    return _prefill(*args, **kwargs)
