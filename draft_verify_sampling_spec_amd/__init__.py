"""MI355X-native batched draft verification (speculative decoding).

The hot path is the HIP library ``libspec_verify.so`` (C ABI in
``include/spec_verify.h``); ``binding`` is a thin ctypes layer over it for
torch tensors. Build with ``python -m draft_verify_sampling_spec_amd.build``.
"""
from .binding import (HiddenVerify, MarkovDraft, SpecVerify, head_stats, load,  # noqa: F401
                      philox_words, schedule_budgets, verify_noalloc)
