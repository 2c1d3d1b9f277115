"""CPU oracle for global L2-norm gradient clipping (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never does, and shares no code with it.
"""
from .oracle import (F32, F16, BF16, DTYPES, Oracle, default, decode_bits, encode, sumsq, tensor_sumsq, decide,
                     scale_, clip_, clip_per_tensor_, accumulate_, accumulate_clip_, adamw, clip_adamw, amp_avg, amp_update, clip_amp_, lib_path,
                     shards, clip_sharded_)

__all__ = ["F32", "F16", "BF16", "DTYPES", "Oracle", "default", "decode_bits", "encode", "sumsq", "tensor_sumsq",
           "decide", "scale_", "clip_", "clip_per_tensor_", "accumulate_", "accumulate_clip_", "adamw", "clip_adamw", "amp_avg", "amp_update", "clip_amp_", "lib_path", "shards",
           "clip_sharded_"]
