"""The five workloads at their stated sizes (and workload 3 with MXFP4 keys as number 6),
generated once per test session and kept on the GPU (shared by the score, top-k and select
tests)."""
import synth
from gpu_util import Uploaded, say

_CACHE = {}


def full_case(cfg: int):
    if cfg not in _CACHE:
        _CACHE.clear()  # keep at most one full-size workload resident
        say(f"[full] generating workload {cfg}")
        case = synth.full_size(cfg)
        _CACHE[cfg] = (case, Uploaded(case))
    return _CACHE[cfg]
