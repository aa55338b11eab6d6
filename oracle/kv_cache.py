"""Plain CPU oracle for the FP8 KV cache with recalibrated scales.

TEST INFRASTRUCTURE ONLY. Imported by tests/, by __graft_entry__.smoke() and
by the cpu_baseline leg of bench.py, and by nothing else. The GPU library
never calls it and shares no code with it.

Sources: [FP8-RL] 66260.cn news item on NVIDIA's FP8-RL, KV-cache paragraph:
the technique is extended to compressing the KV cache, with scale factors
calibrated dynamically and re-adjusted after each model update.  [NV-RL]
nmedialink.com repost of the NeMo-RL FP8 blog, section on the KV cache and
attention: FP8 is brought into the KV cache (and attention) of the rollout.

The pages give neither the granularity nor the calibration data, so:

R15 One FP32 scale per tensor: one for a layer's K cache and one for its V
    cache (the plainest reading; the common per-tensor KV-cache scale).
R16 Recalibration after a weight update: amax = max |x| over the K (or V)
    rows of a calibration batch, then the scale pair of jet_oracle's reading
    R2: s = fl32(max(amax, 2^-96) / 448), r = fl32(448 / max(amax, 2^-96)).
R17 Appending tokens: the rows of K (V) are quantized with the stored r,
    codes = enc(fl32(x * r)) with jet_oracle's encoder (reading R3: round to
    nearest even, saturating at +-448, so values beyond the calibration
    batch's amax saturate), and written to the cache rows named by a slot
    index per token; a negative slot (a padding token) writes nothing.
"""
from __future__ import annotations

import numpy as np

from oracle.jet_oracle import e4m3_encode, fl32, scale_pair


def kv_calibrate(k, v):
    """R15-R16: ((s_k, r_k), (s_v, r_v)) as float32 scalars from the BF16 rows of
    a calibration batch (float32 arrays holding BF16 values)."""
    out = []
    for x in (k, v):
        amax = np.float32(np.max(np.abs(np.asarray(x, np.float32)))) if np.size(x) else np.float32(0.0)
        s, r = scale_pair(np.array([amax], np.float32))
        out.append((np.float32(s[0]), np.float32(r[0])))
    return tuple(out)


def kv_codes(x, r) -> np.ndarray:
    """R17: E4M3 codes of the rows of x with the stored multiplier r."""
    return e4m3_encode(fl32(np.asarray(x, np.float32) * np.float32(r)))


def kv_append(cache, x, slots, r) -> np.ndarray:
    """R17: a copy of cache [slots_total, D] (uint8) with row slots[t] set to the
    codes of x[t] for every t with slots[t] >= 0."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    codes = kv_codes(x, r)
    for t, slot in enumerate(np.asarray(slots, np.int64)):
        if slot >= 0:
            out[slot] = codes[t]
    return out
