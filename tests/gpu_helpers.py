"""Shared helpers of the GPU parity tests: host<->device moves, edge-value
inputs, and the comparison rules (bit-exact codes and scales; GEMM
tolerances)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import jet_oracle as O
from fp8_blockwise_quantized_amd import inputs


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 array of BF16 values -> BF16 CUDA tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def assert_bits_equal(got, ref, what: str) -> None:
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    if got.dtype == np.float32:
        g, r = got.view(np.uint32), ref.astype(np.float32).view(np.uint32)
    else:
        g, r = got, ref
    bad = np.argwhere(g != r)
    if bad.size:
        idx = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches; first at {idx}: got {got[idx]!r} "
                             f"({g[idx]:#x}) want {ref[idx]!r} ({r[idx]:#x})")


def edge_matrix(K: int = 512) -> np.ndarray:
    """Rows of hard cases for the quantizers, every value BF16-representable.

    Rows: zeros; negative zeros; BF16 subnormals; every E4M3 value and every
    midpoint between neighbours (ties) in groups whose amax is 448 (r = 1), and
    the same times 2^-30 and 2^10 (r a power of two, ties kept); a group below
    the 2^-96 amax floor; values near the BF16 maximum; an outlier-channel row.
    """
    assert K % 128 == 0
    rows = []
    rows.append(np.zeros(K, np.float32))
    rows.append(np.full(K, -0.0, np.float32))
    rng = np.random.default_rng(77)
    sub = rng.integers(1, 0x80, size=K).astype(np.uint32) << 16
    sub |= (rng.integers(0, 2, size=K).astype(np.uint32) << 31)
    rows.append(sub.view(np.float32))
    pos = O.DECODE[:0x7F]
    vals = np.concatenate([pos, (pos[:-1] + pos[1:]) / 2])
    vals = np.concatenate([vals, -vals])
    rng.shuffle(vals)
    need = K
    v = np.resize(vals, need).astype(np.float32)
    for g in range(K // 128):
        v[g * 128 + (g * 37) % 128] = 448.0 if g % 2 == 0 else -448.0
    rows.append(v)
    rows.append((v * np.float32(2.0 ** -30)).astype(np.float32))
    rows.append((v * np.float32(2.0 ** 10)).astype(np.float32))
    rows.append(inputs.to_bf16_values(rng.uniform(-1e-30, 1e-30, K).astype(np.float32)))
    big = inputs.to_bf16_values(rng.uniform(-3.3e38, 3.3e38, K).astype(np.float32))
    rows.append(big)
    rows.append(inputs.activations_with_outliers(1, K, seed=5)[0])
    return np.stack(rows).astype(np.float32)


def oracle_absprod(a64: np.ndarray, b64: np.ndarray) -> np.ndarray:
    """|A| . |B|^T in float64: the scale of accumulation rounding per element."""
    return np.abs(a64) @ np.abs(b64).T


# Accumulation allowance.  The gfx950 FP8 MFMA (16x16x128 f8f6f4, and the
# legacy 16x16x32 fp8 alike) sums its products in sub-blocks at a resolution of
# about 2^-14 of the sub-block's largest product (measured: 448*448 + 1 returns
# 448*448 inside one sub-block; the worst error over random full-range codes is
# 2^-12.4 * sum|a*b|).  The kernels fold each 128-wide step into FP32, so the
# error of one output is a few such roundings per step; 2^-11 * sum_k|a_k*b_k|
# bounds it with margin.
ACC_ALLOW = 2.0 ** -11
FRO_F32 = 1e-4      # FP32 outputs: relative Frobenius bound (the target is 1e-3)
FRO_BF16 = 1e-3     # BF16 outputs, against bf16_rne(fl32(reference))


def check_f32_output(got: np.ndarray, ref: np.ndarray, absprod: np.ndarray, what: str) -> float:
    """FP32 output rule: every element within ACC_ALLOW * sum_k|a_k b_k| of the
    float64 reference, and relative Frobenius error <= FRO_F32."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    tol = ACC_ALLOW * absprod + 1e-38
    bad = np.argwhere(err > tol)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements outside tolerance; first {i}: "
                             f"got {got[i]!r} want {ref[i]!r} tol {tol[i]!r}")
    den = np.linalg.norm(ref)
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))
    assert rel <= FRO_F32, f"{what}: relative Frobenius error {rel:.3e} > {FRO_F32}"
    return rel


def check_bf16_output(got: np.ndarray, ref: np.ndarray, absprod: np.ndarray, what: str,
                      fro: bool = True) -> float:
    """BF16 output rule: every element within one BF16 ulp of the float64
    reference plus ACC_ALLOW * sum_k|a_k b_k|, and relative Frobenius distance
    to bf16_rne(fl32(reference)) <= FRO_BF16 (fro=False: the element rule
    only, for a piece of an output whose Frobenius distance is checked whole
    with bf16_frobenius)."""
    got = np.asarray(got, np.float64)
    a = np.abs(ref)
    ulp = np.ldexp(1.0, (np.floor(np.log2(np.maximum(a, 1e-300))) - 7).astype(np.int64))
    tol = ulp + ACC_ALLOW * absprod + 1e-38
    err = np.abs(got - ref)
    bad = np.argwhere(err > tol)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements outside tolerance; first {i}: "
                             f"got {got[i]!r} want {ref[i]!r} tol {tol[i]!r}")
    if not fro:
        return 0.0
    return bf16_frobenius([got], [ref], what)


def bf16_frobenius(gots, refs, what: str) -> float:
    """Relative Frobenius distance of BF16 outputs (given in pieces) to
    bf16_rne(fl32(reference)), bounded by FRO_BF16 over the whole output."""
    got = np.concatenate([np.asarray(g, np.float64).ravel() for g in gots])
    target = np.concatenate([O.bf16_rne(O.fl32(np.asarray(r, np.float64))).astype(np.float64).ravel()
                             for r in refs])
    den = np.linalg.norm(target)
    rel = float(np.linalg.norm(got - target) / den) if den > 0 else float(np.linalg.norm(got))
    assert rel <= FRO_BF16, f"{what}: relative Frobenius error {rel:.3e} > {FRO_BF16}"
    return rel
