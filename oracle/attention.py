"""Plain float64 attention and the explicit Ulysses slab permutation (test infrastructure).

Follows the X-Stage explainer (gist.science, arXiv 2607.23264), "Contributions",
FlashAttention-A2A (piggybacking) item: in Ulysses-style sequence-parallel attention the
post-attention all-to-all is fused into FlashAttention, so the fused kernel's result is
that of attention followed by the all-to-all.  The attention itself is the standard
non-causal scaled dot-product attention (the pages name FlashAttention without restating
it; FlashAttention is exact attention).

Readings of points the pages leave open (each listed in the design notes):
* inputs q, k, v are [B, S, H, D] row-major (sequence-major, heads interleaved);
* slab p of the all-to-all holds sequence rows [p*S/P, (p+1)*S/P) of every local head,
  laid out [B, S/P, H, D];
* output rounding is bf16 round-to-nearest-even.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float64: the bits are the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values straight to the nearest bf16 (ties to even); returns uint16 bits.

    bf16 keeps 8 significant bits and fp32's exponent range.  For a normal result the
    quantum is 2^(e-8) where x = m * 2^e, 0.5 <= |m| < 1; below 2^-126 the quantum is the
    subnormal step 2^-133.  np.rint rounds half to even and the scaled values are exact in
    float64, so this is a single correctly rounded step (no fp32 double rounding).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = x[finite]
    m, e = np.frexp(xf)
    normal = (e - 1) >= -126
    q = np.where(normal, np.ldexp(np.rint(np.ldexp(m, 8)), e - 8), np.ldexp(np.rint(np.ldexp(xf, 133)), -133))
    q = np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, xf), q)
    out[finite] = q
    out[~finite] = x[~finite]
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(out)
    bits[nan] = np.uint16(0x7FC0)
    return bits


def attention_weights_fp64(q: np.ndarray, k: np.ndarray, scale: float, b: int, h: int, rows=None) -> np.ndarray:
    """Softmax weights W[i, j] = exp(L_ij - max_j L_ij) / sum_j exp(...), L = scale * q_i . k_j."""
    Q = q[b, :, h, :] if rows is None else q[b, np.asarray(rows), h, :]
    L = scale * (Q @ k[b, :, h, :].T)
    L = L - L.max(axis=1, keepdims=True)
    W = np.exp(L)
    return W / W.sum(axis=1, keepdims=True)


def attention_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, rows=None, block: int = 512) -> np.ndarray:
    """Non-causal softmax(scale * Q K^T) V per (batch, head), all in float64.

    q, k, v: float64 [B, S, H, D].  Returns O [B, S, H, D] or, when ``rows`` (query
    indices) is given, O[:, rows] of shape [B, len(rows), H, D].  Query rows are processed
    in blocks of ``block`` only to bound memory; each block is the plain definition.
    """
    B, S, H, D = q.shape
    row_idx = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, row_idx.size, H, v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            Kt = np.ascontiguousarray(k[b, :, h, :].T)
            Vh = np.ascontiguousarray(v[b, :, h, :])
            for i0 in range(0, row_idx.size, block):
                sel = row_idx[i0:i0 + block]
                L = scale * (q[b, sel, h, :] @ Kt)
                L -= L.max(axis=1, keepdims=True)
                W = np.exp(L)
                W /= W.sum(axis=1, keepdims=True)
                out[b, i0:i0 + sel.size, h, :] = W @ Vh
    return out


def slab_destination(s: int, S: int, P: int):
    """(destination p, row r within slab p) of sequence row s: slab p owns rows [p*S/P, (p+1)*S/P)."""
    if S % P != 0:
        raise ValueError("Ulysses shards need S divisible by P")
    sp = S // P
    p = 0
    while (p + 1) * sp <= s:
        p += 1
    return p, s - p * sp


def ulysses_scatter(o: np.ndarray, P: int) -> np.ndarray:
    """Post-attention all-to-all send layout: slabs[p, b, r, h, d] = o[b, p*S/P + r, h, d].

    Written destination by destination (one copy per destination p of its contiguous
    sequence shard) rather than as a reshape.
    """
    B, S, H, D = o.shape
    if S % P != 0:
        raise ValueError("Ulysses shards need S divisible by P")
    sp = S // P
    slabs = np.empty((P, B, sp, H, D), dtype=o.dtype)
    for p in range(P):
        for b in range(B):
            slabs[p, b] = o[b, p * sp:(p + 1) * sp]
    return slabs


def ulysses_gather(slabs: np.ndarray) -> np.ndarray:
    """Inverse of ``ulysses_scatter``: concatenate the P sequence shards back into [B, S, H, D]."""
    P, B, sp, H, D = slabs.shape
    o = np.empty((B, P * sp, H, D), dtype=slabs.dtype)
    for p in range(P):
        o[:, p * sp:(p + 1) * sp] = slabs[p]
    return o
