"""CPU oracle for attention on 8-bit floating-point inputs.

TEST INFRASTRUCTURE ONLY. Only the test-suite, the package smoke entry and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it and has no CPU fallback.

Source: "Современное состояние Flash Attention на ROCm" (kripta.biz), the
paragraphs on the seven attention variants and on the ranking: the fastest
variant runs the FlashAttention-2 forward with FP8 operands. The page names
FP8 and nothing more: no format, no scaling, no statement of which products
are taken in FP8.

Readings taken where the page is silent:
  * format: the OCP 8-bit float E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
    m / 8 * 2^-6; the one code with all exponent and mantissa bits set is NaN
    (no infinities); the largest finite magnitude is 1.75 * 2^8 = 448.
  * scaling: one positive descale factor per tensor (Q, K, V); the operand is
    the stored value times its descale.
  * what is computed: exact attention of the dequantized operands, in the
    sense of the bf16 forward (masked softmax of scale * Q K^T, times V,
    normalised over every open key; LSE the natural-log logsumexp of the
    scaled scores). Whatever a kernel rounds on the way (probabilities taken
    to FP8 for the second product, the output to bf16) is kernel error and is
    bounded by the tolerance, not modelled here.
"""
import numpy as np

from oracle import attention as OA

F64 = np.float64


def e4m3_decode(codes):
    """Value of each OCP E4M3 code (uint8 array) as float64, from the field
    definition: sign, 4-bit biased exponent (bias 7), 3-bit mantissa."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(F64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)
    return sign * val


def dequantize(codes, descale):
    """Operand values: decoded codes times the tensor's descale factor."""
    if not (np.isfinite(descale) and descale > 0):
        raise ValueError("descale must be positive and finite")
    return e4m3_decode(codes) * F64(descale)


def forward(q8, k8, v8, descales, vectors, scale, block=1024):
    """O and LSE of the dequantized operands. q8: [B, Sq, H, D] uint8 codes,
    k8/v8: [B, Sk, Hkv, D] uint8 codes, descales: (q, k, v)."""
    dq, dk, dv = descales
    return OA.forward(dequantize(q8, dq), dequantize(k8, dk), dequantize(v8, dv), vectors, scale, block=block)


def forward_rows(q8, k8, v8, descales, vectors, scale, b, h, rows):
    """O and LSE of selected query rows of one (batch, head)."""
    dq, dk, dv = descales
    return OA.forward_rows(dequantize(q8, dq), dequantize(k8, dk), dequantize(v8, dv), vectors, scale, b, h, rows)
