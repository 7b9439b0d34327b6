"""Pure-Python brute force of the oracle's definitions, for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Written independently of ``kvq_oracle.c``: fp32
arithmetic is emulated with Python floats rounded through ``struct`` ('f'),
fp16 through ``struct`` ('e', round-half-even), and attention uses plain
Python loops in double precision.  The tests compare the C oracle with this
module bit for bit on codes and to 1e-12 on attention.

A product of two fp32 values is exact in a Python float (48 significant bits
fit in 53), and a quotient or sum rounded first to double and then to fp32
equals the correctly rounded fp32 result (double has more than 2*24+2 bits),
so ``f32(a * b)``, ``f32(a / b)`` and ``f32(a + b)`` are IEEE fp32 operations.

Definitions followed: K as Q8_0 and V as Q4_0 with 32-value blocks and an fp16
scale ("Adaptive KV streaming lands on ROCm ...", "What shipped"; "OSCAR2 KV
Cache benchmark", compression-ratio table); exact softmax attention with
shared KV heads ("Context window and KV cache", GQA and flash-attention
sections).
"""
from __future__ import annotations

import math
import struct

BLOCK = 32


def f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f16_bits(x: float) -> int:
    return struct.unpack("<H", struct.pack("<e", x))[0]


def f16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits))[0]


def round_half_away(x: float) -> int:
    r = math.floor(abs(x) + 0.5)
    return int(r if x >= 0 else -r)


def quant_q8_0_block(xs):
    """One block of 32 fp32 values -> (codes, fp16 scale bits)."""
    assert len(xs) == BLOCK
    xs = [f32(x) for x in xs]
    amax = 0.0
    for x in xs:
        amax = max(amax, abs(x))
    d = f32(amax / 127.0)
    idv = f32(1.0 / d) if d != 0.0 else 0.0
    codes = [round_half_away(f32(x * idv)) for x in xs]
    return codes, f16_bits(d)


def quant_q4_0_block(xs):
    """One block of 32 fp32 values -> (codes 0..15, fp16 scale bits)."""
    assert len(xs) == BLOCK
    xs = [f32(x) for x in xs]
    amax, m = 0.0, 0.0
    for x in xs:
        if abs(x) > amax:
            amax, m = abs(x), x
    d = f32(m / -8.0)
    idv = f32(1.0 / d) if d != 0.0 else 0.0
    codes = []
    for x in xs:
        t = f32(f32(x * idv) + 8.5)
        codes.append(min(15, int(math.floor(t))))
    return codes, f16_bits(d)


BLOCK2 = 128


def quant_int2_block(xs):
    """One block of 128 fp32 values -> (codes 0..3, fp16 scale bits, fp16 zero
    bits): d = (max - min) / 3, code = the nearest of the 4 levels (ties
    upward), clamped at 3; the INT2 codec of the oracle ("OSCAR2 KV Cache
    benchmark", compression-ratio table: 36 bytes per 128 values)."""
    assert len(xs) == BLOCK2
    xs = [f32(x) for x in xs]
    mn, mx = min(xs), max(xs)
    d = f32(f32(mx - mn) / 3.0)
    idv = f32(1.0 / d) if d != 0.0 else 0.0
    codes = []
    for x in xs:
        t = f32(f32(f32(x - mn) * idv) + 0.5)
        codes.append(min(3, int(math.floor(t))))
    return codes, f16_bits(d), f16_bits(mn)


def quantize_rows(rows, kind):
    """rows: list of lists (each a multiple of 32 long) -> (codes rows, scale rows)."""
    fn = quant_q8_0_block if kind == "q8_0" else quant_q4_0_block
    codes, scales = [], []
    for row in rows:
        cr, sr = [], []
        for b in range(0, len(row), BLOCK):
            c, s = fn(row[b:b + BLOCK])
            cr += c
            sr.append(s)
        codes.append(cr)
        scales.append(sr)
    return codes, scales


def attention(q, k, v, n_kv, scale, ctx=None):
    """q: [n_q][n_heads][D] floats; k, v: [ctx][n_kv][D] fp32 floats.

    Quantizes k (Q8_0) and v (Q4_0) itself, then computes exact softmax
    attention with causal positions ctx - n_q + i.  Returns (out, lse) as
    nested lists [n_q][n_heads][D] and [n_q][n_heads]."""
    n_q, n_heads, D = len(q), len(q[0]), len(q[0][0])
    ctx = len(k) if ctx is None else ctx
    G = n_heads // n_kv
    khat = [[None] * n_kv for _ in range(ctx)]
    vhat = [[None] * n_kv for _ in range(ctx)]
    for j in range(ctx):
        for g in range(n_kv):
            (kc,), (ks,) = quantize_rows([k[j][g]], "q8_0")
            (vc,), (vs,) = quantize_rows([v[j][g]], "q4_0")
            khat[j][g] = [f16_value(ks[d // BLOCK]) * kc[d] for d in range(D)]
            vhat[j][g] = [f16_value(vs[d // BLOCK]) * (vc[d] - 8) for d in range(D)]
    out, lse = [], []
    for i in range(n_q):
        pos = ctx - n_q + i
        orow, lrow = [], []
        for h in range(n_heads):
            g = h // G
            s = []
            for j in range(pos + 1):
                acc = 0.0
                for d in range(D):
                    acc += f32(q[i][h][d]) * khat[j][g][d]
                s.append(scale * acc)
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            orow.append([sum(w[j] * vhat[j][g][d] for j in range(pos + 1)) / tot for d in range(D)])
            lrow.append(m + math.log(tot))
        out.append(orow)
        lse.append(lrow)
    return out, lse
