"""High-precision brute-force attention for tiny inputs (a pin for the oracle).

Independent of the float64 oracle: every score, exponential, sum and
quotient is taken element by element in 50-digit decimal arithmetic, with
explicit loops and no matrix routine.  Definition followed: page
"Self-Attention, CUDA kernels and FlashAttention", section 1 (scaled scores,
row softmax, product with V); causal reading: row i sees keys 0..i.
"""
from __future__ import annotations

from decimal import Decimal, localcontext


def attention_bruteforce(q, k, v, scale, causal):
    """q: [Nq][d], k: [Nk][d], v: [Nk][dv] nested sequences of floats.

    Returns (O as list of lists of float, LSE as list of float).
    """
    with localcontext() as ctx:
        ctx.prec = 50
        sc = Decimal(float(scale))
        o_rows, lse = [], []
        for i, qi in enumerate(q):
            visible = [j for j in range(len(k)) if not (causal and j > i)]
            s = {}
            for j in visible:
                acc = Decimal(0)
                for a, b in zip(qi, k[j]):
                    acc += Decimal(float(a)) * Decimal(float(b))
                s[j] = acc * sc
            m = max(s.values())
            w = {j: (s[j] - m).exp() for j in visible}
            z = sum(w.values(), Decimal(0))
            row = []
            for c in range(len(v[0])):
                num = Decimal(0)
                for j in visible:
                    num += w[j] * Decimal(float(v[j][c]))
                row.append(float(num / z))
            o_rows.append(row)
            lse.append(float(m + z.ln()))
        return o_rows, lse
