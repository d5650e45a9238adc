"""Pure-Python brute-force attention for tiny inputs (test helper).

Triple loops with math.fsum, independent of numpy's matmul and of the
oracle's vectorised code.  Used only to pin the oracle.
"""
import math


def fwd(q, k, v, allowed, scale):
    """q: [Tq][Hq][d] nested lists; allowed(h, i, j) -> bool.  Returns O, LSE."""
    Tq, Hq, d = len(q), len(q[0]), len(q[0][0])
    Tk, Hkv = len(k), len(k[0])
    rep = Hq // Hkv
    O = [[[0.0] * d for _ in range(Hq)] for _ in range(Tq)]
    L = [[-math.inf] * Tq for _ in range(Hq)]
    for h in range(Hq):
        g = h // rep
        for i in range(Tq):
            js = [j for j in range(Tk) if allowed(h, i, j)]
            if not js:
                continue
            s = {j: scale * math.fsum(q[i][h][c] * k[j][g][c] for c in range(d)) for j in js}
            m = max(s.values())
            e = {j: math.exp(s[j] - m) for j in js}
            l = math.fsum(e.values())
            for c in range(d):
                O[i][h][c] = math.fsum(e[j] / l * v[j][g][c] for j in js)
            L[h][i] = m + math.log(l)
    return O, L


def bwd(q, k, v, do, allowed, scale):
    """Backward of sum(dO * O) with the brute-force forward's own O and LSE."""
    Tq, Hq, d = len(q), len(q[0]), len(q[0][0])
    Tk, Hkv = len(k), len(k[0])
    rep = Hq // Hkv
    O, L = fwd(q, k, v, allowed, scale)
    dq = [[[0.0] * d for _ in range(Hq)] for _ in range(Tq)]
    dk_terms = [[[[] for _ in range(d)] for _ in range(Hkv)] for _ in range(Tk)]
    dv_terms = [[[[] for _ in range(d)] for _ in range(Hkv)] for _ in range(Tk)]
    for h in range(Hq):
        g = h // rep
        for i in range(Tq):
            js = [j for j in range(Tk) if allowed(h, i, j)]
            if not js:
                continue
            D = math.fsum(do[i][h][c] * O[i][h][c] for c in range(d))
            for j in js:
                s = scale * math.fsum(q[i][h][c] * k[j][g][c] for c in range(d))
                p = math.exp(s - L[h][i])
                dp = math.fsum(do[i][h][c] * v[j][g][c] for c in range(d))
                ds = p * (dp - D)
                for c in range(d):
                    dq[i][h][c] += scale * ds * k[j][g][c]
                    dk_terms[j][g][c].append(scale * ds * q[i][h][c])
                    dv_terms[j][g][c].append(p * do[i][h][c])
    dk = [[[math.fsum(dk_terms[j][g][c]) for c in range(d)] for g in range(Hkv)] for j in range(Tk)]
    dv = [[[math.fsum(dv_terms[j][g][c]) for c in range(d)] for g in range(Hkv)] for j in range(Tk)]
    return dq, dk, dv
