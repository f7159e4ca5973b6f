"""A second, independent implementation of the layer in scalar Python loops.

It exists only to pin the fp64 oracle on tiny shapes: it shares no code with
the oracle (plain `math`, nested lists, one scalar at a time) so a dropped
term, a wrong sign or a transposed index in either shows up as a mismatch.

Same readings as the oracle: window W counts keys including the query, RoPE
pairs dim i with i + r/2 in the first r dims at frequency theta^(-2i/r),
Q head h reads KV head h // G, out = sigmoid(gate) * attention.
"""
import math


def rotate(vec, pos, theta, r):
    out = list(vec)
    if theta == 0 or r == 0:
        return out
    half = r // 2
    for i in range(half):
        w = theta ** (-2.0 * i / r)
        a = pos * w
        c, s = math.cos(a), math.sin(a)
        x, y = vec[i], vec[i + half]
        out[i] = x * c - y * s
        out[i + half] = y * c + x * s
    return out


def attend(qvec, keys, values, scale):
    """keys/values: lists of vectors (already rotated keys)."""
    scores = [scale * sum(a * b for a, b in zip(qvec, kk)) for kk in keys]
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    tot = sum(e)
    d = len(values[0])
    out = [0.0] * d
    for w, vv in zip(e, values):
        for c in range(d):
            out[c] += (w / tot) * vv[c]
    return out


def gate_value(g):
    return 1.0 / (1.0 + math.exp(-g))


def prefill(q, k, v, gate, sliding, window, G, theta, fraction, scale):
    """q[b][t][h][d], k/v[b][t][kv][d], gate[b][t][h] nested lists.
    fraction of head_dim rotated; scale None means 1/sqrt(head_dim)."""
    B, T, Hq = len(q), len(q[0]), len(q[0][0])
    D = len(q[0][0][0])
    r = int(round(fraction * D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    y = []
    for b in range(B):
        yb = []
        for i in range(T):
            yi = []
            for h in range(Hq):
                kv = h // G
                qi = rotate(q[b][i][h], i, theta, r)
                keys, vals = [], []
                for j in range(T):
                    if j > i:
                        continue
                    if sliding and i - j >= window:
                        continue
                    keys.append(rotate(k[b][j][kv], j, theta, r))
                    vals.append(v[b][j][kv])
                a = attend(qi, keys, vals, scale)
                gv = gate_value(gate[b][i][h])
                yi.append([gv * x for x in a])
            yb.append(yi)
        y.append(yb)
    return y
