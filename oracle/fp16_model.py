"""Round-after-operation float16 model of a split reduction (test
infrastructure only).

M4.5 §0x02H: the same exact reduction target, evaluated with every operation
rounded to float16, gives tree-dependent results.  Each value is its own
one-element split; merges follow ``merge_state`` (M4.5 §0x02B, §0x02C) with
each arithmetic result rounded to float16.
"""
import numpy as np

f16 = np.float16


def _state(score, value):
    return (f16(score), f16(1.0), f16(value))        # (m, l, u) of one row


def _merge16(a, b):
    ma, la, ua = a
    mb, lb, ub = b
    m = max(ma, mb)
    alpha = f16(np.exp(f16(ma - m)))
    beta = f16(np.exp(f16(mb - m)))
    l = f16(f16(alpha * la) + f16(beta * lb))
    u = f16(f16(alpha * ua) + f16(beta * ub))
    return (m, l, u)


def sequential(scores, values, order=None):
    idx = list(order) if order is not None else list(range(len(scores)))
    acc = _state(scores[idx[0]], values[idx[0]])
    for i in idx[1:]:
        acc = _merge16(acc, _state(scores[i], values[i]))
    return float(acc[2] / acc[1])


def balanced(scores, values):
    level = [_state(s, v) for s, v in zip(scores, values)]
    while len(level) > 1:
        nxt = [_merge16(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    m, l, u = level[0]
    return float(u / l)
