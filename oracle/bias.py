"""Auxiliary-loss-free bias update.

Source: V3 notes §4 -- after every training step the bias of an overloaded
expert is lowered and that of an underloaded expert raised; §4.1 gives the
update speed gamma = 0.001 (for the first 14.3T tokens); the evolution post
(auxiliary-loss-free section) states the same rule.

Reading taken (the update formula was lost from the page): a fixed step of
gamma in the direction of sign(mean load - load), with the comparison done in
integers as sign(T*K - E*counts[e]) so that it is exact; sign(0) = 0; the loads
are the counts of the current call's T tokens; the result is rounded to
float32:  b[e] = fl32(b[e] + fl32(gamma) * sign(T*K - E*counts[e])).
"""

import numpy as np


def update_bias(bias, counts, n_tokens: int, top_k: int, gamma: float = 0.001):
    b = np.asarray(bias, dtype=np.float32)
    c = np.asarray(counts, dtype=np.int64)
    n_experts = b.shape[0]
    direction = np.sign(np.int64(n_tokens) * top_k - np.int64(n_experts) * c)
    step = np.float32(gamma) * direction.astype(np.float32)   # exact: +-gamma or 0
    return (b + step).astype(np.float32)
