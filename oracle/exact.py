"""Exact exp-kernel density and softmax attention, float64 (test infrastructure only).

Follows "Rumo a Limites Estritos para Atenção em Streaming" (gist.science, pt),
"Definição do Problema": a query q against all n stored key/value pairs.  With the
kernel exp<q, k> (the pages set the temperature through the radius of keys and
queries, so no 1/sqrt(d) factor is applied):

    Z(q) = sum_i exp(<q, k_i>)                  (the KDE normaliser)
    o(q) = sum_i exp(<q, k_i>) v_i / Z(q)       (the attention output)

It is evaluated in the usual max-shifted form, which is the same number:
mu = max_i s_i, Z = e^mu * sum_i e^(s_i - mu), o = sum_i e^(s_i - mu) v_i /
sum_i e^(s_i - mu).  An empty stream gives Z = 0 and o = 0/0 = NaN.
"""

import numpy as np


def exact_attention(K, V, Q, max_block_entries=1 << 24):
    """(out [m, dv], Z [m]) in float64 for one head.

    K [n, d], V [n, dv], Q [m, d]: any real arrays; they are read as float64.
    Queries are processed in blocks so that a block's score matrix holds at most
    ``max_block_entries`` numbers.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    n, m, dv = K.shape[0], Q.shape[0], V.shape[1]
    out = np.empty((m, dv))
    Z = np.empty(m)
    if n == 0:
        Z[:] = 0.0
        out[:] = np.nan
        return out, Z
    bq = max(1, max_block_entries // max(n, 1))
    for q0 in range(0, m, bq):
        q1 = min(m, q0 + bq)
        s = Q[q0:q1] @ K.T                      # scores <q, k_i>
        mu = s.max(axis=1, keepdims=True)
        w = np.exp(s - mu)                      # e^(s_i - mu)
        l = w.sum(axis=1)
        a = w @ V
        Z[q0:q1] = np.exp(mu[:, 0]) * l
        out[q0:q1] = a / l[:, None]
    return out, Z
