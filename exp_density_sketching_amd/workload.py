"""Drive one workload through the C ABI: chunked ingest, sub-stream merges, query,
exact attention.  Orchestration only (the order of calls); no arithmetic here.

Ingest protocol of a workload with ``chunk`` c and ``substreams`` S: the n keys of
each head are cut into S contiguous sub-streams, each ingested into its own sketch
in calls of c keys (c = 0: one call per sub-stream); then sketches 1..S-1 are
merged into sketch 0 in order (the Merge step of Merge-and-Reduce, "Rumo a Limites
Estritos para Atenção em Streaming", "Metodologia", closing paragraph).
"""

from . import _binding as B


def ingest(w, K, V, sketches=None, layout="full"):
    """Ingest K [h, n, d], V [h, n, dv] per the workload's protocol.

    ``sketches``: optional list of S pre-created (and reset) Sketch handles;
    otherwise S new ones of the given storage ``layout`` ("full" or "sym").
    Returns the sketch holding the whole stream (sketch 0) and the list.
    """
    S = max(1, w.substreams)
    n = K.shape[1]
    if sketches is None:
        sketches = [B.sketch_create(w.d, w.dv, w.p, w.h, layout) for _ in range(S)]
    bounds = [n * i // S for i in range(S + 1)]
    for i in range(S):
        lo, hi = bounds[i], bounds[i + 1]
        step = w.chunk if w.chunk > 0 else max(hi - lo, 1)
        for c0 in range(lo, hi, step):
            c1 = min(hi, c0 + step)
            # a chunk of a multi-head stream is strided; the C ABI takes [h][n][d]
            B.sketch_update(sketches[i], K[:, c0:c1].contiguous(), V[:, c0:c1].contiguous())
    for i in range(1, S):
        B.sketch_merge(sketches[0], sketches[i])
    return sketches[0], sketches


def run_sketch(w, K, V, Q, layout="full"):
    """Whole sketch path of a workload: (ohat [h, m, dv], Zhat [h, m], sketch)."""
    sk, _ = ingest(w, K, V, layout=layout)
    out, Z = B.sketch_query(sk, Q)
    return out, Z, sk
