"""Float64 CPU oracle for the polynomial-method sketch and the exact streaming path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or helper
with the HIP library; the only thing both sides share is the seeded input
generator in ``synthetic/``, which holds none of the method's arithmetic.

What it follows (the pages are summaries of a theory paper and print no formula,
listing or worked example for this path; the readings taken are listed in the
repository's design notes):

* "Rumo a Limites Estritos para Atenção em Streaming" (gist.science, pt),
  section "Definição do Problema": a query q is answered against the stream of
  key/value pairs seen so far; the quantities wanted are the kernel-density
  normaliser (softmax KDE) and the attention vector.  The naive answer keeps every
  pair.  -> ``exact.exact_attention`` (kernel exp<q, k>, no extra scale).
* Same page, "Metodologia", pillar "O Método Polinomial" (and the French page
  "Vers des Bornes Serrées pour l'Attention en Flux", "Méthodologie", "La Méthode
  Polynomiale"): the head of the exponential kernel is replaced by a truncated
  Taylor expansion and the stream is summarised by its low-degree moments.
  -> ``sketch.sketch_direct`` (the value the method reaches, written as its plain
  definition) and ``sketch.MomentSketch`` (the method's steps: feature map,
  moments, query).
* Same section, closing paragraph on Merge-and-Reduce: summaries of sub-streams
  are merged.  Moments are sums, so the merge is an addition.
  -> ``sketch.MomentSketch.merge``.
* Same section, pillar "Particionamento de Espaço e Recentramento" (shift a
  dense cluster to the origin): with one fixed centre c,
  exp<q,k> = e^{<q,c>} exp<q, k - c>, so the sketch of the shifted keys k - c
  answers with an extra factor e^{<q,c>} on Zhat (it cancels in ohat).
  -> ``sketch.sketch_direct_centered``.
* ``sym``: the same moments kept once per multiset of tensor indices (the moment
  tensors are symmetric), with the query weight q^alpha / alpha!.  The pages
  leave the storage open; this is the symmetric-tensor reading.
  -> ``sym.SymMomentSketch``.
* ``bounds``: the Lagrange form of the Taylor remainder, carried through the sums
  (derived here; the pages state only asymptotic space bounds).
* ``coreset``: the tail of the expansion, e^x - T_p(x), answered from a weighted
  subset of the stream kept by Merge-and-Reduce, each reduce a discrepancy
  halving (the self-balancing walk of Alweiss, Liu and Sawhney on consecutive
  pairs); same section, pillar "Construções de Coreset Baseadas em Discrepância"
  and the closing Merge-and-Reduce paragraph.  The pages name results, not a
  procedure; the readings are in the module header.
  -> ``coreset.MergeReduceCoreset``, ``coreset.halve``, ``coreset.tail_exp``.

Pins: every function here is checked in ``tests/test_oracle.py`` against brute
force on tiny inputs, closed forms, identities and library routines (see the
docstrings there).  No function of this package is "parity unpinned".
"""

from .exact import exact_attention
from .sketch import (taylor_exp, sketch_direct, sketch_direct_centered, MomentSketch,
                     feature_map)
from .sym import SymMomentSketch, multisets, alpha_factorial, sym_features
from .bounds import (taylor_term_bound, kde_relative_bound, attention_abs_bound,
                     measured_radius)
from . import coreset

__all__ = ["exact_attention", "taylor_exp", "sketch_direct", "sketch_direct_centered",
           "MomentSketch",
           "feature_map", "SymMomentSketch", "multisets", "alpha_factorial",
           "sym_features", "taylor_term_bound", "kde_relative_bound",
           "attention_abs_bound", "measured_radius", "coreset"]
