"""Seeded synthetic workloads for the polynomial-sketch and exact-attention paths.

This package only draws random inputs (keys, values, queries) with the shapes and
value distributions of the five workloads listed below.  It holds none of the
method's arithmetic: no feature map, no moment, no kernel value.  Both the float64
oracle (``oracle/``) and the GPU library's tests and benchmark take their inputs
from here, so the two sides always see the same fp32 bytes.

The stream model (a sequence of key/value pairs read in order, answered at a query
q) is the one stated in "Rumo a Limites Estritos para Atenção em Streaming"
(gist.science, pt), section "Definição do Problema"; the radius r of keys and
queries is how those pages set the temperature regime (same page, regimes 1 and 2).
"""

from .configs import WORKLOADS, Workload, workload
from .generate import generate, generate_head, vectors, values

__all__ = ["WORKLOADS", "Workload", "workload", "generate", "generate_head",
           "vectors", "values"]
