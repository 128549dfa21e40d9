"""The five synthetic workloads (shapes, sizes and value distributions).

Each workload is a stream of n key/value pairs per head, answered at m queries per
head.  Sizes are plain data; D = 1 + d + ... + d^p is the feature count of a
degree-p Kronecker feature map and is listed only so that callers can size buffers.

Distribution names (all drawn in float64, then cast to float32):
  sphere        r * g / |g|,  g ~ N(0, I_d)                 (uniform on the r-sphere)
  gauss_rescale g * r / max_i |g_i| over the whole set       (one factor per set)
  gauss_clip    g * min(1, r / |g|) per vector
  uniform       U[-1, 1] per coordinate
  normal        N(0, 1) per coordinate
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    ident: int
    name: str
    d: int          # key / query dimension
    dv: int         # value dimension
    p: int          # Taylor degree of the sketch
    n: int          # keys per head in the whole stream
    m: int          # queries per head
    h: int          # independent heads
    key_dist: str
    key_r: float
    val_dist: str
    chunk: int      # keys per update call (0: the whole stream in one call)
    substreams: int  # sub-streams ingested into separate sketches, then merged
    seed: int = 0

    @property
    def D(self) -> int:
        return sum(self.d ** j for j in range(self.p + 1))

    def scaled(self, n=None, m=None, h=None, chunk=None, substreams=None):
        """The same workload at other sizes (used for the small parity cases)."""
        kw = {}
        if n is not None:
            kw["n"] = n
        if m is not None:
            kw["m"] = m
        if h is not None:
            kw["h"] = h
        if chunk is not None:
            kw["chunk"] = chunk
        if substreams is not None:
            kw["substreams"] = substreams
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny_high_temp_d4_p3", d=4, dv=4, p=3, n=4096, m=64, h=1,
                key_dist="sphere", key_r=1.0, val_dist="uniform",
                chunk=0, substreams=1),
    2: Workload(2, "sketch_d16_p4_n64k", d=16, dv=16, p=4, n=65536, m=1024, h=1,
                key_dist="sphere", key_r=1.0, val_dist="uniform",
                chunk=4096, substreams=1),
    3: Workload(3, "sketch_d32_p3_n1m_merge4", d=32, dv=32, p=3, n=1048576, m=4096,
                h=1, key_dist="gauss_rescale", key_r=1.5, val_dist="normal",
                chunk=4096, substreams=4),
    4: Workload(4, "decode_32heads_d64_p2_n128k", d=64, dv=64, p=2, n=131072, m=256,
                h=32, key_dist="gauss_clip", key_r=0.75, val_dist="normal",
                chunk=0, substreams=1),
    5: Workload(5, "low_temp_d8_p6_r2", d=8, dv=8, p=6, n=262144, m=2048, h=1,
                key_dist="sphere", key_r=2.0, val_dist="uniform",
                chunk=0, substreams=1),
}


def workload(ident: int) -> Workload:
    return WORKLOADS[int(ident)]
