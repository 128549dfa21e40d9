// Tail coreset kernels: discrepancy halving of point blocks (the "reduce" of
// Merge-and-Reduce) and the tail sums of the kept points.
//
// Source: "Rumo a Limites Estritos para Atenção em Streaming", "Metodologia" >
// "1. Limites Superiores Algorítmicos": coresets built with discrepancy theory
// serve the tail of the exp kernel's expansion, the moments serve its head, and
// Merge-and-Reduce assembles the stream.  The pages give no procedure; the one
// used is the self-balancing walk of Alweiss, Liu and Sawhney (STOC 2021) on
// consecutive pairs, in the feature space of the tail kernel
//     <u(x), u(y)> = R_p(<k_x, k_y>) (1 + <v_x, v_y>),  R_p(x) = e^x - T_p(x),
// with uniforms from SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) used as a
// counter-based generator.
//
// One reduce merges an older block A and a newer block C of B points each (per
// head) into 2B points [A; C] read as B pairs (2t, 2t + 1), and keeps one point of
// each pair.  It runs as two launches over a batch of independent reduces:
//   cs_gram_kernel  -- the pair Gram matrix D[t][s] = <f_t, f_s> (fp64), f_t =
//                      u(x_2t) - u(x_2t+1), upper triangle in 32 x 32 pair tiles;
//   cs_walk_kernel  -- the walk over the pairs in order (fp64), then the kept rows
//                      copied into the output block.
// The walk's decisions are integers decided in float64, the same precision as
// the float64 reference, so the kept sets agree unless a uniform falls within
// rounding of its threshold.
#pragma once

#include "sk_common.h"

#define CS_MAXB 2048       // largest block (points per head)
#define CS_MAXOPS 32       // reduces per launch
#define CS_MAXSEG 64       // point segments of a tail query (buffer + levels)
#define CS_TP 32           // pairs per Gram tile side (64 points)
#define CS_QT 128          // queries per tail-query workgroup
#define CS_PT 32           // points per tail-query stage

// A block of points of every head: rows of head hd start at K + hd * hsK.
struct CsRef {
  const float* K;
  const float* V;
  long long hsK, hsV;      // head strides in floats
};

// One reduce: blocks a (older) and b (newer) -> out (B kept rows per head).
struct CsOp {
  CsRef a, b;
  float* outK;             // [h][B][d]
  float* outV;             // [h][B][dv]
  long long serial;        // reduce number of the handle (uniform counters)
};

struct CsOps {
  CsOp op[CS_MAXOPS];
  int n;
};

// Tail-query segments: the partial buffer (weight 1) and the level blocks
// (weight 2^l), each cut into slices of CS_SLICE points.
struct CsSeg {
  const float* K;
  const float* V;
  long long hsK, hsV;
  int count;               // points per head
  int slice0;              // first global slice index of the segment
  float w;
};
struct CsSegs {
  CsSeg s[CS_MAXSEG];
  int n;
  int nslices;
};
#define CS_SLICE 512

#define CS_NINV 512       // entries of the 1/j table (float64; entry 0 unused)

// SplitMix64: output number `counter` of the sequence whose state starts at seed.
__device__ __forceinline__ unsigned long long cs_splitmix64(unsigned long long seed,
                                                            unsigned long long counter) {
  unsigned long long z = seed + (counter + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ double cs_uniform(unsigned long long seed,
                                             unsigned long long counter) {
  return (double)(cs_splitmix64(seed, counter) >> 11) * 0x1.0p-53;
}

// R_p(x) = sum_{j > p} x^j / j! in float64 for N values x at once: the series
// (terms by the ratio x / j until they stop changing the sum, past the largest
// term), unless its largest term exceeds e^x + sum_{j <= p} |x|^j / j!, where
// e^x - T_p(x) rounds less.  The N series advance together, one 1/j per step for
// all, so their dependent chains overlap; a value whose series has stopped is
// left as it is, so each result is the one its own series alone would give.
// Sums and products are rounded one at a time (no fused multiply-add), as in a
// plain float64 evaluation.
template <int N>
__device__ inline void cs_tail_exp64_n(const double (&x)[N], int p,
                                       const double* __restrict__ cs_inv, double (&out)[N]) {
#pragma clang fp contract(off)
  double term[N], acc[N], big[N];
  bool live[N];
#pragma unroll
  for (int e = 0; e < N; ++e) term[e] = 1.0;
  for (int j = 1; j <= p + 1; ++j) {
    const double ij = cs_inv[j];
#pragma unroll
    for (int e = 0; e < N; ++e) term[e] *= x[e] * ij;
  }
  bool any = false;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    acc[e] = term[e];
    big[e] = fabs(term[e]);
    live[e] = fabs(x[e]) <= 40.0;
    any = any || live[e];
  }
  for (int j = p + 2; any && j < p + 400 && j < CS_NINV; ++j) {
    const double ij = cs_inv[j];
    any = false;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      if (live[e]) {
        term[e] *= x[e] * ij;
        const double nw = acc[e] + term[e];
        big[e] = fmax(big[e], fabs(term[e]));
        if (nw == acc[e] && (double)j > 2.0 * fabs(x[e])) live[e] = false;
        else acc[e] = nw;
        any = any || live[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const double ax = fabs(x[e]);
    double hm = 1.0, t = 1.0;
    for (int i = 1; i <= p; ++i) {
      t *= ax * cs_inv[i];
      hm += t;
    }
    double r = acc[e];
    // (big <= hm already decides for the series without e^x: e^x > 0)
    if (!(ax <= 40.0 && big[e] <= hm)) {
      const double ex = exp(x[e]);
      if (!(ax <= 40.0 && big[e] <= ex + hm)) {
        // e^x - T_p(x), T_p by Horner from the top
        double tp = 1.0;
        for (int i = p; i >= 1; --i) tp = 1.0 + x[e] * cs_inv[i] * tp;
        r = ex - tp;
      }
    }
    out[e] = r;
  }
}

// Pair Gram matrix of a batch of reduces.  Grid: (reduce, head, upper tile) with
// the tile index fastest; 256 threads, thread (ti, tj) = (tid / 16, tid % 16)
// owns points 4 ti .. 4 ti + 3 of the tile's rows (pairs 2 ti, 2 ti + 1) and
// 4 tj .. 4 tj + 3 of its columns, accumulates their 16 key and value dot
// products in float64 over feature chunks of 32 staged in LDS, and writes the 4
// pair entries.  D: [reduce][head][B][B] float64.
__global__ __launch_bounds__(256)
void cs_gram_kernel(CsOps ops, int B, int d, int dv, int p, int h,
                    const double* __restrict__ inv, double* __restrict__ Dws) {
  __shared__ double Rs[32][64];
  __shared__ double Cs[32][64];
  const int tid = threadIdx.x;
  const int nt = B / CS_TP;
  const int ntiles = nt * (nt + 1) / 2;
  const long long lg = blockIdx.x;
  const int tile = (int)(lg % ntiles);
  const int head = (int)((lg / ntiles) % h);
  const int oi = (int)(lg / ((long long)ntiles * h));
  // upper tile (tr, tc), tc >= tr, rows in order
  int tr = 0, rem = tile;
  while (rem >= nt - tr) {
    rem -= nt - tr;
    ++tr;
  }
  const int tc = tr + rem;
  const CsOp& O = ops.op[oi];
  // merged point index i -> row of block a (i < B) or b
  auto rowptr = [&](int i, bool val) -> const float* {
    const CsRef& R = (i < B) ? O.a : O.b;
    const int r = (i < B) ? i : i - B;
    return val ? R.V + head * R.hsV + (long long)r * dv : R.K + head * R.hsK + (long long)r * d;
  };
  const int ti = tid >> 4, tj = tid & 15;
  const int r0 = tr * 2 * CS_TP, c0 = tc * 2 * CS_TP;   // first merged point of rows / cols
  double kd[4][4], vd[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) kd[a][b] = vd[a][b] = 0.0;
  for (int part = 0; part < 2; ++part) {
    const int width = part == 0 ? d : dv;
    for (int f0 = 0; f0 < width; f0 += 32) {
      const int fw = min(32, width - f0);
      // stage 64 row points and 64 column points, features f0 .. f0 + fw - 1
      __syncthreads();
      {
        const int pt = tid >> 2, q = tid & 3;       // 8 features per thread
        for (int k = 0; k < 8; k += 4) {
          const int f = q * 8 + k;
          if (f < fw) {
            const float4 x = *reinterpret_cast<const float4*>(rowptr(r0 + pt, part == 1) + f0 + f);
            const float4 y = *reinterpret_cast<const float4*>(rowptr(c0 + pt, part == 1) + f0 + f);
            Rs[f][pt] = x.x; Rs[f + 1][pt] = x.y; Rs[f + 2][pt] = x.z; Rs[f + 3][pt] = x.w;
            Cs[f][pt] = y.x; Cs[f + 1][pt] = y.y; Cs[f + 2][pt] = y.z; Cs[f + 3][pt] = y.w;
          }
        }
      }
      __syncthreads();
      for (int f = 0; f < fw; ++f) {
        double rv[4], cv[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          rv[a] = Rs[f][4 * ti + a];
          cv[a] = Cs[f][4 * tj + a];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            if (part == 0) kd[a][b] = fma(rv[a], cv[b], kd[a][b]);
            else vd[a][b] = fma(rv[a], cv[b], vd[a][b]);
          }
      }
    }
  }
  double g[4][4], xs[16], rs[16];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) xs[4 * a + b] = kd[a][b];
  cs_tail_exp64_n<16>(xs, p, inv, rs);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) g[a][b] = rs[4 * a + b] * (1.0 + vd[a][b]);
  double* Dh = Dws + ((long long)oi * h + head) * (long long)B * B;
#pragma unroll
  for (int P = 0; P < 2; ++P)
#pragma unroll
    for (int Qq = 0; Qq < 2; ++Qq) {
      const int t = tr * CS_TP + 2 * ti + P;
      const int s = tc * CS_TP + 2 * tj + Qq;
      Dh[(long long)t * B + s] = g[2 * P][2 * Qq] - g[2 * P][2 * Qq + 1] -
                                 g[2 * P + 1][2 * Qq] + g[2 * P + 1][2 * Qq + 1];
    }
}

// The walk of one reduce and one head (one workgroup of 256 threads), then the
// kept rows.  Pairs go in blocks of 64: the block's 64 x 64 upper Gram entries go
// to LDS, wave 0 decides the 64 pairs in order (lane j holds <psi, f_j> and adds
// e_i D[i][j] after pair i's decision, taken by lane i and read by every lane),
// then all threads add the block's 64 terms, in pair order, to the running
// <psi, f_s> of every later pair.  Every <psi, f_s> thus gets its terms in pair
// order, as in the sequential walk.  Decision of pair t: P = (1 - alpha/c)/2
// clamped to [0, 1] (1/2 when c = 0), U from counter (serial * H + head) * B + t,
// e = +1 (keep point 2t + 1) when U < P, else -1 (keep point 2t).
__global__ __launch_bounds__(256)
void cs_walk_kernel(CsOps ops, int B, int d, int dv, int h, const double* __restrict__ Dws,
                    double c0, unsigned long long seed) {
  __shared__ double alpha[CS_MAXB];
  __shared__ double blk[64][65];
  __shared__ signed char eps[CS_MAXB];
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int head = blockIdx.x % h;
  const int oi = blockIdx.x / h;
  const CsOp& O = ops.op[oi];
  const double* Dh = Dws + ((long long)oi * h + head) * (long long)B * B;
  // threshold c = c0 * max_t |f_t|^2
  double mx = 0.0;
  for (int t = tid; t < B; t += 256) mx = fmax(mx, Dh[(long long)t * B + t]);
  red[tid] = mx;
  for (int t = tid; t < B; t += 256) alpha[t] = 0.0;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] = fmax(red[tid], red[tid + st]);
    __syncthreads();
  }
  const double c = c0 * red[0];
  for (int t0 = 0; t0 < B; t0 += 64) {
    for (int e = tid; e < 64 * 64; e += 256) {
      const int i = e >> 6, j = e & 63;
      blk[i][j] = (j > i) ? Dh[(long long)(t0 + i) * B + t0 + j] : 0.0;
    }
    __syncthreads();
    if (tid < 64) {
      const unsigned long long ctr =
          ((unsigned long long)O.serial * (unsigned long long)h + (unsigned long long)head) *
              (unsigned long long)B + (unsigned long long)(t0 + lane);
      const double U = cs_uniform(seed, ctr);
      double a = alpha[t0 + lane];
      int mine = 0;
      for (int i = 0; i < 64; ++i) {
        const double P = c > 0.0 ? fmin(1.0, fmax(0.0, 0.5 * (1.0 - a / c))) : 0.5;
        const int dec = (U < P) ? 1 : -1;
        const int e = __shfl(dec, i, 64);
        if (lane == i) mine = e;
        if (lane > i) a = fma((double)e, blk[i][lane], a);
      }
      alpha[t0 + lane] = a;
      eps[t0 + lane] = (signed char)mine;
    }
    __syncthreads();
    for (int s = t0 + 64 + tid; s < B; s += 256) {
      double x = alpha[s];
      for (int i = 0; i < 64; ++i) x = fma((double)eps[t0 + i], Dh[(long long)(t0 + i) * B + s], x);
      alpha[s] = x;
    }
    __syncthreads();
  }
  // kept rows: pair t keeps merged point 2t + 1 (e = +1) or 2t
  float* oK = O.outK + (long long)head * B * d;
  float* oV = O.outV + (long long)head * B * dv;
  const int d4 = d / 4, dv4 = dv / 4;
  for (int e = tid; e < B * (d4 + dv4); e += 256) {
    const int t = e / (d4 + dv4), c4 = e - t * (d4 + dv4);
    const int i = 2 * t + (eps[t] > 0 ? 1 : 0);
    const CsRef& R = (i < B) ? O.a : O.b;
    const int r = (i < B) ? i : i - B;
    if (c4 < d4)
      reinterpret_cast<float4*>(oK + (long long)t * d)[c4] =
          reinterpret_cast<const float4*>(R.K + head * R.hsK + (long long)r * d)[c4];
    else
      reinterpret_cast<float4*>(oV + (long long)t * dv)[c4 - d4] =
          reinterpret_cast<const float4*>(R.V + head * R.hsV + (long long)r * dv)[c4 - d4];
  }
}

// Copies rows [r0, r0 + rows) of every head of a (K, V) block into rows [w0, ...)
// of a library block of B rows per head.
__global__ __launch_bounds__(256)
void cs_copy_rows_kernel(const float* __restrict__ K, const float* __restrict__ V,
                         long long hsK, long long hsV, long long r0, int rows, int d, int dv,
                         float* __restrict__ oK, float* __restrict__ oV, int B, int w0, int h) {
  const int d4 = d / 4, dv4 = dv / 4, per = rows * (d4 + dv4);
  const long long total = (long long)per * h;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (long long)gridDim.x * 256) {
    const int head = (int)(e / per);
    const int x = (int)(e - (long long)head * per);
    const int r = x / (d4 + dv4), c4 = x - r * (d4 + dv4);
    if (c4 < d4)
      reinterpret_cast<float4*>(oK + ((long long)head * B + w0 + r) * d)[c4] =
          reinterpret_cast<const float4*>(K + head * hsK + (r0 + r) * d)[c4];
    else
      reinterpret_cast<float4*>(oV + ((long long)head * B + w0 + r) * dv)[c4 - d4] =
          reinterpret_cast<const float4*>(V + head * hsV + (r0 + r) * dv)[c4 - d4];
  }
}

// R_p(x) in float32 for the tail sums: the series for |x| <= 16 (terms by the
// ratio x / j until they stop changing the sum past the largest one), else
// e^x - T_p(x).
__device__ inline float cs_tail_exp32(float x, int p, const float* __restrict__ inv) {
  const float ax = fabsf(x);
  if (ax > 16.f) {
    float tp = 1.f;
    for (int i = p; i >= 1; --i) tp = 1.f + x * inv[i] * tp;
    return expf(x) - tp;
  }
  float term = 1.f;
  for (int j = 1; j <= p + 1; ++j) term *= x * inv[j];
  float acc = term;
  for (int j = p + 2; j < p + 80; ++j) {
    term *= x * inv[j];
    const float nw = acc + term;
    if (nw == acc && (float)j > 2.f * ax) break;
    acc = nw;
  }
  return acc;
}

// Tail sums of a query tile against one slice of points: partial [1 + dv] per
// (head, query, slice): sum_s w R_p(<q, k_s>) [1, v_s].  One thread per query
// (its query in registers), points staged CS_PT at a time in LDS.
template <int D, int DV>
__global__ __launch_bounds__(CS_QT)
void cs_tail_kernel(const float* __restrict__ Q, long long m, int p, CsSegs segs,
                    float* __restrict__ parts) {
  __shared__ float Ks[CS_PT][D];
  __shared__ float Vs[CS_PT][DV];
  __shared__ float inv[96];
  const int tid = threadIdx.x;
  const int qt = blockIdx.x, slice = blockIdx.y, head = blockIdx.z;
  for (int j = tid; j < 96; j += CS_QT) inv[j] = j == 0 ? 1.f : 1.f / (float)j;
  // the slice's segment
  int sg = 0;
  while (sg + 1 < segs.n && segs.s[sg + 1].slice0 <= slice) ++sg;
  const CsSeg S = segs.s[sg];
  const int p0 = (slice - S.slice0) * CS_SLICE;
  const int np = min(CS_SLICE, S.count - p0);
  const long long q = (long long)qt * CS_QT + tid;
  const bool qv = q < m;
  float qr[D];
  const float* Qh = Q + ((long long)head * m + (qv ? q : 0)) * D;
#pragma unroll
  for (int a = 0; a < D; a += 4) {
    const float4 x = *reinterpret_cast<const float4*>(Qh + a);
    qr[a] = x.x; qr[a + 1] = x.y; qr[a + 2] = x.z; qr[a + 3] = x.w;
  }
  float z = 0.f, acc[DV];
#pragma unroll
  for (int c = 0; c < DV; ++c) acc[c] = 0.f;
  const float* Kb = S.K + head * S.hsK + (long long)p0 * D;
  const float* Vb = S.V + head * S.hsV + (long long)p0 * DV;
  for (int s0 = 0; s0 < np; s0 += CS_PT) {
    const int ns = min(CS_PT, np - s0);
    __syncthreads();
    for (int e = tid; e < CS_PT * (D / 4); e += CS_QT) {
      const int r = e / (D / 4), c4 = e - r * (D / 4);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < ns) x = reinterpret_cast<const float4*>(Kb + (long long)(s0 + r) * D)[c4];
      *reinterpret_cast<float4*>(&Ks[r][4 * c4]) = x;
    }
    for (int e = tid; e < CS_PT * (DV / 4); e += CS_QT) {
      const int r = e / (DV / 4), c4 = e - r * (DV / 4);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < ns) x = reinterpret_cast<const float4*>(Vb + (long long)(s0 + r) * DV)[c4];
      *reinterpret_cast<float4*>(&Vs[r][4 * c4]) = x;
    }
    __syncthreads();
    for (int j = 0; j < ns; ++j) {
      float s = 0.f;
#pragma unroll
      for (int a = 0; a < D; ++a) s = fmaf(qr[a], Ks[j][a], s);
      const float r = S.w * cs_tail_exp32(s, p, inv);
      z += r;
#pragma unroll
      for (int c = 0; c < DV; ++c) acc[c] = fmaf(r, Vs[j][c], acc[c]);
    }
  }
  if (qv) {
    float* P = parts + (((long long)head * m + q) * segs.nslices + slice) * (1 + DV);
    P[0] = z;
#pragma unroll
    for (int c = 0; c < DV; ++c) P[1 + c] = acc[c];
  }
}

// Adds the tail to the head answer in place: per (head, query), the slice
// partials in slice order, then Z = Zh + tZ, out = (out Zh + tN) / Z.
__global__ __launch_bounds__(256)
void cs_tail_combine(const float* __restrict__ parts, int nslices, long long m, int dv,
                     float* __restrict__ out, float* __restrict__ Z) {
  __shared__ float tz;
  const long long hq = blockIdx.x;
  const int c = threadIdx.x;
  const float* P = parts + hq * (long long)nslices * (1 + dv);
  float s = 0.f;
  if (c <= dv)
    for (int k = 0; k < nslices; ++k) s += P[(long long)k * (1 + dv) + c];
  if (c == 0) tz = s;
  __syncthreads();
  const float zh = Z[hq];
  const float zt = zh + tz;
  if (c >= 1 && c <= dv) out[hq * dv + c - 1] = (out[hq * dv + c - 1] * zh + s) / zt;
  __syncthreads();
  if (c == 0) Z[hq] = zt;
}

// Canonical export of the points: per head [points][d], [points][dv], [points]
// (the buffer first, then the levels by increasing level).
__global__ __launch_bounds__(256)
void cs_export_kernel(CsSegs segs, int d, int dv, int h, long long npts,
                      float* __restrict__ K, float* __restrict__ V, float* __restrict__ W) {
  const int per = d + dv + 1;
  const long long total = (long long)h * npts * per;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (long long)gridDim.x * 256) {
    const int head = (int)(e / (npts * per));
    const long long x = e - (long long)head * npts * per;
    const long long pt = x / per;
    const int c = (int)(x - pt * per);
    int sg = 0;
    long long base = 0;
    while (sg < segs.n && pt >= base + segs.s[sg].count) {
      base += segs.s[sg].count;
      ++sg;
    }
    const CsSeg& S = segs.s[sg];
    const long long r = pt - base;
    if (c < d)
      K[((long long)head * npts + pt) * d + c] = S.K[head * S.hsK + r * d + c];
    else if (c < d + dv)
      V[((long long)head * npts + pt) * dv + c - d] = S.V[head * S.hsV + r * dv + c - d];
    else
      W[(long long)head * npts + pt] = S.w;
  }
}
