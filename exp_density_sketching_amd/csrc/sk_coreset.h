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
#define CS_QT 32           // queries per tail-query workgroup
#define CS_TPQ 4           // threads per query in the tail query
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
// (weight 2^l), each cut into slices of up to CS_SLICE points (the tail query
// picks the length per call).
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
#define CS_SLICE 512     // longest tail-query slice (points)

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

// R_p(x) = sum_{j > p} x^j / j! in float64 for N values x at once.  For
// |x| <= p + 1 the series x^(p+1) / (p+1)! * sum_k coef[k] x^k with coef[k] =
// (p+1)! / (p+1+k)! (the handle's table, coef[0] = 1), one fused multiply-add
// per term by Horner from the top, its terms counted for the largest such |x| of
// the N values (until the ratio of the next term to the first falls below
// 2^-56), so every value advances through the same instructions; there the
// terms shrink from the first on, so the sum's rounding stays within a few units
// of the last place of the largest term.  For |x| > p + 1, e^x - T_p(x), T_p by
// Horner: for x > p + 1, e^x exceeds twice T_p(x); below -(p + 1), T_p(x) and e^x
// do not cancel (T_p is positive for even p, negative there for odd p).  (The
// float64 oracle chooses between the plain series and e^x - T_p(x) by the size of
// the series' largest term; both are accurate to a few units of the last place,
// which a Gram entry of the walk needs.)
template <int N>
__device__ inline void cs_tail_exp64_c(const double (&x)[N], int p,
                                       const double* __restrict__ cs_inv,
                                       const double* __restrict__ coef, double (&out)[N]) {
#pragma clang fp contract(off)
  const double lim = (double)(p + 1);
  double X = 0.0;
#pragma unroll
  for (int e = 0; e < N; ++e)
    if (fabs(x[e]) <= lim) X = fmax(X, fabs(x[e]));
  int nt = 0;
  for (double t = 1.0; t > 0x1p-56 && p + 2 + nt < CS_NINV;) {
    ++nt;
    t *= X * cs_inv[p + 1 + nt];
  }
  double hh[N], xp[N];
  const double cn = coef[nt];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    hh[e] = cn;
    xp[e] = 1.0;
  }
  for (int k = nt - 1; k >= 0; --k) {
    const double ck = coef[k];
#pragma unroll
    for (int e = 0; e < N; ++e) hh[e] = fma(hh[e], x[e], ck);
  }
  for (int j = 1; j <= p + 1; ++j) {
    const double ij = cs_inv[j];
#pragma unroll
    for (int e = 0; e < N; ++e) xp[e] *= x[e] * ij;
  }
#pragma unroll
  for (int e = 0; e < N; ++e) {
    double r = xp[e] * hh[e];
    if (fabs(x[e]) > lim) {
      double tp = 1.0;
      for (int i = p; i >= 1; --i) tp = 1.0 + x[e] * cs_inv[i] * tp;
      r = exp(x[e]) - tp;
    }
    out[e] = r;
  }
}

typedef double doublex4 __attribute__((ext_vector_type(4)));

// Pair Gram matrix of a batch of reduces.  Grid: (reduce, head, upper tile) with
// the tile index fastest; 256 threads in 4 waves.  The tile's 64 row points and
// 64 column points (32 pairs each) are staged in LDS (fp32, as given), up to 128
// features of [k | v] at a time with one barrier; wave w takes rows
// 32 (w >> 1) .. + 31 and columns 32 (w & 1) .. + 31 as 2 x 2 blocks of
// v_mfma_f64_16x16x4_f64 on the features widened to float64 (A: lane l gives row
// slot l % 16 at feature l / 16 of the k-step, B the same for the column; the
// 16 x 16 result: lane l holds row slots l / 16 + 4 i, i = 0..3, of column
// l % 16), the key products and the value products in separate accumulators.
// Row slot m holds point 4 (m % 4) + m / 4 of the block, so that lane l holds
// points 4 (l / 16) + i: the two pairs 2 (l / 16) and 2 (l / 16) + 1.  Each entry
// then becomes g = R_p(<k, k'>) (1 + <v, v'>), and the pair entry
//     D[t][s] = ((g[2t][2s] - g[2t][2s+1]) - g[2t+1][2s]) + g[2t+1][2s+1]
// is formed by lane pairs (the two columns of a pair are neighbouring lanes; the
// even lane writes pair row 2 (l / 16), the odd lane the next).
// D: [reduce][head][B][B] float64.
#define CS_GF 128          // features staged at once
#define CS_GLD 80          // LDS row stride (floats): the 4 features of a k-step hit 4 bank groups
__global__ __launch_bounds__(256)
void cs_gram_kernel(CsOps ops, int B, int d, int dv, int p, int h,
                    const double* __restrict__ inv, double* __restrict__ Dws) {
  __shared__ float Rs[CS_GF][CS_GLD];
  __shared__ float Cs[CS_GF][CS_GLD];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  const int r0 = tr * 2 * CS_TP, c0 = tc * 2 * CS_TP;   // first merged point of rows / cols
  // the staging thread's point pt (tid / 4) of the rows and of the columns: its key
  // and value rows (merged point i < B: block a, else b)
  const int pt = tid >> 2, q = tid & 3;
  auto rows_of = [&](int i, const float*& k, const float*& v) {
    const CsRef& R = (i < B) ? O.a : O.b;
    const int r = (i < B) ? i : i - B;
    k = R.K + head * R.hsK + (long long)r * d;
    v = R.V + head * R.hsV + (long long)r * dv;
  };
  const float *rk, *rv, *ck, *cv;
  rows_of(r0 + pt, rk, rv);
  rows_of(c0 + pt, ck, cv);
  const int wr = wave >> 1, wc = wave & 1;
  const int l16 = lane & 15, lk = lane >> 4;
  const int rslot = 4 * (l16 & 3) + (l16 >> 2);         // point of the lane's row slot
  doublex4 kacc[2][2], vacc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) kacc[a][b] = vacc[a][b] = doublex4{0.0, 0.0, 0.0, 0.0};
  // k-steps [k0, k1) of the staged features into acc
  auto steps = [&](int k0, int k1, doublex4 (&acc)[2][2]) {
    for (int ks = k0; ks < k1; ks += 4) {
      const int f = ks + lk;
      const double a0 = Rs[f][32 * wr + rslot], a1 = Rs[f][32 * wr + 16 + rslot];
      const double b0 = Cs[f][32 * wc + l16], b1 = Cs[f][32 * wc + 16 + l16];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
    }
  };
  const int F = d + dv;
  for (int f0 = 0; f0 < F; f0 += CS_GF) {
    const int fw = min(CS_GF, F - f0);
    // stage 64 row and 64 column points, features f0 .. f0 + fw - 1 of [k | v]:
    // thread (pt, q) loads float4s q, q + 4, ... of its point (a float4 never
    // straddles k and v, as d is a multiple of 4)
    __syncthreads();
    for (int f = 4 * q; f < fw; f += 16) {
      const int g = f0 + f;
      const float4 x = *reinterpret_cast<const float4*>(g < d ? rk + g : rv + (g - d));
      const float4 y = *reinterpret_cast<const float4*>(g < d ? ck + g : cv + (g - d));
      Rs[f][pt] = x.x; Rs[f + 1][pt] = x.y; Rs[f + 2][pt] = x.z; Rs[f + 3][pt] = x.w;
      Cs[f][pt] = y.x; Cs[f + 1][pt] = y.y; Cs[f + 2][pt] = y.z; Cs[f + 3][pt] = y.w;
    }
    __syncthreads();
    const int kend = min(fw, max(0, d - f0));      // staged key features: [0, kend)
    steps(0, kend, kacc);
    steps(kend, fw, vacc);
  }
  double* Dh = Dws + ((long long)oi * h + head) * (long long)B * B;
  const bool odd = lane & 1;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    // the row block's 8 entries per lane (2 column blocks x 4 rows), one series run
    double xs[8], rs[8];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[4 * cb + i] = kacc[rb][cb][i];
    cs_tail_exp64_c<8>(xs, p, inv, inv + CS_NINV, rs);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      double g[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) g[i] = rs[4 * cb + i] * (1.0 + vacc[rb][cb][i]);
      // the even lane (column 2s) forms pair row 2 (l / 16) from rows 0, 1 and needs
      // the odd lane's rows 0, 1; the odd lane (column 2s + 1) forms the next pair
      // row from rows 2, 3 and needs the even lane's
      const double ra = __shfl_xor(odd ? g[0] : g[2], 1);
      const double rbv = __shfl_xor(odd ? g[1] : g[3], 1);
      const double Dv = odd ? ((ra - g[2]) - rbv) + g[3] : ((g[0] - ra) - g[1]) + rbv;
      const int t = tr * CS_TP + ((32 * wr + 16 * rb + 4 * lk) >> 1) + (odd ? 1 : 0);
      const int sc = tc * CS_TP + ((32 * wc + 16 * cb + l16) >> 1);
      Dh[(long long)t * B + sc] = Dv;
    }
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
// e = +1 (keep point 2t + 1) when U < P, else -1 (keep point 2t); for c > 0 the
// kernel tests the same condition as alpha < c (1 - 2U).
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
      // U < P = clamp((1 - a / c) / 2, 0, 1) is a < c (1 - 2 U) for c > 0 (1 - 2 U is
      // exact: U is a multiple of 2^-53), so each decision is one compare and the
      // wave's mask, the chain from one pair's sum to the next one decision long
      const double thr = c * (1.0 - 2.0 * U);
      const bool half = U < 0.5;
      double a = alpha[t0 + lane];
      int mine = 0;
      for (int i = 0; i < 64; ++i) {
        const unsigned long long m = __ballot(c > 0.0 ? a < thr : half);
        const double e = ((m >> i) & 1ull) ? 1.0 : -1.0;
        if (lane == i) mine = e > 0.0 ? 1 : -1;
        a = fma(e, blk[i][lane], a);           // blk[i][j] = 0 for j <= i
      }
      alpha[t0 + lane] = a;
      eps[t0 + lane] = (signed char)mine;
    }
    __syncthreads();
    // (the block's column entries loaded 16 at a time, then added in pair order)
    for (int s = t0 + 64 + tid; s < B; s += 256) {
      double x = alpha[s];
      const double* col = Dh + (long long)t0 * B + s;
      for (int i0 = 0; i0 < 64; i0 += 16) {
        double dcol[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) dcol[u] = col[(long long)(i0 + u) * B];
#pragma unroll
        for (int u = 0; u < 16; ++u) x = fma((double)eps[t0 + i0 + u], dcol[u], x);
      }
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
// (head, query, slice): sum_s w R_p(<q, k_s>) [1, v_s].  CS_TPQ threads per query
// (its query in registers in each), thread r taking points r, r + CS_TPQ, .. of
// every stage of CS_PT points staged in LDS (rows padded by 4 floats, so the
// float4 reads of the CS_TPQ points hit separate banks); the dot product in four
// independent partial sums; the query's CS_TPQ partials added in a fixed tree
// (xor shuffles) at the end.
template <int D, int DV>
__global__ __launch_bounds__(CS_QT * CS_TPQ)
void cs_tail_kernel(const float* __restrict__ Q, long long m, int p, CsSegs segs,
                    int slice_pts, float* __restrict__ parts) {
  constexpr int NTH = CS_QT * CS_TPQ;
  __shared__ float Ks[CS_PT][D + 4];
  __shared__ float Vs[CS_PT][DV + 4];
  __shared__ float inv[96];
  const int tid = threadIdx.x;
  const int ql = tid / CS_TPQ, rr = tid % CS_TPQ;
  const int qt = blockIdx.x, slice = blockIdx.y, head = blockIdx.z;
  for (int j = tid; j < 96; j += NTH) inv[j] = j == 0 ? 1.f : 1.f / (float)j;
  // the slice's segment
  int sg = 0;
  while (sg + 1 < segs.n && segs.s[sg + 1].slice0 <= slice) ++sg;
  const CsSeg S = segs.s[sg];
  const int p0 = (slice - S.slice0) * slice_pts;
  const int np = min(slice_pts, S.count - p0);
  const long long q = (long long)qt * CS_QT + ql;
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
    for (int e = tid; e < CS_PT * (D / 4); e += NTH) {
      const int r = e / (D / 4), c4 = e - r * (D / 4);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < ns) x = reinterpret_cast<const float4*>(Kb + (long long)(s0 + r) * D)[c4];
      *reinterpret_cast<float4*>(&Ks[r][4 * c4]) = x;
    }
    for (int e = tid; e < CS_PT * (DV / 4); e += NTH) {
      const int r = e / (DV / 4), c4 = e - r * (DV / 4);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < ns) x = reinterpret_cast<const float4*>(Vb + (long long)(s0 + r) * DV)[c4];
      *reinterpret_cast<float4*>(&Vs[r][4 * c4]) = x;
    }
    __syncthreads();
    for (int j = rr; j < ns; j += CS_TPQ) {
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
      for (int a = 0; a < D; a += 4) {
        const float4 k = *reinterpret_cast<const float4*>(&Ks[j][a]);
        d0 = fmaf(qr[a], k.x, d0);
        d1 = fmaf(qr[a + 1], k.y, d1);
        d2 = fmaf(qr[a + 2], k.z, d2);
        d3 = fmaf(qr[a + 3], k.w, d3);
      }
      const float r = S.w * cs_tail_exp32((d0 + d1) + (d2 + d3), p, inv);
      z += r;
#pragma unroll
      for (int c = 0; c < DV; c += 4) {
        const float4 v = *reinterpret_cast<const float4*>(&Vs[j][c]);
        acc[c] = fmaf(r, v.x, acc[c]);
        acc[c + 1] = fmaf(r, v.y, acc[c + 1]);
        acc[c + 2] = fmaf(r, v.z, acc[c + 2]);
        acc[c + 3] = fmaf(r, v.w, acc[c + 3]);
      }
    }
  }
  // the query's partials: lanes 4 ql .. 4 ql + 3, the same fixed tree in each
#pragma unroll
  for (int o = 1; o < CS_TPQ; o <<= 1) {
    z += __shfl_xor(z, o);
#pragma unroll
    for (int c = 0; c < DV; ++c) acc[c] += __shfl_xor(acc[c], o);
  }
  if (qv && rr == 0) {
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
