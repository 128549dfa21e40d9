// Query of the moment sketch: Zhat(q) = sum_j <q^(x)j, M_j>/j!,
// Ntilde(q) = sum_j <q^(x)j, N_j>/j!, ohat = Ntilde / Zhat.
// Source: "Rumo a Limites Estritos para Atenção em Streaming", "Metodologia",
// pillar "O Método Polinomial" (answering from the low-degree moments).
//
// With the level-fold layout (see sk_update.h), level j contributes
//     Y_j[q][e] = sum_a q^(x)j[a] * X_j[a][e]
// then  Zhat += sum_{e<d} q[e] Y_j[q][e] / (j+1)!     (this is M_{j+1}, j < p)
//       Ntilde[c] += Y_j[q][d + c] / j!  (j < p),   Y_p[q][c] / p!  (j = p)
// plus the count for M_0.  The feature index a is split into s leading digits
// a_hi and t trailing digits a_lo, q^(x)j[a] = q^(x)s[a_hi] q^(x)t[a_lo], so
//     Y_j[q][e] = sum_{a_lo} q^(x)t[a_lo] * sum_{a_hi} q^(x)s[a_hi] X_j[a_hi][(a_lo, e)].
// The inner sum is a GEMM whose columns (a_lo, e) are rows of X_j read as they lie
// in memory; t is the fewest digits that give it at least 128 columns, or none
// when the level's own columns fill half of them.  One workgroup owns
// 128 queries x 128 columns x a range of a_hi: per stage of 32 rows it forms the
// query features q^(x)s in LDS, stages the state rows through LDS (fetched one
// stage ahead into registers) and runs the same 2x2 v_mfma_f32_32x32x2_f32 register
// tile per wave as the update.  The epilogue multiplies by q^(x)t[a_lo] (and by
// q[e]/(j+1)! or 1/j!), folds a_lo through LDS in column order and writes a
// [128][C] partial; sk_query_finish adds the partials in tile order.
#pragma once

#include "sk_common.h"

#define SK_TMQ 128
#define SK_TNQ 128

template <int LOGD>
__global__ __launch_bounds__(SK_WG, 2)
void sk_query_kernel(const float* __restrict__ Q, long long m,
                     const float* __restrict__ X, long long head_stride,
                     const QryTile* __restrict__ tiles, int ntiles, int nqt,
                     long long PB, float* __restrict__ parts) {
  constexpr int d = 1 << LOGD;
  constexpr int dmask = d - 1;
  constexpr int LDQ = SK_TMQ + 1;
  constexpr int LDA = SK_TMQ + SK_PAD;
  constexpr int LDB = SK_TNQ + SK_PAD;
  constexpr int LDY = SK_TNQ + 1;
  // digits of a row index that overlap its lowest four bits
  constexpr int NV = (4 + LOGD - 1) / LOGD;
  static_assert(NV <= 2, "d >= 4");
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // 1-D grid over (tile, query tile, head), tile fastest: tiles of different
  // levels differ in length, so they are dealt round-robin over the XCDs
  const long long lg = blockIdx.x;
  const int tile_id = (int)(lg % ntiles);
  const int qt = (int)((lg / ntiles) % nqt);
  const long long head = lg / ((long long)nqt * ntiles);
  const QryTile T = tiles[tile_id];

  float* Qs = lds;                    // [d][LDQ]       query tile, transposed
  float* At = Qs + d * LDQ;           // [SK_KB][LDA]   features q^(x)s[a_hi]
  float* Bt = At + SK_KB * LDA;       // [SK_KB][LDB]   state rows
  float* Ys = At;                     // [64][LDY]      epilogue (reuses At, Bt)

  const long long q0 = (long long)qt * SK_TMQ;
  {
    const float* Qh = Q + (head * m + q0) * d;
    const long long qrem = m - q0;
    for (int i = tid; i < SK_TMQ * d; i += SK_WG) {
      const int qq = i / d, c = i - qq * d;
      Qs[c * LDQ + qq] = (qq < qrem) ? Qh[i] : 0.f;
    }
  }

  const float* Xh = X + head * head_stride + T.xoff;
  const int s = T.s;
  // Feature thread: query qq, rows 16 kp + u (u < 16) of every 32-row stage.  A
  // stage starts at a multiple of 32, so row ab + 16 kp + u has the bits of ab,
  // kp and u in disjoint places: its digits above bit 3 are the same for all 16
  // rows of the thread (one product per stage), and only the (at most two)
  // digits overlapping bits 0..3 change with u, by compile-time amounts.
  const int qq = tid % SK_TMQ;
  const int kp = __builtin_amdgcn_readfirstlane(tid / SK_TMQ);
  const float* Qq = Qs + qq;
  const int wr0 = (wave >> 1) * 64;                 // wave's queries
  const int wc0 = (wave & 1) * 64;                  // wave's columns
  const int l32 = lane & 31, lhi = lane >> 5;

  float4 breg[4];
  auto fetch = [&](long long ab) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = tid + r * SK_WG;
      const int row = i >> 5, c = (i & 31) * 4;
      const long long a = ab + row;
      const int col = T.col0 + c;
      breg[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (a < T.a1 && col < T.N)
        breg[r] = *reinterpret_cast<const float4*>(Xh + a * T.N + col);
    }
  };

  floatx16 acc00 = {0}, acc01 = {0}, acc10 = {0}, acc11 = {0};
  __syncthreads();
  if (T.a0 < T.a1) fetch(T.a0);
  for (long long ab = T.a0; ab < T.a1; ab += SK_KB) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = tid + r * SK_WG;
      *reinterpret_cast<float4*>(Bt + (i >> 5) * LDB + (i & 31) * 4) = breg[r];
    }
    // features q^(x)s[a_hi] of this thread's query for rows ab + 16 kp + u
    {
      const long long rb = ab + 16 * kp;            // first row of the thread
      float hpre = 1.f;
#pragma unroll
      for (int i = NV; i < SK_MAXDIG; ++i)
        if (i < s) hpre *= Qq[(int)((rb >> (LOGD * i)) & dmask) * LDQ];
      const long long rem = T.a1 - rb;              // rows of the thread still in range
      const int nvs = s < NV ? s : NV;
      const float* Q0 = Qq + (int)(rb & dmask) * LDQ;
      const float* Q1 = Qq + (int)((rb >> LOGD) & dmask) * LDQ;
      float f[16];
      if (nvs == 0) {
#pragma unroll
        for (int u = 0; u < 16; ++u) f[u] = hpre;
      } else if (nvs == 1) {
#pragma unroll
        for (int u = 0; u < 16; ++u) f[u] = hpre * Q0[(u & dmask) * LDQ];
      } else {
#pragma unroll
        for (int u = 0; u < 16; ++u)
          f[u] = hpre * Q0[(u & dmask) * LDQ] * Q1[((u >> LOGD) & dmask) * LDQ];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) At[(16 * kp + u) * LDA + qq] = (u < rem) ? f[u] : 0.f;
    }
    __syncthreads();
    if (ab + SK_KB < T.a1) fetch(ab + SK_KB);
    float a0 = At[lhi * LDA + wr0 + l32];
    float a1 = At[lhi * LDA + wr0 + 32 + l32];
    float b0 = Bt[lhi * LDB + wc0 + l32];
    float b1 = Bt[lhi * LDB + wc0 + 32 + l32];
#pragma unroll
    for (int ks = 0; ks < SK_KB / 2; ++ks) {
      float na0 = 0.f, na1 = 0.f, nb0 = 0.f, nb1 = 0.f;
      if (ks + 1 < SK_KB / 2) {
        const int kr = 2 * (ks + 1) + lhi;
        na0 = At[kr * LDA + wr0 + l32];
        na1 = At[kr * LDA + wr0 + 32 + l32];
        nb0 = Bt[kr * LDB + wc0 + l32];
        nb1 = Bt[kr * LDB + wc0 + 32 + l32];
      }
      acc00 = mfma32x32x2(a0, b0, acc00);
      acc01 = mfma32x32x2(a0, b1, acc01);
      acc10 = mfma32x32x2(a1, b0, acc10);
      acc11 = mfma32x32x2(a1, b1, acc11);
      a0 = na0; a1 = na1; b0 = nb0; b1 = nb1;
    }
    __syncthreads();
  }

  // Epilogue, 64 queries at a time: weight each column by q^(x)t[a_lo] and by
  // q[e]/(j+1)! (M_{j+1} part) or 1/j! (N_j part), then fold a_lo.
  const int C = T.C, t = T.t;
  float* P = parts + (head * nqt + qt) * PB + T.pofs;   // [SK_TMQ][C]
  const floatx16* accs[4] = {&acc00, &acc01, &acc10, &acc11};
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
    if ((wave >> 1) == half) {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int i = bi >> 1, jj = bi & 1;
        const int cl = wc0 + 32 * jj + l32;
        const int col = T.col0 + cl;
        const bool valid = col < T.N;
        const int alo = col / C;
        const int e = col - alo * C;
        const bool zcol = (!T.top) && (e < d);
        const floatx16 a = *accs[bi];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * i + acc_row(r, lane);   // 0..63 inside this half
          const int q = wr0 + ql;
          float w = 0.f;
          if (valid) {
            w = zcol ? Qs[e * LDQ + q] * T.wz : T.wn;
            if (t == 1) {                     // the common case, without the loop
              w *= Qs[(alo & dmask) * LDQ + q];
            } else {
              for (int c = 0; c < t; ++c)
                w *= Qs[((alo >> (LOGD * (t - 1 - c))) & dmask) * LDQ + q];
            }
          }
          Ys[ql * LDY + cl] = a[r] * w;
        }
      }
    }
    __syncthreads();
    const int cmod = T.col0 % C;
    for (int pi = tid; pi < 64 * C; pi += SK_WG) {
      const int ql = pi / C, e = pi - ql * C;
      int cl = e - cmod;
      if (cl < 0) cl += C;
      float sum = 0.f;
      for (; cl < SK_TNQ && T.col0 + cl < T.N; cl += C) sum += Ys[ql * LDY + cl];
      P[(long long)(64 * half + ql) * C + e] = sum;
    }
  }
}

// Sum the partials of every tile, add the count, divide.  One workgroup per
// (head, query).  A tile's record holds columns fc0 .. fc0 + fw - 1 of its level;
// a column col < d of a lower level holds a share of Zhat, col >= d one of
// Ntilde[col - d] (top-level tiles hold only the Ntilde columns, at col - d), so
// entry column c of the query (c < d: Zhat shares, c >= d: Ntilde[c - d]) takes
// record column c - sh of every tile whose [sh, sh + fw) holds c (FinTile.sh).
// The tiles are split over S = 256 / (d + dv) groups of d + dv threads: group g
// adds the tiles g, g + S, g + 2S, ... in that order (eight loads in flight per
// thread), then the group sums are added in group order; Zhat is the count plus
// the query's Zhat columns in four running sums by column mod 4, added as
// (s0 + s1) + (s2 + s3).  The tile table is staged in LDS once.
#define SK_QFIN_LDS 512
struct FinTile {
  long long pofs;   // record offset in a query tile's block of partials
  int fw;           // record width
  int sh;           // entry column of record column 0
};
__global__ __launch_bounds__(256)
void sk_query_finish(const float* __restrict__ parts, const FinTile* __restrict__ fin,
                     int ntiles, int nqt, long long PB, long long m, int d, int dv,
                     float count, const float* __restrict__ Q,
                     const float* __restrict__ center, float* __restrict__ out,
                     float* __restrict__ Z) {
  __shared__ long long tp[SK_QFIN_LDS];
  __shared__ int tw[SK_QFIN_LDS];
  __shared__ int ts[SK_QFIN_LDS];
  __shared__ float red[256];
  __shared__ float zq;
  const int tid = threadIdx.x;
  const int cols = d + dv;
  const int S = cols >= 256 ? 1 : 256 / cols;
  const long long gq = blockIdx.x;                  // head * m + query
  const long long head = gq / m, q = gq - head * m;
  const long long qt = q / SK_TMQ;
  const int ql = (int)(q - qt * SK_TMQ);
  const float* P = parts + (head * nqt + qt) * PB;
  const bool staged = ntiles <= SK_QFIN_LDS;
  if (staged) {
    for (int i = tid; i < ntiles; i += 256) {
      const FinTile f = fin[i];
      tp[i] = f.pofs;
      tw[i] = f.fw;
      ts[i] = f.sh;
    }
  }
  __syncthreads();
  const int g = tid / cols, c = tid - g * cols;
  float acc = 0.f;
  if (g < S) {
    for (int t0 = g; t0 < ntiles; t0 += 8 * S) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = t0 + u * S;
        x[u] = 0.f;
        if (t < ntiles) {
          long long pofs;
          int fw, sh;
          if (staged) { pofs = tp[t]; fw = tw[t]; sh = ts[t]; }
          else { const FinTile f = fin[t]; pofs = f.pofs; fw = f.fw; sh = f.sh; }
          const int cc = c - sh;
          if (cc >= 0 && cc < fw) x[u] = P[pofs + (long long)ql * fw + cc];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += x[u];
    }
  }
  red[tid] = acc;
  __syncthreads();
  float v = 0.f;
  if (tid < cols) {
    v = red[tid];
    for (int k = 1; k < S; ++k) v += red[k * cols + tid];
  }
  __syncthreads();
  if (tid < cols) red[tid] = v;
  __syncthreads();
  if (tid == 0) {
    float z0 = 0.f, z1 = 0.f, z2 = 0.f, z3 = 0.f;
    for (int e = 0; e < d; e += 4) {
      z0 += red[e]; z1 += red[e + 1]; z2 += red[e + 2]; z3 += red[e + 3];
    }
    float zz = ((z0 + z1) + (z2 + z3)) + count;
    zq = zz;
    // with a centre c the moments are those of k - c: the returned Zhat carries
    // e^{<q,c>}, which cancels in ohat
    float f = 1.f;
    if (center != nullptr) {
      const float* qv = Q + (head * m + q) * d;
      float dot = 0.f;
      for (int e = 0; e < d; ++e) dot += qv[e] * center[head * d + e];
      f = expf(dot);
    }
    Z[head * m + q] = zz * f;
  }
  __syncthreads();
  if (tid >= d && tid < cols) out[(head * m + q) * dv + (tid - d)] = v / zq;
}
