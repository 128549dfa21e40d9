// One streaming decode step of the moment sketch: per head, append one key/value
// pair and answer one query over the stream including it (the stream of key/value
// pairs answered query by query: "Rumo a Limites Estritos para Atenção em
// Streaming", "Definição do Problema"; the moments and their query: "Metodologia",
// pillar "O Método Polinomial").
//
// Every stored entry x of row r and column e changes by the rank-one term
//     x += f_k(r) * u[e]          (u = [k, v] below the top, u = v at the top)
// with f_k(r) the row's key feature (k^(x)j[a] in the full layout, k^beta in the
// multiset layout), and the answer is a weighted sum of the updated entries:
//     Zhat   = count + sum over the M columns of  w(r, e) * x,
//     Ntilde = sum over the N columns of          w(r, e) * x,
// w = the query weight of the entry (full layout: q^(x)j[a]/j! times q[e]/(j+1)
// on the M columns; multiset layout: q^beta/beta!, and on the M columns
// q[e]/(multiplicity of e in beta + 1) when e is at least the largest index of
// beta, 0 otherwise).  So one pass over the state -- one read and one write of
// every float -- both appends and answers; the step is bound by HBM (or the
// Infinity Cache when the state fits).
#pragma once

#include "sk_common.h"
#include "sk_sym.h"

#define ST_FLOATS 8192    // state floats per workgroup at most (32 KB)
#define ST_ROWS 1024      // rows per workgroup at most

// One row range of one block (full layout: a level j; multiset layout: the lower
// or the top block) of one head's state.
struct StepTile {
  long long xoff;    // float offset of the block in one head's state
  long long row0;    // first row (block rows)
  int nrows;         // rows of the tile, <= ST_ROWS
  int C;             // row width
  int top;           // 1: the columns are v only
  int level;         // full layout: the level j (row a has j base-d digits); -1: multiset
  int rc0;           // multiset layout: canonical row of the block's row 0
  float wn;          // full layout: 1/j!
  float wz;          // full layout: 1/(j+1)
};

__global__ __launch_bounds__(256)
void sk_step_kernel(float* __restrict__ X, long long head_stride,
                    const StepTile* __restrict__ tiles, int ntiles, int d, int dv, int logd,
                    const float* __restrict__ kin, const float* __restrict__ vin,
                    const float* __restrict__ qin, SymTables tb,
                    float* __restrict__ parts, const float* __restrict__ center) {
  __shared__ float ks[128], vs[128], qs[128];
  __shared__ float fk[ST_ROWS], fq[ST_ROWS];
  __shared__ int lastr[ST_ROWS], lmulr[ST_ROWS];
  __shared__ float red[1024];
  const int tid = threadIdx.x;
  const int tile = (int)(blockIdx.x % ntiles);
  const long long head = blockIdx.x / ntiles;
  const StepTile T = tiles[tile];
  for (int i = tid; i < d; i += 256) {
    ks[i] = kin[head * d + i] - (center != nullptr ? center[head * d + i] : 0.f);
    qs[i] = qin[head * d + i];
  }
  for (int i = tid; i < dv; i += 256) vs[i] = vin[head * dv + i];
  __syncthreads();
  const int dmask = d - 1;
  for (int r = tid; r < T.nrows; r += 256) {
    float a = 1.f, b = 1.f;
    if (T.level >= 0) {
      const long long row = T.row0 + r;
      for (int c = 0; c < T.level; ++c) {
        const int dig = (int)((row >> (logd * c)) & dmask);
        a *= ks[dig];
        b *= qs[dig];
      }
      b *= T.wn;
    } else {
      const int cid = T.rc0 + (int)T.row0 + r;
      const unsigned long long code = tb.code[cid];
      const int cnt = (int)(code >> 56);
      for (int c = 0; c < cnt; ++c) {
        const int dig = (int)((code >> (8 * c)) & 0xffu);
        a *= ks[dig];
        b *= qs[dig];
      }
      b *= tb.winv[cid];
      lastr[r] = tb.last[cid];
      lmulr[r] = tb.lmul[cid];
    }
    fk[r] = a;
    fq[r] = b;
  }
  __syncthreads();

  // thread: column group c4 (4 columns), rows rp, rp + RP, ...
  const int C = T.C, C4 = C >> 2;
  const int RP = 256 / C4;
  const int rp = tid / C4, c4 = tid - rp * C4;
  const bool act = rp < RP;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (act) {
    float u[4];
    int col[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      col[i] = 4 * c4 + i;
      u[i] = T.top ? vs[col[i]] : (col[i] < d ? ks[col[i]] : vs[col[i] - d]);
    }
    float* Xb = X + head * head_stride + T.xoff + (long long)T.row0 * C + 4 * c4;
    for (int r = rp; r < T.nrows; r += RP) {
      float4* px = reinterpret_cast<float4*>(Xb + (long long)r * C);
      float4 x = *px;
      const float a = fk[r], w = fq[r];
      x.x += a * u[0];
      x.y += a * u[1];
      x.z += a * u[2];
      x.w += a * u[3];
      *px = x;
      const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = col[i];
        float wt = w;
        if (!T.top && e < d) {
          if (T.level >= 0) {
            wt = w * qs[e] * T.wz;
          } else {
            const int last = lastr[r];
            wt = (last == d || e > last) ? w * qs[e]
                 : (e == last ? w * qs[e] / (float)(lmulr[r] + 1) : 0.f);
          }
        }
        acc[i] += wt * xv[i];
      }
    }
  }
  // column sums over the row phases, in phase order
  if (act) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[rp * C + 4 * c4 + i] = acc[i];
  }
  __syncthreads();
  float* rec = parts + (head * ntiles + tile) * (long long)(1 + dv);
  for (int c = tid; c < C; c += 256) {
    float sum = 0.f;
    for (int p = 0; p < RP; ++p) sum += red[p * C + c];
    red[c] = sum;   // phase 0 row, read only by this thread before
  }
  __syncthreads();
  if (tid == 0) {
    float z = 0.f;
    if (!T.top)
      for (int e = 0; e < d; ++e) z += red[e];
    rec[0] = z;
  }
  for (int c = tid; c < dv; c += 256) rec[1 + c] = red[T.top ? c : d + c];
}

// Per head: Zhat = count + the sum of the tiles' Zhat parts, Ntilde likewise (a
// fixed order: interleaved running sums, each in tile order, added in order),
// ohat = Ntilde / Zhat; with a centre c the moments are those of k - c and the
// returned Zhat carries the factor e^{<q,c>} (which cancels in ohat).
__global__ __launch_bounds__(256)
void sk_step_finish(const float* __restrict__ parts, int ntiles, int d, int dv, float count,
                    const float* __restrict__ qin, const float* __restrict__ center,
                    float* __restrict__ out, float* __restrict__ Z) {
  __shared__ float ps[256];
  __shared__ float zs;
  const int tid = threadIdx.x;
  const long long head = blockIdx.x;
  const int cols = 1 + dv;
  // L threads per record column (L * cols <= 256): thread j of column c adds the
  // tiles j, j + L, ... in tile order, 16 loads in flight at a time (the records
  // come from other XCDs' writes, so each load is a long round trip); the
  // column's L sums are then added in thread order
  const int L = std::max(1, std::min(64, 256 / cols));
  const int c = tid / L, j = tid - c * L;
  const float* P = parts + head * ntiles * (long long)cols;
  float a = 0.f;
  if (c < cols) {
    const float* Pc = P + c;
    int t = j;
    for (; t + 15 * L < ntiles; t += 16 * L) {
      float r[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) r[u] = Pc[(long long)(t + u * L) * cols];
#pragma unroll
      for (int u = 0; u < 16; ++u) a += r[u];
    }
    for (; t < ntiles; t += L) a += Pc[(long long)t * cols];
  }
  ps[tid] = a;
  __syncthreads();
  float sum = 0.f;
  if (c < cols && j == 0)
    for (int i = 0; i < L; ++i) sum += ps[tid + i];
  __syncthreads();
  if (c < cols && j == 0) ps[c] = sum;
  __syncthreads();
  if (tid == 0) {
    zs = ps[0] + count;
    float f = 1.f;
    if (center != nullptr) {
      float dot = 0.f;
      for (int e = 0; e < d; ++e) dot += qin[head * d + e] * center[head * d + e];
      f = expf(dot);
    }
    Z[head] = zs * f;
  }
  __syncthreads();
  for (int cc = tid; cc < dv; cc += 256) out[head * dv + cc] = ps[1 + cc] / zs;
}
