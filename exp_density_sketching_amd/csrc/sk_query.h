// Query of the moment sketch: Zhat(q) = sum_j <q^(x)j, M_j>/j!,
// Ntilde(q) = sum_j <q^(x)j, N_j>/j!, ohat = Ntilde / Zhat.
// Source: "Rumo a Limites Estritos para Atenção em Streaming", "Metodologia",
// pillar "O Método Polinomial" (answering from the low-degree moments).
//
// With the level-fold layout (see sk_update.h), level j contributes
//     Y_j[q][e] = sum_a q^(x)j[a] * X_j[a][e]
// and then  Zhat += sum_{e<d} q[e] Y_j[q][e] / (j+1)!   (M_{j+1}, j < p)
//           Ntilde[c] += Y_j[q][d + c] / j!   (j < p),  Y_p[q][c] / p!  (j = p)
// plus the count for M_0.  Y_j is a GEMM with the query features on the left;
// one workgroup owns 128 queries x 32 columns x a range of feature rows a, forms
// the features q^(x)j[a] in LDS and streams the state rows through LDS into
// v_mfma_f32_32x32x2_f32.  The epilogue applies the per-column weight and writes
// a 128 x 32 partial; sk_query_finish sums the partials in a fixed order.
#pragma once

#include "sk_common.h"

#define SK_TMQ 128

__global__ __launch_bounds__(SK_WG, 2)
void sk_query_kernel(const float* __restrict__ Q, long long m, int d, int logd,
                     const float* __restrict__ X, long long head_stride,
                     const QryTile* __restrict__ tiles, int ntiles, int nqt,
                     const float* __restrict__ wts,  // [p+2]: 1/j!
                     float* __restrict__ parts) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile_id = blockIdx.x % ntiles;
  const int qt = blockIdx.x / ntiles;
  const long long head = blockIdx.y;
  const QryTile T = tiles[tile_id];
  const int j = T.level;

  const int LDQ = SK_TMQ + 1;
  const int LDA = SK_TMQ + SK_PAD;
  const int LDB = 32;
  float* Qs = lds;                    // [d][LDQ]   transposed query tile
  float* At = Qs + d * LDQ;           // [SK_KB][LDA] query features
  float* Bt = At + SK_KB * LDA;       // [SK_KB][LDB] state rows

  const long long q0 = (long long)qt * SK_TMQ;
  const float* Qh = Q + (head * m + q0) * d;
  const long long qrem = m - q0;
  for (int i = tid; i < SK_TMQ * d; i += SK_WG) {
    const int qq = i / d, c = i - qq * d;
    Qs[c * LDQ + qq] = (qq < qrem) ? Qh[i] : 0.f;
  }

  const float* Xh = X + head * head_stride + T.xoff;
  const int C = T.C;
  const long long arows = 1LL << (logd * j);   // d^j rows in level j
  const long long a1 = T.a1 < arows ? T.a1 : arows;

  // feature assignment: query qq, rows kk = kp, kp + 2, ...
  const int qq = tid % SK_TMQ, kp = tid / SK_TMQ;
  const int dmask = d - 1;
  const int l32 = lane & 31, lhi = lane >> 5;
  // state-row copy assignment: row kk = tid / 8, four columns at (tid % 8) * 4
  const int bk = tid >> 3, bc = (tid & 7) * 4;
  const bool bcol_ok = (T.e0 + bc) < C;

  floatx16 acc = {0};
  __syncthreads();

  for (long long ab = T.a0; ab < a1; ab += SK_KB) {
    // 1. state rows [ab, ab + SK_KB) x columns [e0, e0 + 32) -> LDS
    {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      const long long a = ab + bk;
      if (a < a1 && bcol_ok)
        x = *reinterpret_cast<const float4*>(Xh + a * C + T.e0 + bc);
      *reinterpret_cast<float4*>(Bt + bk * LDB + bc) = x;
    }
    // 2. features q^(x)j[a]: the product of the j digits of a, reusing the
    //    prefix (leading j-1 digits) while it does not change
    {
      long long cur_pre = -1;
      float pre_val = 0.f;
      for (int kk = kp; kk < SK_KB; kk += SK_WG / SK_TMQ) {
        const long long a = ab + kk;
        float f = 0.f;
        if (a < a1) {
          if (j == 0) {
            f = 1.f;
          } else {
            const long long pre = a >> logd;
            if (pre != cur_pre) {
              float pv = 1.f;
              for (int c = 0; c < j - 1; ++c) {
                const int dig = (int)((pre >> (logd * (j - 2 - c))) & dmask);
                pv *= Qs[dig * LDQ + qq];
              }
              cur_pre = pre;
              pre_val = pv;
            }
            f = pre_val * Qs[(int)(a & dmask) * LDQ + qq];
          }
        }
        At[kk * LDA + qq] = f;
      }
    }
    __syncthreads();
    // 3. MFMA: wave w owns queries [32 w, 32 w + 32)
#pragma unroll 4
    for (int ks = 0; ks < SK_KB / 2; ++ks) {
      const int kr = 2 * ks + lhi;
      const float a = At[kr * LDA + wave * 32 + l32];
      const float b = Bt[kr * LDB + l32];
      acc = mfma32x32x2(a, b, acc);
    }
    __syncthreads();
  }

  // Epilogue: weight each column, write the 128 x 32 partial of this tile.
  const int e = T.e0 + l32;
  const bool zcol = (!T.top) && (e < d);
  const float wz = wts[j + 1];
  const float wn = wts[j];
  float* P = parts + (((head * nqt + qt) * (long long)ntiles) + tile_id) * (SK_TMQ * 32);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int q = wave * 32 + acc_row(r, lane);
    float v;
    if (e >= C) v = 0.f;
    else if (zcol) v = acc[r] * Qs[e * LDQ + q] * wz;
    else v = acc[r] * wn;
    P[q * 32 + l32] = v;
  }
}

// Sum the partials of every tile in tile order, add the count, divide.
// One workgroup per (query, head); thread 0 forms Zhat, thread 1 + c forms
// Ntilde[c].
__global__ __launch_bounds__(256)
void sk_query_finish(const float* __restrict__ parts, const QryTile* __restrict__ tiles,
                     int ntiles, int nqt, long long m, int d, int dv, float count,
                     float* __restrict__ out, float* __restrict__ Z) {
  __shared__ float zs;
  const long long q = blockIdx.x;
  const long long head = blockIdx.y;
  const int slot = threadIdx.x;
  const int qt = (int)(q / SK_TMQ), qi = (int)(q % SK_TMQ);
  const float* P = parts + ((head * nqt + qt) * (long long)ntiles) * (SK_TMQ * 32) + qi * 32;
  float acc = 0.f;
  if (slot == 0) {
    for (int ti = 0; ti < ntiles; ++ti) {
      const QryTile T = tiles[ti];
      if (T.top || T.e0 >= d) continue;
      const float* row = P + (long long)ti * (SK_TMQ * 32);
      const int lim = min(32, min(d, T.C) - T.e0);
      for (int c = 0; c < lim; ++c) acc += row[c];
    }
    acc += count;
    zs = acc;
  } else if (slot <= dv) {
    const int c = slot - 1;
    for (int ti = 0; ti < ntiles; ++ti) {
      const QryTile T = tiles[ti];
      const int e = T.top ? c : d + c;
      if (e < T.e0 || e >= T.e0 + 32 || e >= T.C) continue;
      acc += P[(long long)ti * (SK_TMQ * 32) + (e - T.e0)];
    }
  }
  __syncthreads();
  const float zh = zs;
  if (slot == 0) Z[head * m + q] = zh;
  else if (slot <= dv) out[(head * m + q) * dv + (slot - 1)] = acc / zh;
}
