// Moment update: X += sum over a key range of L(k) R(k, v)^T, features built on chip.
//
// State layout of one head ("level-fold" layout).  For level j = 0..p the block
// X_j has d^j rows and C_j columns, C_j = d + dv below the top level and
// C_p = dv at the top:
//     X_j[a][e]     = M_{j+1}[a*d + e]      for j < p, e < d
//     X_j[a][d + c] = N_j[a][c]             for j < p
//     X_p[a][c]     = N_p[a][c]
// with M_j = sum_i k_i^(x)j and N_j = sum_i k_i^(x)j v_i^T in row-major Kronecker
// order, and M_0 = the key count (kept on the host).  Every moment of degree
// 1..p appears exactly once, because M_{j+1} = sum_i k_i^(x)j k_i^T: the degree-
// (j+1) moment comes out of the same contraction as N_j.  So the whole update is
//     X_j = sum_i k_i^(x)j (x) u_i,   u_i = [k_i, v_i] (j < p),  u_i = v_i (j = p).
// Taylor moments of the polynomial method: "Rumo a Limites Estritos para Atenção
// em Streaming", "Metodologia", pillar "O Método Polinomial".
//
// Each level is a GEMM over keys.  Its Kronecker index is split into s leading
// digits (GEMM rows, features L = k^(x)s) and t = j - s trailing digits plus the
// column e (GEMM columns, features R = k^(x)t (x) u).  Row-major order makes the
// GEMM output exactly the rows of X_j, so tiles write contiguous rows.
//
// One workgroup (4 waves) owns a 256/wc x 64*wc output tile and a key range.  Per
// stage of SK_KB keys it copies the K and V rows to LDS with 128-bit loads, forms
// the L and R feature tiles in LDS (never in HBM), and every wave runs a 64x64
// register tile (2x2 blocks of v_mfma_f32_32x32x2_f32, fp32 in and out).
#pragma once

#include "sk_common.h"

__global__ __launch_bounds__(SK_WG, 2)
void sk_update_kernel(const float* __restrict__ K, const float* __restrict__ V,
                      long long n, int d, int dv, int logd,
                      const UpdTile* __restrict__ tiles, int ntiles,
                      long long keys_per_split,
                      float* __restrict__ out, long long head_stride,
                      long long split_stride, int accumulate) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile_id = blockIdx.x % ntiles;
  const long long split = blockIdx.x / ntiles;
  const long long head = blockIdx.y;
  const UpdTile T = tiles[tile_id];

  const int wc = T.wc;
  const int TM = SK_WG / wc;          // 256, 128 or 64 rows
  const int TN = 64 * wc;             // 64, 128 or 256 columns
  const int LDL = TM + SK_PAD;
  const int LDR = TN + SK_PAD;
  float* Ks = lds;                    // [SK_KB][d]
  float* Vs = Ks + SK_KB * d;         // [SK_KB][dv]
  float* Lt = Vs + SK_KB * dv;        // [SK_KB][LDL]
  float* Rt = Lt + SK_KB * LDL;       // [SK_KB][LDR]

  const long long k_begin = split * keys_per_split;
  long long k_end = k_begin + keys_per_split;
  if (k_end > n) k_end = n;

  const float* Kh = K + head * n * d;
  const float* Vh = V + head * n * dv;

  // Feature assignment (fixed for the whole key loop).
  const int s = T.s, t = T.t;
  const int dmask = d - 1;
  const int rL = tid % TM, kpL = tid / TM, stepL = SK_WG / TM;
  const int gL = T.row0 + rL;
  const bool validL = gL < T.M;
  int dl[SK_MAXDIG];
#pragma unroll
  for (int c = 0; c < SK_MAXDIG; ++c)
    dl[c] = (c < s) ? ((gL >> (logd * (s - 1 - c))) & dmask) : 0;

  const int cR = tid % TN, kpR = tid / TN, stepR = SK_WG / TN;
  const int gR = T.col0 + cR;
  const bool validR = gR < T.N;
  const int alo = gR / T.C;             // trailing Kronecker digits of the column
  const int e = gR - alo * T.C;         // position inside u
  int dr[SK_MAXDIG];
#pragma unroll
  for (int c = 0; c < SK_MAXDIG; ++c)
    dr[c] = (c < t) ? ((alo >> (logd * (t - 1 - c))) & dmask) : 0;
  // u = [k, v] below the top level, u = v at the top level
  const float* usrc;
  int ustride;
  if (!T.top && e < d) { usrc = Ks + e; ustride = d; }
  else { usrc = Vs + (T.top ? e : e - d); ustride = dv; }

  const int wr0 = (wave / wc) * 64;
  const int wc0 = (wave % wc) * 64;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  floatx16 acc00 = {0}, acc01 = {0}, acc10 = {0}, acc11 = {0};

  const int nK4 = SK_KB * d / 4;
  const int nV4 = SK_KB * dv / 4;
  const int d4 = d >> 2, dv4 = dv >> 2;

  for (long long kb0 = k_begin; kb0 < k_end; kb0 += SK_KB) {
    const long long left = k_end - kb0;
    const int nk = left < SK_KB ? (int)left : SK_KB;
    // 1. K and V rows of this stage -> LDS (rows past the range read as zero)
    const float4* Kg = reinterpret_cast<const float4*>(Kh + kb0 * d);
    const float4* Vg = reinterpret_cast<const float4*>(Vh + kb0 * dv);
    for (int i = tid; i < nK4; i += SK_WG) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i / d4 < nk) x = Kg[i];
      reinterpret_cast<float4*>(Ks)[i] = x;
    }
    for (int i = tid; i < nV4; i += SK_WG) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i / dv4 < nk) x = Vg[i];
      reinterpret_cast<float4*>(Vs)[i] = x;
    }
    __syncthreads();
    // 2. feature tiles: L = prod of s key entries, R = prod of t key entries * u[e]
    for (int kk = kpL; kk < SK_KB; kk += stepL) {
      const float* kr = Ks + kk * d;
      float f = validL ? 1.f : 0.f;
#pragma unroll
      for (int c = 0; c < SK_MAXDIG; ++c)
        if (c < s) f *= kr[dl[c]];
      Lt[kk * LDL + rL] = f;
    }
    for (int kk = kpR; kk < SK_KB; kk += stepR) {
      const float* kr = Ks + kk * d;
      float f = validR ? usrc[kk * ustride] : 0.f;
#pragma unroll
      for (int c = 0; c < SK_MAXDIG; ++c)
        if (c < t) f *= kr[dr[c]];
      Rt[kk * LDR + cR] = f;
    }
    __syncthreads();
    // 3. fp32 MFMA over the stage: two keys per instruction
#pragma unroll 4
    for (int ks = 0; ks < SK_KB / 2; ++ks) {
      const int kr = 2 * ks + lhi;
      const float a0 = Lt[kr * LDL + wr0 + l32];
      const float a1 = Lt[kr * LDL + wr0 + 32 + l32];
      const float b0 = Rt[kr * LDR + wc0 + l32];
      const float b1 = Rt[kr * LDR + wc0 + 32 + l32];
      acc00 = mfma32x32x2(a0, b0, acc00);
      acc01 = mfma32x32x2(a0, b1, acc01);
      acc10 = mfma32x32x2(a1, b0, acc10);
      acc11 = mfma32x32x2(a1, b1, acc11);
    }
    __syncthreads();
  }

  // Epilogue: rows of X_j are contiguous, so (row, col) -> xoff + row * N + col.
  float* o = out + split * split_stride + head * head_stride + T.xoff;
  const floatx16* accs[4] = {&acc00, &acc01, &acc10, &acc11};
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    const int i = bi >> 1, jj = bi & 1;
    const int col = T.col0 + wc0 + 32 * jj + l32;
    if (col >= T.N) continue;
    const floatx16 a = *accs[bi];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = T.row0 + wr0 + 32 * i + acc_row(r, lane);
      if (row < T.M) {
        const long long idx = (long long)row * T.N + col;
        if (accumulate) o[idx] += a[r];
        else o[idx] = a[r];
      }
    }
  }
}
