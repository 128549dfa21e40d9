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
#include "sk_elementwise.h"

// Multiplies f[u] by the key entries named by S digit offsets dg[0..S), for the
// keys at base + STEP * u.  S is a compile-time count so that every LDS read of
// the S digits is issued before the first product (no wait per digit).
template <int S, int CH, int STEP>
__device__ __forceinline__ void mul_digits(float (&f)[CH], const float* __restrict__ Ks,
                                           const int* dg, int base) {
  // keys in sub-chunks of SUB so that at most 16 values are in flight
  constexpr int SUB = (16 / S) < CH ? ((16 / S) > 0 ? (16 / S) : 1) : CH;
#pragma unroll
  for (int u0 = 0; u0 < CH; u0 += SUB) {
    float v[S][SUB];
#pragma unroll
    for (int c = 0; c < S; ++c)
#pragma unroll
      for (int u = 0; u < SUB; ++u)
        if (u0 + u < CH) v[c][u] = Ks[dg[c] + base + STEP * (u0 + u)];
#pragma unroll
    for (int c = 0; c < S; ++c)
#pragma unroll
      for (int u = 0; u < SUB; ++u)
        if (u0 + u < CH) f[u0 + u] *= v[c][u];
  }
}

// The same for a digit count n known only at run time (uniform across the
// workgroup: one scalar branch per call).
template <int CH, int STEP>
__device__ __forceinline__ void mul_digits_n(int n, float (&f)[CH], const float* __restrict__ Ks,
                                             const int* dg, int base) {
  switch (n) {
    case 0: break;
    case 1: mul_digits<1, CH, STEP>(f, Ks, dg, base); break;
    case 2: mul_digits<2, CH, STEP>(f, Ks, dg, base); break;
    case 3: mul_digits<3, CH, STEP>(f, Ks, dg, base); break;
    case 4: mul_digits<4, CH, STEP>(f, Ks, dg, base); break;
    case 5: mul_digits<5, CH, STEP>(f, Ks, dg, base); break;
    case 6: mul_digits<6, CH, STEP>(f, Ks, dg, base); break;
    case 7: mul_digits<7, CH, STEP>(f, Ks, dg, base); break;
    default: mul_digits<8, CH, STEP>(f, Ks, dg, base); break;
  }
}

template <int WC, bool CENTER, int NPF>
__device__ __forceinline__
void sk_update_tile(const float* __restrict__ K, const float* __restrict__ V,
                    long long n, long long hkeys, int d, int dv, int logd, const UpdTile& T,
                    long long split, long long head, long long keys_per_split,
                    float* __restrict__ out, long long head_stride,
                    long long split_stride, int accumulate,
                    const float* __restrict__ center) {
  constexpr int TM = SK_WG / WC;      // 256, 128 or 64 rows
  constexpr int TN = 64 * WC;         // 64, 128 or 256 columns
  constexpr int LDL = TM + SK_PAD;
  constexpr int LDR = TN + SK_PAD;
  constexpr int STEPL = SK_WG / TM, NKL = SK_KB / STEPL;   // keys per thread (L)
  constexpr int STEPR = SK_WG / TN, NKR = SK_KB / STEPR;   // keys per thread (R)
  constexpr int CHL = NKL < 16 ? NKL : 16, CHR = NKR < 16 ? NKR : 16;  // keys per pass
  // NPF: float4 of K (and of V) per thread per stage, 32 max(d, dv) / 1024
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // K and V of a stage are stored transposed, [component][key] with an odd row
  // stride, so a thread's keys sit at compile-time offsets from one base.
  constexpr int LDK = SK_KB + 1;
  float* Ks = lds;                    // [d][LDK]
  float* Vs = Ks + d * LDK;           // [dv][LDK]
  float* Lt = Vs + dv * LDK;          // [SK_KB][LDL]
  float* Rt = Lt + SK_KB * LDL;       // [SK_KB][LDR]
  float* Cs = Rt + SK_KB * LDR;       // [d] the sketch's centre

  const long long k_begin = split * keys_per_split;
  long long k_end = k_begin + keys_per_split;
  if (k_end > n) k_end = n;

  const float* Kh = K + head * hkeys * d;     // hkeys: keys between heads (>= n)
  const float* Vh = V + head * hkeys * dv;

  // Feature assignment (fixed for the whole key loop): row rL of the L tile for
  // keys kpL + STEPL*u, column cR of the R tile for keys kpR + STEPR*u.
  const int s = T.s, t = T.t;
  const int dmask = d - 1;
  const int rL = tid % TM, kpL = tid / TM;
  const int gL = T.row0 + rL;
  const bool validL = gL < T.M;
  int dl[SK_MAXDIG];   // LDS offsets of the key components named by the digits
#pragma unroll
  for (int c = 0; c < SK_MAXDIG; ++c)
    dl[c] = ((c < s) ? ((gL >> (logd * (s - 1 - c))) & dmask) : 0) * LDK + kpL;

  const int cR = tid % TN, kpR = tid / TN;
  const int gR = T.col0 + cR;
  const bool validR = gR < T.N;
  const int alo = gR / T.C;             // trailing Kronecker digits of the column
  const int e = gR - alo * T.C;         // position inside u
  int dr[SK_MAXDIG];
#pragma unroll
  for (int c = 0; c < SK_MAXDIG; ++c)
    dr[c] = ((c < t) ? ((alo >> (logd * (t - 1 - c))) & dmask) : 0) * LDK + kpR;
  // u = [k, v] below the top level, u = v at the top level
  const float* usrc = ((!T.top && e < d) ? Ks + e * LDK
                                         : Vs + (T.top ? e : e - d) * LDK) + kpR;

  const int wr0 = (wave / WC) * 64;
  const int wc0 = (wave % WC) * 64;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  floatx16 acc00 = {0}, acc01 = {0}, acc10 = {0}, acc11 = {0};

  const int nK4 = SK_KB * d / 4;
  const int nV4 = SK_KB * dv / 4;
  const int d4 = d >> 2, dv4 = dv >> 2;

  // Next stage's K and V rows are fetched into registers while the MFMAs of the
  // current stage run; rows past the key range read as zero.
  // keys are shifted by the sketch's centre as they are staged into LDS (the
  // centre is kept in LDS); rows past the key range stay zero
  constexpr bool centered = CENTER;
  if (centered) {   // uniform: every thread takes the same branch
    for (int i = tid; i < d; i += SK_WG) Cs[i] = center[head * d + i];
    __syncthreads();
  }
  float4 kreg[NPF], vreg[NPF];
  auto fetch = [&](long long kb0) {
    const long long left = k_end - kb0;
    const int nk = left < SK_KB ? (int)left : SK_KB;
    const float4* Kg = reinterpret_cast<const float4*>(Kh + kb0 * d);
    const float4* Vg = reinterpret_cast<const float4*>(Vh + kb0 * dv);
#pragma unroll
    for (int r = 0; r < NPF; ++r) {
      const int i = tid + r * SK_WG;
      kreg[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      vreg[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < nK4 && i / d4 < nk) kreg[r] = Kg[i];
      if (i < nV4 && i / dv4 < nk) vreg[r] = Vg[i];
    }
  };

  if (k_begin < k_end) fetch(k_begin);
  for (long long kb0 = k_begin; kb0 < k_end; kb0 += SK_KB) {
    // 1. this stage's K and V rows -> LDS, transposed
    const long long left = k_end - kb0;
    const int nk = left < SK_KB ? (int)left : SK_KB;
#pragma unroll
    for (int r = 0; r < NPF; ++r) {
      const int i = tid + r * SK_WG;
      if (i < nK4) {
        const int key = i / d4, c = 4 * (i - key * d4);
        float4 kv = kreg[r];
        if (centered && key < nk) {
          kv.x -= Cs[c]; kv.y -= Cs[c + 1]; kv.z -= Cs[c + 2]; kv.w -= Cs[c + 3];
        }
        Ks[(c + 0) * LDK + key] = kv.x;
        Ks[(c + 1) * LDK + key] = kv.y;
        Ks[(c + 2) * LDK + key] = kv.z;
        Ks[(c + 3) * LDK + key] = kv.w;
      }
      if (i < nV4) {
        const int key = i / dv4, c = 4 * (i - key * dv4);
        Vs[(c + 0) * LDK + key] = vreg[r].x;
        Vs[(c + 1) * LDK + key] = vreg[r].y;
        Vs[(c + 2) * LDK + key] = vreg[r].z;
        Vs[(c + 3) * LDK + key] = vreg[r].w;
      }
    }
    __syncthreads();
    // 2. feature tiles: L = prod of s key entries, R = u[e] * prod of t entries,
    //    all digit reads of a chunk of the thread's keys issued together.
#pragma unroll
    for (int h0 = 0; h0 < NKL; h0 += CHL) {
      float f[CHL];
#pragma unroll
      for (int u = 0; u < CHL; ++u) f[u] = validL ? 1.f : 0.f;
      mul_digits_n<CHL, STEPL>(s, f, Ks, dl, STEPL * h0);
#pragma unroll
      for (int u = 0; u < CHL; ++u) Lt[(kpL + STEPL * (h0 + u)) * LDL + rL] = f[u];
    }
#pragma unroll
    for (int h0 = 0; h0 < NKR; h0 += CHR) {
      float f[CHR];
#pragma unroll
      for (int u = 0; u < CHR; ++u) f[u] = validR ? usrc[STEPR * (h0 + u)] : 0.f;
      mul_digits_n<CHR, STEPR>(t, f, Ks, dr, STEPR * h0);
#pragma unroll
      for (int u = 0; u < CHR; ++u) Rt[(kpR + STEPR * (h0 + u)) * LDR + cR] = f[u];
    }
    __syncthreads();
    if (kb0 + SK_KB < k_end) fetch(kb0 + SK_KB);
    // 3. fp32 MFMA over the stage: two keys per instruction, operands of the
    //    next k-step read while the current ones are in the matrix core
    float a0 = Lt[lhi * LDL + wr0 + l32];
    float a1 = Lt[lhi * LDL + wr0 + 32 + l32];
    float b0 = Rt[lhi * LDR + wc0 + l32];
    float b1 = Rt[lhi * LDR + wc0 + 32 + l32];
#pragma unroll
    for (int ks = 0; ks < SK_KB / 2; ++ks) {
      float na0 = 0.f, na1 = 0.f, nb0 = 0.f, nb1 = 0.f;
      if (ks + 1 < SK_KB / 2) {
        const int kr = 2 * (ks + 1) + lhi;
        na0 = Lt[kr * LDL + wr0 + l32];
        na1 = Lt[kr * LDL + wr0 + 32 + l32];
        nb0 = Rt[kr * LDR + wc0 + l32];
        nb1 = Rt[kr * LDR + wc0 + 32 + l32];
      }
      acc00 = mfma32x32x2(a0, b0, acc00);
      acc01 = mfma32x32x2(a0, b1, acc01);
      acc10 = mfma32x32x2(a1, b0, acc10);
      acc11 = mfma32x32x2(a1, b1, acc11);
      a0 = na0; a1 = na1; b0 = nb0; b1 = nb1;
    }
    __syncthreads();
  }

  // Epilogue: rows of X_j are contiguous, so (row, col) -> xoff + row * N + col.
  // A wave whose 64 rows are all inside the level (nearly every tile) stores
  // without row checks; accumulate is uniform too.
  float* o = out + split * split_stride + head * head_stride + T.xoff;
  const floatx16* accs[4] = {&acc00, &acc01, &acc10, &acc11};
  const bool rows_in = T.row0 + wr0 + 64 <= T.M;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    const int i = bi >> 1, jj = bi & 1;
    const int col = T.col0 + wc0 + 32 * jj + l32;
    if (col >= T.N) continue;
    const floatx16 a = *accs[bi];
    float* ob = o + (long long)(T.row0 + wr0 + 32 * i) * T.N + col;
    if (rows_in && !accumulate) {
#pragma unroll
      for (int r = 0; r < 16; ++r) ob[(long long)acc_row(r, lane) * T.N] = a[r];
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = T.row0 + wr0 + 32 * i + acc_row(r, lane);
        if (row < T.M) {
          float* dst = ob + (long long)acc_row(r, lane) * T.N;
          *dst = accumulate ? *dst + a[r] : a[r];
        }
      }
    }
  }
}

// One launch covers every tile of every level; the tile's shape picks the body.
template <bool CENTER, int NPF>
__global__ __launch_bounds__(SK_WG, 2)
void sk_update_kernel(const float* __restrict__ K, const float* __restrict__ V,
                      long long n, long long hkeys, int d, int dv, int logd,
                      const UpdTile* __restrict__ tiles, int ntiles,
                      long long keys_per_split, int nsplit, int nhead,
                      float* __restrict__ out, long long head_stride,
                      long long split_stride, int accumulate,
                      const float* __restrict__ center, PendingReduce red) {
  // 1-D grid over (tile, split, head), tile fastest, remapped per XCD; blocks
  // past them add the previous call's partials into the state
  const long long total = (long long)ntiles * nsplit * nhead;
  if ((long long)blockIdx.x >= total) {
    pending_reduce_wg(red, (long long)blockIdx.x - total);
    return;
  }
  const long long lg = xcd_remap(blockIdx.x, total);
  const int tile_id = (int)(lg % ntiles);
  const long long split = (lg / ntiles) % nsplit;
  const long long head = lg / ((long long)ntiles * nsplit);
  const UpdTile T = tiles[tile_id];
  if (T.wc == 2)
    sk_update_tile<2, CENTER, NPF>(K, V, n, hkeys, d, dv, logd, T, split, head, keys_per_split, out,
                      head_stride, split_stride, accumulate, center);
  else if (T.wc == 1)
    sk_update_tile<1, CENTER, NPF>(K, V, n, hkeys, d, dv, logd, T, split, head, keys_per_split, out,
                      head_stride, split_stride, accumulate, center);
  else
    sk_update_tile<4, CENTER, NPF>(K, V, n, hkeys, d, dv, logd, T, split, head, keys_per_split, out,
                      head_stride, split_stride, accumulate, center);
}
