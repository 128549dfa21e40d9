// Query of the multiset storage by the last index, for blocks of at least 32
// columns, d <= 64 and multisets of at most two indices: the counterpart of
// sk_query_dgr_kernel for the rows of one multiset size j.
// Source: "Rumo a Limites Estritos para Atenção em Streaming", "Metodologia",
// pillar "O Método Polinomial" (answering from the low-degree moments; the
// pages leave their storage open).
//
// The rows of size j come in runs that share a prefix (the multiset minus its
// largest index): for prefix beta' the run holds beta' + {e} for e = lb .. d - 1
// (lb = the largest index of beta', 0 for the empty prefix), consecutive in the
// block.  A stage of 64 rows holds NF = 64 / d slots of d rows.  A slot holds
// one run a at positions e = lb_a .. d - 1 and, below them, a second run b
// reversed in pairs of positions: index e of run b sits at position
// (d - 1 - e) xor 1, which keeps e's parity, so for every row the lane's query
// component is a register at a compile-time index.  Run b fits when its
// positions (up to d - lb_b - 1, or d - lb_b when that length is odd) stay below
// lb_a rounded down to even, so that the two rows of a k-step (positions 2 i and
// 2 i + 1) always belong to the same run.  The planner pairs long runs with short
// ones, so a level of runs shrinking from d rows to 1 fills its stages.  Row beta' + {e} has the query feature
//     q^(beta' + e) / (beta' + e)! = [q^beta' / beta'!] * q[e] * h
// with h = 1 / (multiplicity of e in beta' + 1) (only e = lb can repeat an index
// of beta').  The bracket is one number per run and query (its component loaded
// a stage ahead); q[e] is the lane's query component in a register at a
// compile-time index of the position (q[p] for run a, q[(d - 1 - p) xor 1] for
// run b, both in the lane's half of the components); h scales the state row
// when it is staged.  Below the top level, column e' < d of row beta holds the
// moment of beta + {e'}, weighted 1 / (multiplicity of e' in beta + 1) relative
// to the row (0 for e' below the row's largest index, whose entries repeat
// others), also applied when staging; the epilogue multiplies those columns by
// q[e'].  k-step groups with no row of
// either run are skipped (wave-uniform).
//
// Everything else follows sk_query_dgr_kernel: v_mfma_f32_32x32x2_f32, 128
// queries (32 per wave) x up to 64 columns per workgroup, state rows through
// double-buffered LDS by bounded buffer loads (rows past the level's last row,
// of empty slots, and columns outside the tile read zeros), one barrier per
// stage, the stage's rows read from LDS a group of k-steps ahead.
#pragma once

#include "sk_common.h"
#include "sk_query_dg.h"
#include "sk_sym.h"

#define SD_R 64            // rows per stage

// Largest multiset size j whose levels the kernel takes (a run's prefix holds at
// most one index).
__host__ __device__ constexpr int sd_max_j(int) { return 2; }

// 1 / k for the multiplicities k = 1, 2, 3 that rows of at most two indices give
// (each the correctly rounded quotient; h / 3 for h = 1 / 2 is then exact too).
__device__ __forceinline__ float sd_recip(int k) {
  return k == 1 ? 1.f : (k == 2 ? 0.5f : 1.f / 3.f);
}

// One run: beta' + {e} for e = lb .. d - 1 (lb = d: no rows).
struct SymDgRun {
  int row0;                // level row of e = 0 (that of e = lb, less lb)
  int lb;                  // first index of the run
  int mlb;                 // multiplicity of lb in beta' (0 for the empty prefix)
  float winv;              // 1 / beta'!
  unsigned long long code; // beta' indices in bytes 0 .. j - 2
};

// One (level, column tile, range of slots) of the multiset query; slot s is the
// run pair runs[2 s] (a, forward) and runs[2 s + 1] (b, reversed).
struct SymDgTile {
  long long xoff;          // float offset of the level's first row in one head's state
  long long pofs;          // offset of the tile's [128][fw] partial in a query-tile block
  int nrows;               // rows of the level
  int C;                   // the block's width (d + dv, or dv at the top)
  int top;
  int j;                   // multiset size of the level's rows
  int col0, fw;            // the tile's columns
  int run0, nrun;          // slots of the tile in the slot table
  int pad_[2];
};

template <int LOGD, int NT>
__device__ __forceinline__ void sd_tile_loop(const SymDgTile& T, const SymDgRun* __restrict__ runs,
                                             const float* __restrict__ Xl,
                                             __amdgpu_buffer_rsrc_t rq, unsigned qoff, float* Bs,
                                             const float* qr, int d_, int tid, int lhi, int l32,
                                             floatx16* acc) {
  constexpr int d = 1 << LOGD;
  constexpr int NF = SD_R / d;                  // slots per stage
  constexpr int LDB = 32 * SK_DGNT + 32;
  constexpr int KS = SD_R / 2;
  constexpr int KG = 4;
  constexpr int NG = KS / KG;
  constexpr int W4 = 8 * NT;
  constexpr int PV = SD_R * W4 / SK_WG;
  const int C = T.C, col0 = T.col0, gw = T.fw, j = T.j;
  const bool lower = !T.top;
  if (j == 0) {
    // the empty multiset: one row, feature 1, every column weighted 1
    if (tid < W4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * tid < gw) v = *reinterpret_cast<const float4*>(Xl + col0 + 4 * tid);
      *reinterpret_cast<float4*>(Bs + 4 * tid) = v;
    }
    __syncthreads();
    const float a = lhi == 0 ? 1.f : 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = mfma32x32x2(a, lhi == 0 ? Bs[32 * t + l32] : 0.f, acc[t]);
    return;
  }
  const int nst = (T.nrun + NF - 1) / NF;
  const __amdgpu_buffer_rsrc_t rx = dg_rsrc(Xl, (unsigned)((long long)T.nrows * C * 4));
  // the thread's stage positions: slot row f d + p, float4 c4 of the tile's columns
  int prow[PV], pc4[PV];
#pragma unroll
  for (int v = 0; v < PV; ++v) {
    const int i = tid + v * SK_WG;
    prow[v] = i / W4;
    pc4[v] = i - prow[v] * W4;
  }
  float4 pre[PV];
  int em[PV];              // the staged rows' last index e | its multiplicity in the row << 8
  // a thread's positions v cover rows v S .. v S + S - 1 of the stage (S = SK_WG /
  // W4 threads per row block); when S <= d they lie in one slot, known per v
  constexpr int S = SK_WG / W4;
  auto fetch = [&](int st) {
#pragma unroll
    for (int v = 0; v < PV; ++v) {
      const int f = S <= d ? (v * S) >> LOGD : prow[v] >> LOGD;
      const int p = prow[v] & (d - 1);
      const int r = st * NF + f;
      unsigned off = DG_OOB;
      int e = p, mult = 1;
      if (r < T.nrun) {
        const SymDgRun A = runs[2 * (T.run0 + r)];
        const SymDgRun B = runs[2 * (T.run0 + r) + 1];
        const int eb = (d - 1 - p) ^ 1;
        const bool ina = p >= A.lb;
        const bool in = ina || eb >= B.lb;
        e = ina ? p : eb;
        const int row = (ina ? A.row0 : B.row0) + e;
        if (in && 4 * pc4[v] < gw)
          off = (unsigned)(((long long)row * C + col0 + 4 * pc4[v]) * 4);
        // e = lb may repeat the largest index of beta': the row's multiplicity of
        // e is then mlb + 1, and its weight relative to beta' 1 / (mlb + 1)
        mult = (in && e == (ina ? A.lb : B.lb) ? (ina ? A.mlb : B.mlb) : 0) + 1;
      }
      pre[v] = dg_ld4(rx, off);
      em[v] = e | (mult << 8);
    }
  };
  // column weights of a staged float4 (rows below the top): e' < e -> 0, e' = e ->
  // 1 / (multiplicity of e in the row + 1), e' > e -> 1; columns >= d -> 1
  auto store = [&](float* B) {
#pragma unroll
    for (int v = 0; v < PV; ++v) {
      float4 x = pre[v];
      const int e = em[v] & 0xff, mult = em[v] >> 8;
      const float h = sd_recip(mult);
      const int c = col0 + 4 * pc4[v];
      float w[4] = {h, h, h, h};
      if (lower) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ec = c + u;
          if (ec < d_) w[u] = ec > e ? h : (ec == e ? h * sd_recip(mult + 1) : 0.f);
        }
      }
      x.x *= w[0]; x.y *= w[1]; x.z *= w[2]; x.w *= w[3];
      *reinterpret_cast<float4*>(B + prow[v] * LDB + 4 * pc4[v]) = x;
    }
  };
  // prefix component of each run of stage st's slots (j = 2; none for j = 1); the
  // brackets q^beta' / beta'! formed at the stage
  float pc[2 * NF];
  auto pfetch = [&](int st) {
#pragma unroll
    for (int i = 0; i < 2 * NF; ++i) {
      const int r = st * NF + i / 2;
      pc[i] = 1.f;
      if (j == 2 && r < T.nrun)
        pc[i] = sk_ld(rq, qoff, (unsigned)(runs[2 * (T.run0 + r) + (i & 1)].code & 0xffu) * 4u);
    }
  };
  auto pform = [&](int st, float* pf, int* lbs) {
#pragma unroll
    for (int i = 0; i < 2 * NF; ++i) {
      const int r = st * NF + i / 2;
      float x = 0.f;
      int lb = d;
      if (r < T.nrun) {
        const SymDgRun R = runs[2 * (T.run0 + r) + (i & 1)];
        x = R.winv * pc[i];
        lb = R.lb;
      }
      pf[i] = x;
      lbs[i] = lb;
    }
  };
  fetch(0);
  pfetch(0);
  for (int st = 0; st < nst; ++st) {
    float* B = Bs + (st & 1) * (SD_R * LDB);
    store(B);
    float pf[2 * NF];
    int lbs[2 * NF];
    pform(st, pf, lbs);
    __syncthreads();
    if (st + 1 < nst) {
      fetch(st + 1);
      pfetch(st + 1);
    }
    const float* Bl = B + lhi * LDB + l32;
    float bv[2][KG][NT];
    auto rd = [&](int g, float (*dst)[NT]) {
#pragma unroll
      for (int k = 0; k < KG; ++k)
#pragma unroll
        for (int t = 0; t < NT; ++t) dst[k][t] = Bl[2 * (g * KG + k) * LDB + 32 * t];
    };
    // group g holds slot rows 8 g .. 8 g + 7: positions (8 g) mod d .. + 7 of slot
    // (8 g) / d (8 <= d), or all of slots 2 g and 2 g + 1 (d = 4)
    auto live = [&](int g) {
      constexpr int GR = 2 * KG;
      if constexpr (d >= GR) {
        const int f = (GR * g) / d, p0 = (GR * g) % d;
        return p0 + GR - 1 >= lbs[2 * f] || p0 <= d - 1 - lbs[2 * f + 1];
      } else {
        const int f = (GR * g) / d;
        return lbs[2 * f] < d || lbs[2 * f + 1] < d || lbs[2 * f + 2] < d || lbs[2 * f + 3] < d;
      }
    };
    rd(0, bv[0]);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) rd(g + 1, bv[(g + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (live(g)) {
        // the lane's row is position 2 i + lhi of slot f: run a's from lb_a rounded
        // down to even on (rows below lb_a there are zeros), run b's of index
        // (d - 1 - 2 i - lhi) xor 1 = 2 (d/2 - 1 - i) + lhi below; the boundary is
        // even, so both rows of a k-step take the same run
#pragma unroll
        for (int k = 0; k < KG; ++k) {
          const int ks = g * KG + k;
          const int f = (2 * ks) / d, i = ks % (d / 2);
          const bool ra = 2 * i >= (lbs[2 * f] & ~1);   // wave-uniform
          const float a = ra ? pf[2 * f] * qr[i] : pf[2 * f + 1] * qr[d / 2 - 1 - i];
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = mfma32x32x2(a, bv[g & 1][k][t], acc[t]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int LOGD>
__global__ __launch_bounds__(SK_WG, 2)
void sk_sym_dg_kernel(const float* __restrict__ Q, long long m, const float* __restrict__ X,
                      long long head_stride, const SymDgTile* __restrict__ tiles, int ntiles,
                      const SymDgRun* __restrict__ runs, int nqt, long long PB,
                      float* __restrict__ parts) {
  constexpr int d = 1 << LOGD;
  static_assert(d <= 64, "d / 2 query components per lane");
  extern __shared__ float lds[];
  float* Bs = lds;                            // [2][SD_R][LDB]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lhi = lane >> 5;
  const long long lg = blockIdx.x;
  const int tile_id = (int)(lg % ntiles);
  const int qt = (int)((lg / ntiles) % nqt);
  const long long head = lg / ((long long)nqt * ntiles);
  const SymDgTile T = tiles[tile_id];
  const long long q0 = (long long)qt * SK_DGQ;
  const long long nq = m - q0 < SK_DGQ ? m - q0 : SK_DGQ;
  const float* Qh = Q + (head * m + q0) * d;
  const __amdgpu_buffer_rsrc_t rq = dg_rsrc(Qh, (unsigned)(nq * d * 4));
  const int ql0 = wave * 32 + l32;
  const unsigned qoff = (unsigned)(ql0 * d * 4);
  float qr[d / 2];
#pragma unroll
  for (int i = 0; i < d / 2; ++i) qr[i] = sk_ld(rq, qoff + 4u * lhi, 8u * i);
  const float* Xl = X + head * head_stride + T.xoff;
  floatx16 acc[SK_DGNT];
#pragma unroll
  for (int t = 0; t < SK_DGNT; ++t) acc[t] = floatx16{0};
  if ((T.fw + 31) / 32 == 1)
    sd_tile_loop<LOGD, 1>(T, runs, Xl, rq, qoff, Bs, qr, d, tid, lhi, l32, acc);
  else
    sd_tile_loop<LOGD, SK_DGNT>(T, runs, Xl, rq, qoff, Bs, qr, d, tid, lhi, l32, acc);

  // epilogue: columns e' < d of a lower level times q[e'], then the [128][fw]
  // partial of columns col0 ..
  float* P = parts + (head * nqt + qt) * PB + T.pofs;
#pragma unroll
  for (int t = 0; t < SK_DGNT; ++t) {
    const int cr = 32 * t + l32;
    const int col = T.col0 + cr;
    if (cr < T.fw) {
      const bool zcol = (!T.top) && (col < d);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = wave * 32 + acc_row(r, lane);
        float w = 1.f;
        if (zcol) w = (q0 + ql < m) ? Qh[(long long)ql * d + col] : 0.f;
        P[(long long)ql * T.fw + cr] = acc[t][r] * w;
      }
    }
  }
}
