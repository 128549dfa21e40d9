// Query of one level by its last digit: Y_j[q][e] = sum_a q^(x)j[a] X_j[a][e] with
// every row a of the level on the GEMM's reduction side and every column e of
// the level (C = d + dv, or dv at the top) on its output side (no trailing digit
// folded into the columns).
// Source: "Rumo a Limites Estritos para Atenção em Streaming", "Metodologia",
// pillar "O Método Polinomial" (answering from the low-degree moments).
//
// Row a = (F, b), F its leading j - 1 digits and b its last digit, has the query
// feature q^(x)j[a] = P_F(q) q[b] with P_F(q) = prod of q over the digits of F.
// So an MFMA's A operand is one query component (from LDS) times a per-prefix
// product (one multiply per lane), and no feature tile is built: the B operand is
// the state rows, staged through double-buffered LDS (one barrier per 32-row
// stage, the next stage's rows fetched into registers during the current one).
// One workgroup = 128 queries (4 waves x 32) x up to 64 columns x a range of
// rows; it writes a [128][fw] partial of its columns, with the column weights
// q[e]/(j+1)! (e < d, below the top) or 1/j!.
//   sk_query_dg_kernel<LOGD>      v_mfma_f32_32x32x2_f32, one or two 32-column
//                                  tiles per wave (C > 16: levels wider than 64
//                                  columns take several 64-column tiles, each with
//                                  its own partial of those columns), every level
//                                  in one launch; the query component from LDS
//   sk_query_dg16_kernel<LOGD>    v_mfma_f32_16x16x4_f32 for 8 < C <= 16 (d <= 16),
//                                  two 16-query tiles per wave, the query
//                                  components in registers
#pragma once

#include "sk_common.h"

#define SK_DGQ 128        // queries per workgroup
#define SK_DGK 32         // rows per stage
#define SK_DGNT 2         // 32-column tiles per wave at most (64-column records)

// Largest-digit-first product of q over the j - 1 leading digits of row index
// F * d + b, i.e. over the digits of F; qs = the query's column of the LDS tile
// (stride ldq per component).
template <int LOGD>
__device__ __forceinline__ float dg_prefix(const float* qs, int ldq, long long F, int nd) {
  float p = 1.f;
  for (int i = 0; i < nd; ++i) {
    p *= qs[(int)(F & ((1 << LOGD) - 1)) * ldq];
    F >>= LOGD;
  }
  return p;
}

// The k-loop of one tile with NT (1 or 2) 32-column tiles per wave: stages of 32
// rows through the double-buffered Bs (row stride LDB), the A operand the lane's
// query component times the stage's prefix, operands read two k-steps ahead.
template <int LOGD, int NT, int LDQ, int LDB>
__device__ __forceinline__ void dg_tile_loop(const QryTile& T, const float* __restrict__ Xh,
                                             float* Bs, const float* qcol, int tid, int lhi,
                                             int l32, floatx16* acc) {
  constexpr int d = 1 << LOGD;
  constexpr int NF = (SK_DGK >> LOGD) > 0 ? (SK_DGK >> LOGD) : 1;   // prefixes per stage
  constexpr int KPF = SK_DGK / 2 / NF;        // k-steps per prefix
  constexpr int W4 = 8 * NT;                  // float4 per stage row
  const int C = T.C, j = T.level, col0 = T.col0, w = T.fw;
  const int ndig = j > 0 ? j - 1 : 0;
  // a stage: 32 rows x 8 NT float4 (columns col0 ..; those >= col0 + w are zero),
  // NT float4 per thread
  float4 pre[NT];
  auto fetch = [&](long long r0) {
#pragma unroll
    for (int v = 0; v < NT; ++v) {
      const int i = tid + v * SK_WG;
      const int row = i / W4, c4 = i - row * W4;
      pre[v] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r0 + row < T.a1 && 4 * c4 < w)
        pre[v] = *reinterpret_cast<const float4*>(Xh + (r0 + row) * C + col0 + 4 * c4);
    }
  };
  auto store = [&](float* dst) {
#pragma unroll
    for (int v = 0; v < NT; ++v) {
      const int i = tid + v * SK_WG;
      const int row = i / W4, c4 = i - row * W4;
      *reinterpret_cast<float4*>(dst + row * LDB + 4 * c4) = pre[v];
    }
  };
  if (j == 0) {
    // level 0: one row, feature 1
    fetch(0);
    store(Bs);
    __syncthreads();
    const float a = lhi == 0 ? 1.f : 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma32x32x2(a, Bs[lhi * LDB + 32 * t + l32], acc[t]);
    return;
  }
  if (T.a0 < T.a1) fetch(T.a0);
  int buf = 0;
  for (long long r0 = T.a0; r0 < T.a1; r0 += SK_DGK, buf ^= 1) {
    const float* B = Bs + buf * (SK_DGK * LDB);
    store(Bs + buf * (SK_DGK * LDB));
    __syncthreads();
    if (r0 + SK_DGK < T.a1) fetch(r0 + SK_DGK);
    // the stage's rows r0 .. r0 + 31 (r0 a multiple of 32): last digits from
    // b0 = r0 mod d (d >= 32) or from the row alone (d < 32), prefixes per d rows
    float pf[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
      pf[f] = dg_prefix<LOGD>(qcol, LDQ, (r0 + f * (SK_DGK / NF)) >> LOGD, ndig);
    const float* qb = qcol + (d >= SK_DGK ? (int)(r0 & (d - 1)) : 0) * LDQ;
    auto qidx = [&](int ks) {
      const int row = 2 * ks + lhi;
      return (d >= SK_DGK ? row : (row & (d - 1))) * LDQ;
    };
    float qv[3], bv[3][NT];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      qv[u] = qb[qidx(u)];
#pragma unroll
      for (int t = 0; t < NT; ++t) bv[u][t] = B[(2 * u + lhi) * LDB + 32 * t + l32];
    }
#pragma unroll
    for (int ks = 0; ks < SK_DGK / 2; ++ks) {
      if (ks + 2 < SK_DGK / 2) {
        qv[(ks + 2) % 3] = qb[qidx(ks + 2)];
#pragma unroll
        for (int t = 0; t < NT; ++t)
          bv[(ks + 2) % 3][t] = B[(2 * (ks + 2) + lhi) * LDB + 32 * t + l32];
      }
      const float a = pf[ks / KPF] * qv[ks % 3];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = mfma32x32x2(a, bv[ks % 3][t], acc[t]);
    }
  }
}

template <int LOGD>
__global__ __launch_bounds__(SK_WG, 2)
void sk_query_dg_kernel(const float* __restrict__ Q, long long m,
                        const float* __restrict__ X, long long head_stride,
                        const QryTile* __restrict__ tiles, int ntiles, int nqt,
                        long long PB, float* __restrict__ parts) {
  constexpr int d = 1 << LOGD;
  // Qs row stride 161 = 33 mod 64 banks: the A operand's two lane halves (rows b
  // and b + 1), the epilogue's column reads and the prologue's stores all fall
  // on distinct banks; Bs row stride 96 = 32 mod 64 banks for the same reason
  constexpr int LDQ = SK_DGQ + 33;
  constexpr int LDB = 32 * SK_DGNT + 32;
  extern __shared__ float lds[];
  float* Qs = lds;                            // [d][LDQ]
  float* Bs = Qs + d * LDQ;                   // [2][SK_DGK][LDB]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lhi = lane >> 5;
  const long long lg = blockIdx.x;
  // tile slowest (the grid is tiles x heads x query tiles): the launch
  // dispatches the tiles in plan order, the longest first, each for every head
  // and query tile
  const long long per_tile = (long long)gridDim.x / ntiles;
  const int tile_id = (int)(lg / per_tile);
  const int qt = (int)(lg % nqt);
  const long long head = (lg % per_tile) / nqt;
  const QryTile T = tiles[tile_id];
  const long long q0 = (long long)qt * SK_DGQ;
  {
    // the query tile: every load of a thread issued before its LDS stores
    const float* Qh = Q + (head * m + q0) * d;
    const long long qrem = m - q0;
    constexpr int QV = (SK_DGQ * d / 4 + SK_WG - 1) / SK_WG;   // float4 per thread
    float4 qv4[QV];
#pragma unroll
    for (int v = 0; v < QV; ++v) {
      const int i = tid + v * SK_WG;             // float4 index
      const int qq = (4 * i) >> LOGD;
      qv4[v] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < SK_DGQ * d / 4 && qq < qrem) qv4[v] = reinterpret_cast<const float4*>(Qh)[i];
    }
#pragma unroll
    for (int v = 0; v < QV; ++v) {
      const int i = tid + v * SK_WG;
      if (i < SK_DGQ * d / 4) {
        const int qq = (4 * i) >> LOGD, c = (4 * i) & (d - 1);
        Qs[c * LDQ + qq] = qv4[v].x;
        Qs[(c + 1) * LDQ + qq] = qv4[v].y;
        Qs[(c + 2) * LDQ + qq] = qv4[v].z;
        Qs[(c + 3) * LDQ + qq] = qv4[v].w;
      }
    }
  }
  __syncthreads();
  const float* Xh = X + head * head_stride + T.xoff;
  const float* qcol = Qs + wave * 32 + l32;   // the lane's query (A operand row)
  floatx16 acc[SK_DGNT];
#pragma unroll
  for (int t = 0; t < SK_DGNT; ++t) acc[t] = floatx16{0};
  const int nt = (T.fw + 31) / 32;
  if (nt == 1)
    dg_tile_loop<LOGD, 1, LDQ, LDB>(T, Xh, Bs, qcol, tid, lhi, l32, acc);
  else
    dg_tile_loop<LOGD, SK_DGNT, LDQ, LDB>(T, Xh, Bs, qcol, tid, lhi, l32, acc);

  // epilogue: column weights, then the [128][fw] partial of columns fc0 ..
  float* P = parts + (head * nqt + qt) * PB + T.pofs;
#pragma unroll
  for (int t = 0; t < SK_DGNT; ++t) {
    const int cr = 32 * t + l32;               // column inside the record
    const int col = T.fc0 + cr;                // column of the level
    if (cr < T.fw) {
      const bool zcol = (!T.top) && (col < d);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = wave * 32 + acc_row(r, lane);
        const float w = zcol ? Qs[col * LDQ + ql] * T.wz : T.wn;
        P[(long long)ql * T.fw + cr] = acc[t][r] * w;
      }
    }
  }
}

// sk_query_dgr_kernel<LOGD>: the same contraction for d <= 64 with the query
// components in registers instead of an LDS tile.  A stage holds R = 64 rows (32
// at d = 4; it starts at a multiple of R, so a row's last digit is its row within the
// stage mod d, a compile-time index after unrolling); lane (l32, lhi) keeps its
// query's d / 2 components of parity lhi.  With no query tile in LDS only the two
// stage buffers remain there, so more workgroups fit.
//
// Every global read is a raw buffer load against a resource whose range ends
// where the data ends (the tile's rows, the workgroup's queries): a load past it
// returns zero, so a partial stage, the columns outside a narrow tile and the
// queries past m need no branches; a lane with nothing to load points its offset
// past every range (DG_OOB).  The next stage's rows and the query components of
// its prefixes P_F are loaded while the current stage runs, and the state rows of
// a stage are read from LDS one group of k-steps ahead of the MFMAs that use them
// (scheduling barriers keep that order).
//
// A level of C = 8 or 16 columns fills only part of a 32-column MFMA tile, one of
// 32 columns half of a 64-column tile; such a level's tiles (T.t == 1) move its
// last digit b' to the column side: rows are the j - 1 leading digits F (row
// length N = d C), columns (b', e), and the epilogue weights column (b', e) with
// q[b'] and sums over b' (lane shuffles inside each 32-lane half for C < 32, then
// over the wave's column tiles) into a [128][C] partial.
#define DG_OOB 0x80000000u

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dg_rsrc(const float* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ float4 dg_ld4(__amdgpu_buffer_rsrc_t r, unsigned voff) {
  // (the whole vector is reinterpreted at once: bit casts of single elements of
  // the loaded vector compiled to one dword load broadcast to all four)
  const floatx4v v =
      __builtin_bit_cast(floatx4v, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// High digits of F whose query components are loaded a stage ahead; deeper
// digits (levels of narrow keys beyond these) are loaded when used.
template <int LOGD>
struct DgDigits {
  static constexpr int d = 1 << LOGD;
  // rows per stage: 64 (d itself at d = 64), 32 at d = 4 (whose stages would
  // otherwise take 16 prefixes of two varying digits)
  static constexpr int R = LOGD >= 3 ? (d > 64 ? d : 64) : SK_DGK;
  static constexpr int NF = R >> LOGD;                 // prefixes per stage
  static constexpr int LV = NF > d ? 2 : 1;            // low digits of F varying in a stage
  static constexpr int MAXH = LOGD >= 6 ? 2 : (LOGD == 5 ? 3 : 4);
};

template <int LOGD, int NT>
__device__ __forceinline__ void dgr_tile_loop(const QryTile& T, const float* __restrict__ Xh,
                                              __amdgpu_buffer_rsrc_t rq, unsigned qoff,
                                              float* Bs, const float* qr, int gw, int tid,
                                              int lhi, int l32, floatx16* acc) {
  using G = DgDigits<LOGD>;
  constexpr int d = 1 << LOGD;
  constexpr int R = G::R, NF = G::NF, LV = G::LV, MAXH = G::MAXH;
  constexpr int LDB = 32 * SK_DGNT + 32;
  constexpr int KS = R / 2;                       // k-steps per stage
  constexpr int KG = 4;                           // k-steps per group of LDS reads
  constexpr int NG = KS / KG;
  constexpr int W4 = 8 * NT;                      // float4 per stage row
  constexpr int PV = R * W4 / SK_WG;              // float4 per thread and stage
  static_assert(R * W4 % SK_WG == 0 && KS % KG == 0, "stage shape");
  // row length N (C, or d C with the last digit on the column side), gw GEMM
  // columns from col0, s digits on the row side
  const long long N = T.N;
  if (T.s == 0) {
    // no digit on the row side: one row, feature 1
    if (tid < W4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * tid < gw) v = *reinterpret_cast<const float4*>(Xh + T.col0 + 4 * tid);
      *reinterpret_cast<float4*>(Bs + 4 * tid) = v;
    }
    __syncthreads();
    const float a = lhi == 0 ? 1.f : 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = mfma32x32x2(a, lhi == 0 ? Bs[32 * t + l32] : 0.f, acc[t]);
    return;
  }
  const int ndig = T.s - 1;                       // digits of F
  const long long nrows = T.a1 - T.a0;
  const int nst = (int)((nrows + R - 1) / R);
  // the tile's rows: loads past row a1 return zero
  const __amdgpu_buffer_rsrc_t rx = dg_rsrc(Xh + T.a0 * N, (unsigned)(nrows * N * 4));
  const unsigned sbytes = (unsigned)(R * N * 4);  // bytes per stage
  unsigned voff[PV];
#pragma unroll
  for (int v = 0; v < PV; ++v) {
    const int i = tid + v * SK_WG;
    const int row = i / W4, c4 = i - row * W4;
    voff[v] = (4 * c4 < gw) ? (unsigned)((row * N + T.col0 + 4 * c4) * 4) : DG_OOB;
  }
  float4 pre[PV];
  auto fetch = [&](int st) {
#pragma unroll
    for (int v = 0; v < PV; ++v) pre[v] = dg_ld4(rx, voff[v] + (unsigned)st * sbytes);
  };
  // query component c of the lane's query (c wave-uniform)
  auto qld = [&](int c) { return sk_ld(rq, qoff, (unsigned)c * 4u); };
  // prefix components of stage st: the LV low digits of F0 + f (f < NF) and the
  // MAXH digits above them; unconditional loads (digit 0 where none is needed),
  // the unused ones replaced by 1 when the prefixes are formed
  float plo[NF * LV], phi[MAXH];
  auto pfetch = [&](int st) {
    const long long F0 = (T.a0 + (long long)st * R) >> LOGD;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < LV; ++i)
        plo[f * LV + i] = qld(i < ndig ? (int)(((F0 + f) >> (LOGD * i)) & (d - 1)) : 0);
#pragma unroll
    for (int i = 0; i < MAXH; ++i)
      phi[i] = qld(LV + i < ndig ? (int)((F0 >> (LOGD * (LV + i))) & (d - 1)) : 0);
  };
  auto pform = [&](int st, float* pf) {
    const long long F0 = (T.a0 + (long long)st * R) >> LOGD;
    float h = 1.f;
#pragma unroll
    for (int i = 0; i < MAXH; ++i) h *= (LV + i < ndig) ? phi[i] : 1.f;
    for (int i = LV + MAXH; i < ndig; ++i) h *= qld((int)((F0 >> (LOGD * i)) & (d - 1)));
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      float x = h;
#pragma unroll
      for (int i = 0; i < LV; ++i) x *= (i < ndig) ? plo[f * LV + i] : 1.f;
      pf[f] = x;
    }
  };
  fetch(0);
  pfetch(0);
  for (int st = 0; st < nst; ++st) {
    float* B = Bs + (st & 1) * (R * LDB);
#pragma unroll
    for (int v = 0; v < PV; ++v) {
      const int i = tid + v * SK_WG;
      const int row = i / W4, c4 = i - row * W4;
      *reinterpret_cast<float4*>(B + row * LDB + 4 * c4) = pre[v];
    }
    float pf[NF];
    pform(st, pf);
    __syncthreads();
    if (st + 1 < nst) {
      fetch(st + 1);
      pfetch(st + 1);
    }
    // k-step ks multiplies rows 2 ks and 2 ks + 1 (lane half lhi): last digit
    // (2 ks + lhi) mod d, i.e. register ks mod d/2, prefix ks / (d/2)
    const float* Bl = B + lhi * LDB + l32;
    float bv[2][KG][NT];
    auto rd = [&](int g, float (*dst)[NT]) {
#pragma unroll
      for (int k = 0; k < KG; ++k)
#pragma unroll
        for (int t = 0; t < NT; ++t) dst[k][t] = Bl[2 * (g * KG + k) * LDB + 32 * t];
    };
    rd(0, bv[0]);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) rd(g + 1, bv[(g + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        const int ks = g * KG + k;
        const float a = pf[ks / (d / 2)] * qr[ks % (d / 2)];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma32x32x2(a, bv[g & 1][k][t], acc[t]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int LOGD>
__global__ __launch_bounds__(SK_WG, 2)
void sk_query_dgr_kernel(const float* __restrict__ Q, long long m,
                         const float* __restrict__ X, long long head_stride,
                         const QryTile* __restrict__ tiles, int ntiles, int nqt,
                         long long PB, float* __restrict__ parts) {
  constexpr int d = 1 << LOGD;
  static_assert(d <= 64, "d / 2 query components per lane");
  extern __shared__ float lds[];
  float* Bs = lds;                            // [2][R][LDB]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lhi = lane >> 5;
  const long long lg = blockIdx.x;
  // tile slowest (the grid is tiles x heads x query tiles): the launch
  // dispatches the tiles in plan order, the longest first, each for every head
  // and query tile
  const long long per_tile = (long long)gridDim.x / ntiles;
  const int tile_id = (int)(lg / per_tile);
  const int qt = (int)(lg % nqt);
  const long long head = (lg % per_tile) / nqt;
  const QryTile T = tiles[tile_id];
  const long long q0 = (long long)qt * SK_DGQ;
  // the workgroup's queries: loads past query m - 1 return zero
  const long long nq = m - q0 < SK_DGQ ? m - q0 : SK_DGQ;
  const float* Qh = Q + (head * m + q0) * d;
  const __amdgpu_buffer_rsrc_t rq = dg_rsrc(Qh, (unsigned)(nq * d * 4));
  const int ql0 = wave * 32 + l32;            // the lane's query (A operand row)
  const unsigned qoff = (unsigned)(ql0 * d * 4);
  float qr[d / 2];
#pragma unroll
  for (int i = 0; i < d / 2; ++i) qr[i] = sk_ld(rq, qoff + 4u * lhi, 8u * i);
  const float* Xh = X + head * head_stride + T.xoff;
  floatx16 acc[SK_DGNT];
#pragma unroll
  for (int t = 0; t < SK_DGNT; ++t) acc[t] = floatx16{0};
  // GEMM columns of the tile: its record's fw, or nalo groups of C with the
  // last digit on the column side
  const int gw = T.t ? T.nalo * T.C : T.fw;
  if ((gw + 31) / 32 == 1)
    dgr_tile_loop<LOGD, 1>(T, Xh, rq, qoff, Bs, qr, gw, tid, lhi, l32, acc);
  else
    dgr_tile_loop<LOGD, SK_DGNT>(T, Xh, rq, qoff, Bs, qr, gw, tid, lhi, l32, acc);

  // epilogue: column weights, then the [128][fw] partial of columns fc0 ..  The
  // weights read other queries' components than the lane's own: the workgroup's
  // query tile goes to LDS first (the stage buffers are free once every wave is
  // past its last stage), zeros past query m - 1.
  constexpr int LDQ = d + 1;
  float* Qs = lds;                            // [SK_DGQ][LDQ]
  if (T.t || (!T.top && T.fc0 < d)) {         // uniform
    __syncthreads();
    for (int i = tid; i < SK_DGQ * d / 4; i += SK_WG) {
      const int ql = (4 * i) >> LOGD, c = (4 * i) & (d - 1);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ql < nq) v = *reinterpret_cast<const float4*>(Qh + (long long)ql * d + c);
      float* dst = Qs + ql * LDQ + c;
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
    __syncthreads();
  }
  float* P = parts + (head * nqt + qt) * PB + T.pofs;
  if (T.t) {
    // column (b', e) = col0 + 32 t + l32 (C divides 32): weight q[b'] times e's
    // weight, summed over b' into the [128][C] partial
    const int C = T.C;
    float y[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) y[r] = 0.f;
#pragma unroll
    for (int t = 0; t < SK_DGNT; ++t) {
      if (32 * t < gw) {
        const int gc = T.col0 + 32 * t + l32;
        const int bp = gc / C, e = gc - bp * C;
        const bool zcol = (!T.top) && (e < d);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float* qrow = Qs + (wave * 32 + acc_row(r, lane)) * LDQ;
          y[r] += acc[t][r] * (qrow[bp] * (zcol ? qrow[e] * T.wz : T.wn));
        }
      }
    }
    // lanes l32 and l32 ^ 16 (and ^ 8 when C = 8) of a half share e (C = 32:
    // each lane its own e, the wave's column tiles summed above)
    if (C <= 16) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        y[r] += __shfl_xor(y[r], 16);
        if (C == 8) y[r] += __shfl_xor(y[r], 8);
      }
    }
    if (l32 < C) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = wave * 32 + acc_row(r, lane);
        P[(long long)ql * C + l32] = y[r];
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < SK_DGNT; ++t) {
    const int cr = 32 * t + l32;
    const int col = T.fc0 + cr;
    if (cr < T.fw) {
      const bool zcol = (!T.top) && (col < d);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = wave * 32 + acc_row(r, lane);
        const float w = zcol ? Qs[ql * LDQ + col] * T.wz : T.wn;
        P[(long long)ql * T.fw + cr] = acc[t][r] * w;
      }
    }
  }
}

template <int LOGD>
__global__ __launch_bounds__(SK_WG, 2)
void sk_query_dg16_kernel(const float* __restrict__ Q, long long m,
                          const float* __restrict__ X, long long head_stride,
                          const QryTile* __restrict__ tiles, int ntiles, int nqt,
                          long long PB, float* __restrict__ parts) {
  constexpr int d = 1 << LOGD;
  static_assert(d <= 16, "the 16-column path holds d / 4 query components per tile");
  constexpr int LDQ = SK_DGQ + 1;
  constexpr int LDB = 16 + 4;
  constexpr int NF = SK_DGK >> LOGD;          // prefixes per stage (2, 4 or 8)
  constexpr int KPF = SK_DGK / 4 / NF;        // k-steps per prefix
  constexpr int QR = d / 4;                   // query components per lane and tile
  extern __shared__ float lds[];
  float* Qs = lds;                            // [d][LDQ]
  float* Bs = Qs + d * LDQ;                   // [2][SK_DGK][LDB]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kk = lane >> 4;
  const long long lg = blockIdx.x;
  const int tile_id = (int)(lg % ntiles);
  const int qt = (int)((lg / ntiles) % nqt);
  const long long head = lg / ((long long)nqt * ntiles);
  const QryTile T = tiles[tile_id];
  const int C = T.C, j = T.level;
  const long long q0 = (long long)qt * SK_DGQ;
  {
    const float* Qh = Q + (head * m + q0) * d;
    const long long qrem = m - q0;
    for (int i = tid; i < SK_DGQ * d; i += SK_WG) {
      const int qq = i >> LOGD, c = i & (d - 1);
      Qs[c * LDQ + qq] = (qq < qrem) ? Qh[i] : 0.f;
    }
  }
  __syncthreads();
  const float* Xh = X + head * head_stride + T.xoff;
  const int ndig = j > 0 ? j - 1 : 0;
  // two 16-query tiles per wave: the lane's queries and their components
  // q[4 i + kk] (the last digits b = kk mod 4 the lane's A entries take)
  const float* qc[2];
  float qr[2][QR];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    qc[u] = Qs + wave * 32 + 16 * u + l16;
#pragma unroll
    for (int i = 0; i < QR; ++i) qr[u][i] = qc[u][(4 * i + kk) * LDQ];
  }
  float2 pre;                                  // 32 rows x 16 columns: 2 floats a thread
  auto fetch = [&](long long r0) {
    const int row = tid >> 3, c2 = tid & 7;
    pre = make_float2(0.f, 0.f);
    if (r0 + row < T.a1 && 2 * c2 < C)
      pre = *reinterpret_cast<const float2*>(Xh + (r0 + row) * C + 2 * c2);
  };
  floatx4v acc[2];
  acc[0] = floatx4v{0.f, 0.f, 0.f, 0.f};
  acc[1] = acc[0];
  if (T.a0 < T.a1) fetch(T.a0);
  int buf = 0;
  for (long long r0 = T.a0; r0 < T.a1; r0 += SK_DGK, buf ^= 1) {
    float* B = Bs + buf * (SK_DGK * LDB);
    *reinterpret_cast<float2*>(B + (tid >> 3) * LDB + 2 * (tid & 7)) = pre;
    __syncthreads();
    if (r0 + SK_DGK < T.a1) fetch(r0 + SK_DGK);
    float pf[2][NF];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f)
        pf[u][f] = (j == 0) ? 1.f : dg_prefix<LOGD>(qc[u], LDQ, (r0 + f * (SK_DGK / NF)) >> LOGD, ndig);
#pragma unroll
    for (int ks = 0; ks < SK_DGK / 4; ++ks) {
      const int row = 4 * ks + kk;
      const float bv = B[row * LDB + l16];
      // last digit of row r0 + row: 4 (ks mod d/4) + kk (r0 is a multiple of 32)
      const int bi = ks % QR;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float a = (j == 0) ? (r0 + row == 0 ? 1.f : 0.f) : pf[u][ks / KPF] * qr[u][bi];
        acc[u] = mfma16x16x4(a, bv, acc[u]);
      }
    }
  }
  float* P = parts + (head * nqt + qt) * PB + T.pofs;
  if (l16 < C) {
    const int col = l16;
    const bool zcol = (!T.top) && (col < d);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ql = wave * 32 + 16 * u + 4 * kk + r;
        const float w = zcol ? Qs[col * LDQ + ql] * T.wz : T.wn;
        P[(long long)ql * C + col] = acc[u][r] * w;
      }
  }
}
