// Multiset ("symmetric") storage of the Taylor moments.
//
// The moment tensors M_j = sum_i k_i^(x)j and N_j = sum_i k_i^(x)j v_i^T are
// symmetric in their tensor indices, so one entry per multiset alpha of indices
// carries all of them:  M^s[alpha] = sum_i k_i^alpha,  N^s[alpha] = sum_i k_i^alpha v_i,
// k^alpha = prod_l k[a_l] for the sorted tuple alpha = (a_1 <= ... <= a_j).  An
// entry stands for j!/alpha! tuples of the Kronecker power (alpha! = product of
// the factorials of the multiplicities), so the query weight of an entry is
// q^alpha / alpha! and
//     Zhat(q) = sum_alpha q^alpha M^s[alpha] / alpha!,   Ntilde likewise with N^s.
// Taylor moments of the polynomial method: "Rumo a Limites Estritos para Atenção
// em Streaming", "Metodologia", pillar "O Método Polinomial" (the pages leave the
// storage of the low-degree moments open).
//
// Canonical rows: every multiset of size 0..p, sizes in increasing order and each
// size in lexicographic order of the sorted tuples.  Storage of one head, two
// blocks of raw moments (merge is an addition):
//   lower block, rows = the multisets beta of size < p (R_lo rows), d + dv columns:
//       X[beta][e]     = sum_i k_i^beta k_i[e]      (e < d)
//       X[beta][d + c] = N^s[beta][c]
//   top block, rows = the multisets of size p (R_top rows), dv columns:
//       X[beta][c]     = N^s[beta][c]
// M^s[alpha] of a nonempty alpha is X[beta][e] with beta = alpha minus its largest
// index e (entries with e below the largest index of beta repeat other entries and
// carry no query weight); M^s of the empty multiset is the key count, kept on the
// host.  With u = [k, v] (lower) or u = v (top), each block is the GEMM
//     X += sum_keys  k^beta  u^T
// whose row features are built on chip: k^beta = k^prefix(beta) * k[last(beta)],
// with the prefix products of a stage kept in LDS and the product with the last
// component formed in registers as the MFMA operand.  v_mfma_f32_16x16x4_f32
// (columns in blocks of 16) keeps narrow blocks (d + dv = 16, 32) dense.
#pragma once

#include "sk_common.h"
#include "sk_elementwise.h"

#define SY_KB 32                 // keys per update stage
#ifndef SY_LDK
// row stride of the transposed key/value stage: the A operand reads rows
// last(row) for 16 rows and 4 keys at once; stride 34 puts them on distinct banks
// (32 banks per half-wave)
#define SY_LDK 34
#endif
#define SY_NS 256                // prefix slots per update row tile
#define SY_LDP (SY_NS + 16)      // row stride of the prefix products (bank spread)
#define SY_TQ 128                // queries per query tile
#define SY_QKB 32                // state rows per query stage
#define SY_MAXP 7                // sizes up to 7: digits in bytes 0..6, size in byte 7

// Per-canonical-row tables (device arrays, built once per sketch).
struct SymTables {
  const unsigned long long* code;  // sorted indices in bytes 0..j-1, j in byte 7
  const int* prefix;               // canonical row of alpha minus its largest index; -1 if empty
  const int* last;                 // largest index; d for the empty multiset
  const int* lmul;                 // multiplicity of the largest index (0 if empty)
  const float* winv;               // 1 / alpha!
  const int* rslot;                // slot of the row's prefix in its update row tile
  const int* slots;                // prefix rows of the update row tiles (-1 = empty prefix)
};

// One (row tile, column tile) of a block's update GEMM.
struct SymUpdTile {
  long long xoff;    // float offset of the block in one head's state
  int rc0;           // canonical row of the block's row 0
  int row0, nrows;   // the tile's rows (block rows)
  int col0, C;       // first column; the block's width (d + dv, or dv at the top)
  int top;           // 1 for the top block (u = v)
  int slot0, nslots; // the tile's prefix slots in SymTables::slots
  int cb;            // column blocks of 16 per wave: 1, 2 or 4
  int rb;            // row blocks of 16 per wave: 1, 2 or 4 (tile 64*rb x 16*cb)
};

// One (row range, column tile) of a block's query GEMM
//     Y[q][col] = sum_{beta in range} q^beta * W[beta][col],
// W = the stored entries times their query weights (1/beta! for the N columns;
// for column e < d of the lower block, 1/(beta + e)! if e is at least the largest
// index of beta and 0 otherwise).  The epilogue multiplies column e < d by q[e]
// (its Zhat share) and writes a [SY_TQ][C] partial; column tiles of one row range
// share the partial and write disjoint columns.
struct SymQryTile {
  long long xoff;    // float offset of the block in one head's state
  long long pofs;    // offset of the row range's [SY_TQ][C] partial in a query-tile block
  int rc0;           // canonical row of the block's row 0
  int row0, nrows;   // the range's rows (block rows)
  int col0, C, top;
  int cb;            // column blocks of 16: 1, 2, 4 or 8
  int pad_;
};

// ---------------------------------------------------------------------------
// Update: one workgroup = 4 waves stacked along the rows, each wave 16*RB rows x
// 16*CB columns (RB * CB <= 16 accumulator blocks), so a tile is 64*RB rows and
// at most SY_NS = 256 prefix slots.  Per stage of SY_KB keys:
//   1. the stage's K and V rows -> LDS, transposed ([component][key]), with two
//      extra key rows: all ones (the empty prefix and the empty multiset) and all
//      zeros (rows and columns outside the block);
//   2. prefix products P[key][slot] = k^prefix: thread t owns slot t for the
//      whole tile, with the LDS offsets of its prefix's indices in registers, and
//      reads the stage's keys at compile-time offsets from them;
//   3. per k-step of 4 keys, each lane forms its A operand P[key][slot(row)] *
//      k[last(row)] in a register and reads its B operand u[key][col] from LDS.
// ---------------------------------------------------------------------------
template <int RB, int CB, bool CENTER>
__device__ __forceinline__
void sk_sym_update_tile(const float* __restrict__ K, const float* __restrict__ V,
                        long long n, long long hkeys, int d, int dv, const SymUpdTile& T,
                        const SymTables& tb,
                        long long split, long long head, long long keys_per_split,
                        float* __restrict__ out, long long head_stride,
                        long long split_stride, int accumulate,
                        const float* __restrict__ center) {
  static_assert(RB * CB <= 16 && 64 * RB <= SY_NS, "tile shape");
  constexpr int LDK = SY_LDK;
  constexpr int NPF = 4;              // float4 per thread per stage, for d, dv <= 128
  constexpr int PK = 8;               // keys per pass of the prefix products
  extern __shared__ float lds[];
  float* Ks = lds;                                  // [d + 2][LDK]
  float* Vs = Ks + (d + 2) * LDK;                   // [dv][LDK]
  float* P = Vs + dv * LDK;                         // [SY_KB][SY_LDP]
  float* Cs = P + SY_KB * SY_LDP;                   // [d] the sketch's centre
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;

  const long long k_begin = split * keys_per_split;
  long long k_end = k_begin + keys_per_split;
  if (k_end > n) k_end = n;
  const float* Kh = K + head * hkeys * d;     // hkeys: keys between heads (>= n)
  const float* Vh = V + head * hkeys * dv;

  for (int i = tid; i < LDK; i += SK_WG) {
    Ks[d * LDK + i] = 1.f;
    Ks[(d + 1) * LDK + i] = 0.f;
  }
  // this thread's prefix slot (fixed for the tile; with few slots, up to four
  // threads share a slot and take different chunks of PK keys): the slot's
  // indices as LDS row offsets
  const int ns = T.nslots;
  const int G = ns <= 64 ? 4 : (ns <= 128 ? 2 : 1);
  const bool pown = tid < G * ns;
  const int pslot = pown ? tid % ns : 0;
  const int pc0 = pown ? tid / ns : SY_KB / PK;
  int pcnt = 0;
  int pdo[SY_MAXP - 1];
  {
    const int id = pown ? tb.slots[T.slot0 + pslot] : -1;
    const unsigned long long c = id < 0 ? 0ull : tb.code[id];
    pcnt = (int)(c >> 56);
#pragma unroll
    for (int q = 0; q < SY_MAXP - 1; ++q) pdo[q] = (int)((c >> (8 * q)) & 0xffu) * LDK;
  }

  // A operand: row 16 rb + li of the wave's rows, key 4 ks + lk of the k-step
  int pa[RB], ka[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wave * 16 * RB + 16 * rb + li;
    const bool ok = r < T.nrows;
    const int cid = T.rc0 + T.row0 + r;
    const int slot = ok ? tb.rslot[cid] : 0;
    const int last = ok ? tb.last[cid] : d + 1;
    pa[rb] = lk * SY_LDP + slot;
    ka[rb] = last * LDK + lk;
  }
  // B operand: column 16 cb + li of the tile, key 4 ks + lk
  int ub[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int col = T.col0 + 16 * cb + li;
    int row;
    if (col >= T.C) row = d + 1;                    // zeros
    else if (T.top) row = d + 2 + col;              // Vs row
    else if (col < d) row = col;                    // Ks row
    else row = d + 2 + (col - d);                   // Vs row
    ub[cb] = row * LDK + lk;
  }

  floatx4v acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = floatx4v{0.f, 0.f, 0.f, 0.f};

  const int nK4 = SY_KB * d / 4, nV4 = SY_KB * dv / 4;
  const int d4 = d >> 2, dv4 = dv >> 2;
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
    const int nk = left < SY_KB ? (int)left : SY_KB;
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
  for (long long kb0 = k_begin; kb0 < k_end; kb0 += SY_KB) {
    const long long left = k_end - kb0;
    const int nk = left < SY_KB ? (int)left : SY_KB;
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
    for (int kc = pc0; kc < SY_KB / PK; kc += G) {
      const int k0 = kc * PK;
      float f[PK];
#pragma unroll
      for (int u = 0; u < PK; ++u) f[u] = 1.f;
#pragma unroll
      for (int q = 0; q < SY_MAXP - 1; ++q) {
        if (q < pcnt) {
          const float* src = Ks + pdo[q] + k0;
#pragma unroll
          for (int u = 0; u < PK; ++u) f[u] *= src[u];
        }
      }
      float* dst = P + k0 * SY_LDP + pslot;
#pragma unroll
      for (int u = 0; u < PK; ++u) dst[u * SY_LDP] = f[u];
    }
    __syncthreads();
    if (kb0 + SY_KB < k_end) fetch(kb0 + SY_KB);
#pragma unroll
    for (int ks = 0; ks < SY_KB / 4; ++ks) {
      float b[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) b[cb] = lds[ub[cb] + 4 * ks];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float a = P[pa[rb] + 4 * ks * SY_LDP] * Ks[ka[rb] + 4 * ks];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mfma16x16x4(a, b[cb], acc[rb][cb]);
      }
    }
    __syncthreads();
  }

  float* O = out + head * head_stride + split * split_stride + T.xoff;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = T.col0 + 16 * cb + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wave * 16 * RB + 16 * rb + 4 * lk + r;
        if (row < T.nrows && col < T.C) {
          float* dst = O + (long long)(T.row0 + row) * T.C + col;
          const float v = acc[rb][cb][r];
          *dst = accumulate ? *dst + v : v;
        }
      }
    }
  }
}

// All (tile, key split, head) of one tile shape (RB, CB) in one launch; the 1-D
// grid is remapped so that each XCD takes a contiguous range (tiles that read
// the same keys share an L2).  One kernel per shape keeps each shape's register
// count its own: at most 128 VGPRs, four waves per SIMD, so the stages of other
// workgroups cover the latency of a workgroup's barriers (two waves for the
// 16-block shape, whose accumulators alone take 64 registers).
template <int RB, int CB, bool CENTER>
__global__ __launch_bounds__(SK_WG, (RB * CB >= 16) ? 2 : 4)
void sk_sym_update_kernel(const float* __restrict__ K, const float* __restrict__ V,
                          long long n, long long hkeys, int d, int dv,
                          const SymUpdTile* __restrict__ tiles, int ntiles, SymTables tb,
                          long long keys_per_split, int nsplit, int nhead,
                          float* __restrict__ out, long long head_stride,
                          long long split_stride, int accumulate,
                          const float* __restrict__ center, PendingReduce red) {
  const long long total = (long long)ntiles * nsplit * nhead;
  if ((long long)blockIdx.x >= total) {   // the previous call's partials -> state
    pending_reduce_wg(red, (long long)blockIdx.x - total);
    return;
  }
  const long long lg = xcd_remap(blockIdx.x, total);
  const int tile = (int)(lg % ntiles);
  const long long split = (lg / ntiles) % nsplit;
  const long long head = lg / ((long long)ntiles * nsplit);
  const SymUpdTile T = tiles[tile];
  sk_sym_update_tile<RB, CB, CENTER>(K, V, n, hkeys, d, dv, T, tb, split, head,
                                     keys_per_split, out, head_stride, split_stride,
                                     accumulate, center);
}

// ---------------------------------------------------------------------------
// Query: one workgroup = SY_TQ queries x 16*CB columns x one row range of a
// block.  Wave w owns queries 32 w .. 32 w + 31 (two 16-row blocks) and every
// column block.  Per stage of SY_QKB state rows: the query features q^beta
// (product of the row's indices, read from the query tile in LDS) and the
// weighted state rows go to LDS; the weighted rows of the next stage are fetched
// into registers while the MFMAs run.
// ---------------------------------------------------------------------------
template <int CB>
__device__ __forceinline__
void sk_sym_query_tile(const float* __restrict__ Q, long long m, int d,
                       const float* __restrict__ X, long long head_stride,
                       const SymQryTile& T, const SymTables& tb, int qt, long long head,
                       long long PB, float* __restrict__ parts) {
  constexpr int TN = 16 * CB;
  constexpr int LDQ = SY_TQ + 4;                      // rows 16-byte aligned (float4 reads)
  constexpr int LDA = SY_TQ + 16;                     // rows 16 banks apart
  constexpr int LDB = TN <= 16 ? 16 : (TN + 63) / 64 * 64 + 16;
  constexpr int NB4 = SY_QKB * TN / 4;                // float4 of a weighted stage
  constexpr int NBR = (NB4 + SK_WG - 1) / SK_WG;
  extern __shared__ float lds[];
  float* Qs = lds;                                    // [d][LDQ] query tile, transposed
  float* At = Qs + d * LDQ;                           // [SY_QKB][LDA] features
  float* Bt = At + SY_QKB * LDA;                      // [SY_QKB][LDB] weighted rows
  unsigned long long* Rc =
      reinterpret_cast<unsigned long long*>(Bt + SY_QKB * LDB);   // [SY_QKB] row codes
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;

  const long long q0 = (long long)qt * SY_TQ;
  {
    const float* Qh = Q + (head * m + q0) * d;
    const long long qrem = m - q0;
    for (int i = tid; i < SY_TQ * d; i += SK_WG) {
      const int qq = i / d, c = i - qq * d;
      Qs[c * LDQ + qq] = (qq < qrem) ? Qh[i] : 0.f;
    }
  }
  const float* Xb = X + head * head_stride + T.xoff;
  const int C = T.C;
  const bool lower = !T.top;

  // weighted state rows of the stage starting at block row rb0 -> registers
  float4 breg[NBR];
  auto fetch = [&](int rb0) {
#pragma unroll
    for (int r = 0; r < NBR; ++r) {
      const int i = tid + r * SK_WG;
      breg[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      const int row = i / (TN / 4), c4 = 4 * (i - row * (TN / 4));
      const int br = rb0 + row;                         // block row
      const int col = T.col0 + c4;
      if (i < NB4 && row < SY_QKB && br < T.row0 + T.nrows && col < C) {
        const int cid = T.rc0 + br;
        const float4 x = *reinterpret_cast<const float4*>(Xb + (long long)br * C + col);
        const float w = tb.winv[cid];
        float w4[4] = {w, w, w, w};
        if (lower) {
          const int last = tb.last[cid];
          const float wl = w / (float)(tb.lmul[cid] + 1);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int e = col + u;
            if (e < d) w4[u] = (e > last || last == d) ? w : (e == last ? wl : 0.f);
          }
        }
        breg[r] = make_float4(x.x * w4[0], x.y * w4[1], x.z * w4[2], x.w * w4[3]);
      }
    }
  };

  floatx4v acc[2][CB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = floatx4v{0.f, 0.f, 0.f, 0.f};

  const int fr = tid >> 3, fq = 16 * (tid & 7);       // feature thread: row, first query
  static_assert(SY_QKB * SY_TQ / 16 == SK_WG, "one feature thread per row and 16 queries");
  const int r_end = T.row0 + T.nrows;
  __syncthreads();
  if (T.nrows > 0) fetch(T.row0);
  for (int rb0 = T.row0; rb0 < r_end; rb0 += SY_QKB) {
#pragma unroll
    for (int r = 0; r < NBR; ++r) {
      const int i = tid + r * SK_WG;
      if (i < NB4) {
        const int row = i / (TN / 4), c4 = 4 * (i - row * (TN / 4));
        *reinterpret_cast<float4*>(Bt + row * LDB + c4) = breg[r];
      }
    }
    if (tid < SY_QKB) {
      const int br = rb0 + tid;
      Rc[tid] = br < r_end ? tb.code[T.rc0 + br] : ~0ull;   // size 255: outside
    }
    __syncthreads();
    // features q^beta: thread (row fr, queries fq .. fq + 15), the row's indices
    // decoded once and each one's 16 query components read as four float4
    {
      const unsigned long long c = Rc[fr];
      const int cnt = (int)(c >> 56);
      float4 f[4];
#pragma unroll
      for (int v = 0; v < 4; ++v)
        f[v] = cnt == 255 ? make_float4(0.f, 0.f, 0.f, 0.f) : make_float4(1.f, 1.f, 1.f, 1.f);
      if (cnt != 255) {
        for (int k = 0; k < cnt; ++k) {
          const float* qs = Qs + (int)((c >> (8 * k)) & 0xffu) * LDQ + fq;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float4 x = *reinterpret_cast<const float4*>(qs + 4 * v);
            f[v].x *= x.x; f[v].y *= x.y; f[v].z *= x.z; f[v].w *= x.w;
          }
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) *reinterpret_cast<float4*>(At + fr * LDA + fq + 4 * v) = f[v];
    }
    __syncthreads();
    if (rb0 + SY_QKB < r_end) fetch(rb0 + SY_QKB);
#pragma unroll
    for (int ks = 0; ks < SY_QKB / 4; ++ks) {
      const int kr = 4 * ks + lk;
      float b[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) b[cb] = Bt[kr * LDB + 16 * cb + li];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float a = At[kr * LDA + 32 * wave + 16 * rb + li];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mfma16x16x4(a, b[cb], acc[rb][cb]);
      }
    }
    __syncthreads();
  }

  // epilogue: column e < d of the lower block times q[e]; [SY_TQ][C] partial
  float* Pp = parts + (head * ((m + SY_TQ - 1) / SY_TQ) + qt) * PB + T.pofs;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = T.col0 + 16 * cb + li;
      if (col < C) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ql = 32 * wave + 16 * rb + 4 * lk + r;
          float v = acc[rb][cb][r];
          if (lower && col < d) v *= Qs[col * LDQ + ql];
          Pp[(long long)ql * C + col] = v;
        }
      }
    }
  }
}

__global__ __launch_bounds__(SK_WG, 2)
void sk_sym_query_kernel(const float* __restrict__ Q, long long m, int d,
                         const float* __restrict__ X, long long head_stride,
                         const SymQryTile* __restrict__ tiles, int ntiles, int nqt,
                         SymTables tb, long long PB, float* __restrict__ parts) {
  const long long lg = blockIdx.x;
  const int tile = (int)(lg % ntiles);
  const int qt = (int)((lg / ntiles) % nqt);
  const long long head = lg / ((long long)nqt * ntiles);
  const SymQryTile T = tiles[tile];
  switch (T.cb) {
    case 1: sk_sym_query_tile<1>(Q, m, d, X, head_stride, T, tb, qt, head, PB, parts); break;
    case 2: sk_sym_query_tile<2>(Q, m, d, X, head_stride, T, tb, qt, head, PB, parts); break;
    case 4: sk_sym_query_tile<4>(Q, m, d, X, head_stride, T, tb, qt, head, PB, parts); break;
    default: sk_sym_query_tile<8>(Q, m, d, X, head_stride, T, tb, qt, head, PB, parts); break;
  }
}

// Canonical view [h][D_sym][1 + dv]: column 0 = M^s, columns 1.. = N^s.
__global__ void sk_sym_export_kernel(const float* __restrict__ X, long long XS, SymTables tb,
                                     long long Dsym, long long Rlo, int d, int dv, float count,
                                     float* __restrict__ dst, long long total) {
  const int W = 1 + dv;
  const int Cl = d + dv;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const long long head = i / (Dsym * W);
    const long long rem = i - head * Dsym * W;
    const long long r = rem / W;
    const int c = (int)(rem - r * W);
    const float* Xh = X + head * XS;
    float v;
    if (c == 0) {
      const int pre = tb.prefix[r];
      v = (r == 0) ? count : Xh[(long long)(pre < 0 ? 0 : pre) * Cl + tb.last[r]];
    } else if (r < Rlo) {
      v = Xh[r * Cl + d + c - 1];
    } else {
      v = Xh[Rlo * Cl + (r - Rlo) * dv + c - 1];
    }
    dst[i] = v;
  }
}
