// Moment update for key widths d >= 16, organised around the Kronecker digits.
// Same contraction and state layout as sk_update.h (level j holds
// X_j[a][e] = sum_i k_i^(x)j[a] u_i[e], u = [k, v] below the top level and
// u = v at the top; Taylor moments of the polynomial method, "Rumo a Limites
// Estritos para Atenção em Streaming", "Metodologia", pillar "O Método
// Polinomial").
//
// Write the row index of level j >= 3 as a = (F, b2, b1, c): c the last digit,
// b1 the one before, b2 the one before that and F the leading j - 3 digits.  Then
//     X_j[(F, b2, b1, c)][e] = sum_i (k_i[c] k_i[b1]) * (u_i[e] k_i[b2] P_F(k_i)),
//     P_F(k) = prod of k[f] over the digits f of F,
// so a block over (b1, c) rows and (b2, e) columns is a v_mfma_f32_32x32x2_f32
// product over keys (two keys per instruction) whose operands are the raw key
// and value components, each scaled by one key component.  The 32 rows of a
// block are (x, c) for a pair b1 = b1p + x, x in {0, 1}, and 16 values of c; the
// 32 columns are, by the level's row width C:
//   C <= 16 ("pair"):   (y, e) for a pair b2 = b2p + y and the 16 values of e,
//   C > 16 ("single"):  32 values of e for one b2,
// and at level 2 (no b2 digit, "wide") 32 values of e.  A wave owns a unit: 4
// b1 pairs x 2 b2 pairs (or b2 values, or 32-column chunks), one 16-chunk of c
// and F, i.e. 8 blocks (128 accumulator registers).  Per two keys it loads the
// key and value components it needs (buffer loads, 64 contiguous bytes per
// 16-lane row) with the unit's b1 (b2) digits lined up in the row (at d = 16 by
// rotating the row of c components, ds_bpermute; at d >= 32 by loading them
// rotated), and forms each operand with one
// VALU multiply whose second factor is a DPP row broadcast (v_mul_f32_dpp
// row_newbcast): 6 such multiplies feed 8 matrix instructions, and no feature
// tile passes through LDS.  Levels 0 and 1 (no b1 digit) run a small 16x16x4
// path: level 1 is k[c] u[e], level 0 the sum of u[e] (A operand 1 in row 0).
//
// v_mfma_f32_32x32x2_f32: lane l supplies A[l % 32][l / 32] and
// B[l / 32][l % 32]; accumulator register r of lane l holds
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  Here l / 32 is the key of the
// step, and within a 16-lane DPP row (lanes 16 q .. 16 q + 15) the row parity
// q & 1 is x (A side) or y (B side, pair mode) and the lane's position m is c
// or e mod 16.
#pragma once

#include "sk_common.h"
#include "sk_reduce.h"

#include <type_traits>
#include <utility>

#define KR_WAVES 4          // independent waves per workgroup
#define KR_PF 3             // key steps fetched ahead
#define KR_SLOTS 4          // prefetch ring slots (one more than KR_PF: a step
                            // loads into the slot the previous step consumed)
#define KR_NA 4             // b1 pairs per unit
#define KR_NB 2             // b2 pairs (pair mode), b2 values (single) or 32-column chunks (wide)
#define KR_MAXF 4           // leading digits F per unit

// Unit modes
#define KR_SMALL 0          // levels 0 and 1
#define KR_PAIR 1           // levels >= 3, C <= 16
#define KR_SINGLE 2         // levels >= 3, C > 16
#define KR_WIDE 3           // level 2

// One unit of work.
struct KrUnit {
  long long xoff;   // float offset of level j inside one head's state
  int j;            // level
  int C;            // row width of the level (d + dv, or dv at the top)
  int top;          // 1 at the top level (u = v)
  int mode;         // KR_SMALL, KR_PAIR, KR_SINGLE or KR_WIDE
  int F;            // leading digits (KR_PAIR, KR_SINGLE) as a number in base d
  int b2;           // first b2 digit (KR_PAIR, KR_SINGLE)
  int b1;           // first b1 digit (not KR_SMALL)
  int rc;           // 16-chunk of the last digit c (not KR_SMALL)
  int ct;           // column chunk: 32 wide (KR_SINGLE), 64 wide (KR_WIDE), 16 wide (KR_SMALL)
  int pad_;
};

// Key splits of one launch.  The units form groups of consecutive units (heavy
// units first); group g cuts the keys into ns[g] splits of kps[g] keys, so that a
// unit doing less work per key takes longer key ranges and every wave of the
// launch has about the same work.  Split s of a unit writes partial buffer s;
// buffers ns[g] .. nsplit - 1 of a group with fewer splits get zeros in its rows
// (from the wave of split s' mod ns[g]), so the reduce adds nsplit buffers
// everywhere.
#define KR_MAXG 4
struct KrSplits {
  int ngroup;
  int nsplit;                    // partial buffers (the largest ns[g])
  int unit0[KR_MAXG + 1];        // first unit of each group; unit0[ngroup] = unit count
  int ns[KR_MAXG];               // splits of each group
  long long item0[KR_MAXG + 1];  // first item of each group within a head; item0[ngroup] = items
  long long kps[KR_MAXG];        // keys per split of each group
  int rev;                       // 1: a head's items taken lightest group first
};

// src[lane N of this lane's 16-lane row] * y: one v_mul_f32_dpp row_newbcast.
template <int N>
__device__ __forceinline__ float kr_bmul(float src, float y) {
  const float b = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, src), 0x150 + N, 0xf, 0xf,
                                         false));
  return b * y;
}

// u component e of one key: a key component below the top level for e < d,
// else a value component; zero past the row width or the value width.
__device__ __forceinline__ float kr_u(const float* __restrict__ krow, const float* __restrict__ vrow,
                                      int e, int d, int dv, int C, int top, bool ok) {
  if (!ok || e >= C) return 0.f;
  if (!top && e < d) return krow[e];
  const int c = top ? e : e - d;
  return c < dv ? vrow[c] : 0.f;
}

// Key and value components are read with raw buffer loads (sk_rsrc / sk_ld): a
// resource at the split's first row, the lane's byte offset in a vector register
// and the step's row offset in a scalar one, so a load costs no per-lane address
// arithmetic.  Offsets stay below 2^31 (the host cuts longer key ranges into
// several launches).

// One unit at levels >= 2 (see the layout above), specialised by mode, number
// of blocks per b1 pair (NBE), number of leading digits (NF) and whether u is
// the value row alone (TOP; the pair mode always is), so that a key step is
// straight-line code: loads for a later step, the centring, two row rotations,
// 4 + NBE fused broadcast multiplies and 4 NBE matrix instructions.  Columns
// past the row width hold whatever their (in-bounds) loads give and are never
// stored: a column of the product depends on its own B column only.  Steps past
// the last full pair of keys (the ring runs in groups of four, the last group
// separately) re-read that pair's rows with zero A operands, so they add nothing.
template <int RT, bool CENTER, int MODE, int NBE, int NF, bool TOP>
__device__ __forceinline__
void kr_body(const KrUnit& U, const float* __restrict__ Kh, const float* __restrict__ Vh, int dv,
             long long k_begin, long long k_end, const float* __restrict__ cen,
             float* __restrict__ o, int accumulate, int nzero, long long zstride) {
  constexpr int d = 16 * RT;
  constexpr int LOGD = RT == 1 ? 4 : RT == 2 ? 5 : RT == 4 ? 6 : 7;
  constexpr int NBU = MODE == KR_WIDE ? NBE : 1;     // distinct u operands
  const int lane = threadIdx.x & 63;
  const int m = lane & 15;
  const int khalf = lane >> 5;                        // key of the step
  const int l32 = lane & 31;
  const int par = (lane >> 4) & 1;                    // x (A rows) or y (B columns, pair mode)
  const int rowbase = lane & 48;
  // Steps of two keys.  The npair full steps read their rows at a row base that
  // is the same for the whole wave (keys k_begin + 2 st and k_begin + 2 st + 1,
  // the step clamped to the last full one), so a load is a scalar base plus a
  // fixed lane offset; a lone last key (odd count) gets a step of its own.
  const long long nk = k_end - k_begin;
  const int npair = (int)(nk >> 1);
  const float* Kb = Kh + k_begin * d;
  const float* Vb = Vh + k_begin * dv;
  // u columns: byte offsets into the key row (lk) and the value row (lv) and
  // which of the two the lane takes (column 0 for columns past the row width)
  unsigned lk[NBU], lv[NBU];
  bool usel[NBU];
#pragma unroll
  for (int y = 0; y < NBU; ++y) {
    const int e = MODE == KR_PAIR ? m : MODE == KR_SINGLE ? 32 * U.ct + l32 : 64 * U.ct + 32 * y + l32;
    const bool fromk = !TOP && e < d;
    const int col = fromk ? e : (TOP ? e : e - d);
    const bool valid = e < U.C && (fromk || col < dv);
    lk[y] = 4u * (unsigned)(khalf * d + (fromk && valid ? col : 0));
    lv[y] = 4u * (unsigned)(khalf * dv + (!fromk && valid ? col : 0));
    usel[y] = fromk;
  }
  float cu[NBU];
#pragma unroll
  for (int y = 0; y < NBU; ++y) {
    const int e = MODE == KR_PAIR ? m : MODE == KR_SINGLE ? 32 * U.ct + l32 : 64 * U.ct + 32 * y + l32;
    cu[y] = (CENTER && !TOP && e < d) ? cen[e] : 0.f;
  }
  const int q1 = U.b1 >> 4, q2 = U.b2 >> 4;
  // byte offsets of the key components
  const unsigned la = 4u * (unsigned)(khalf * d + 16 * U.rc + m);
  const int src1 = (rowbase + ((m + (U.b1 & 15) + par) & 15)) * 4;
  const int src2 = (rowbase + ((m + (U.b2 & 15) + (MODE == KR_PAIR ? par : 0)) & 15)) * 4;
  // d >= 32: the b1 and b2 components are loaded already rotated (lane m of the
  // row gets the component the rotation would bring it; measured faster there),
  // at d = 16 they come from the c components by a row rotation
  constexpr bool ROTL = RT > 1;
  const int rot1 = 16 * q1 + ((m + (U.b1 & 15) + par) & 15);
  const int rot2 = 16 * q2 + ((m + (U.b2 & 15) + (MODE == KR_PAIR ? par : 0)) & 15);
  const unsigned lx1 = 4u * (unsigned)(khalf * d + rot1);
  const unsigned lx2 = 4u * (unsigned)(khalf * d + rot2);
  const float cx1 = CENTER ? cen[rot1] : 0.f;
  const float cx2 = CENTER ? cen[rot2] : 0.f;
  int fdig[NF > 0 ? NF : 1];
  unsigned lf[NF > 0 ? NF : 1];
  float cf[NF > 0 ? NF : 1];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    fdig[f] = (U.F >> (LOGD * (NF - 1 - f))) & (d - 1);
    lf[f] = 4u * (unsigned)(khalf * d + fdig[f]);
    cf[f] = CENTER ? cen[fdig[f]] : 0.f;
  }
  const float ca = CENTER ? cen[16 * U.rc + m] : 0.f;

  // prefetch ring (static slots)
  // (below the top level a u column comes from the key or the value row: both are
  // loaded into the ring and the lane's choice is made when the step uses them,
  // so that no select waits on a load just issued)
  constexpr int NUK = TOP ? 1 : NBU;
  float ra[KR_SLOTS], r1[KR_SLOTS], r2[KR_SLOTS], ru[KR_SLOTS][NBU], rk2[KR_SLOTS][NUK],
      rf[KR_SLOTS][NF > 0 ? NF : 1];
  // one step's components from the key row at byte offset sk and the value row
  // at sv (both relative to the split's first rows), lane offsets less adjk/adjv
  const __amdgpu_buffer_rsrc_t rk = sk_rsrc(Kb), rv = sk_rsrc(Vb);
  auto load = [&](unsigned sk, unsigned sv, unsigned adjk, unsigned adjv, float& va, float& v1,
                  float& v2, float (&vu)[NBU], float (&vk)[NUK], float (&vf)[NF > 0 ? NF : 1]) {
    va = sk_ld(rk, la - adjk, sk);
    if constexpr (ROTL) {
      v1 = sk_ld(rk, lx1 - adjk, sk);
      if (MODE != KR_WIDE) v2 = sk_ld(rk, lx2 - adjk, sk);
    }
#pragma unroll
    for (int y = 0; y < NBU; ++y) {
      vu[y] = sk_ld(rv, lv[y] - adjv, sv);        // the top level: u = v
      if constexpr (!TOP) vk[y] = sk_ld(rk, lk[y] - adjk, sk);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) vf[f] = sk_ld(rk, lf[f] - adjk, sk);
  };
  // unconditional (no merge of old and new slots); CLAMP re-reads the last full
  // pair for steps past it, else the step must lie before it
  const int lastp = npair > 0 ? 2 * (npair - 1) : 0;
  auto fetch = [&](int st, int sl, auto clamp_c) {
    const int off = !decltype(clamp_c)::value || 2 * st < lastp ? 2 * st : lastp;   // uniform
    load((unsigned)off * (4u * d), (unsigned)off * (4u * dv), 0u, 0u, ra[sl], r1[sl], r2[sl],
         ru[sl], rk2[sl], rf[sl]);
  };
  if (npair > 0) {
#pragma unroll
    for (int s = 0; s < KR_PF; ++s) fetch(s, s, std::true_type{});
  }

  floatx16 acc[KR_NA][NBE];
#pragma unroll
  for (int x = 0; x < KR_NA; ++x)
#pragma unroll
    for (int y = 0; y < NBE; ++y) acc[x][y] = floatx16{0};

  // the row rotations of the key components holding b1 and b2 for a step:
  // lane 2 x of row parity x' gets k[b1 + 2 x + x'], and lane 2 y of parity y'
  // k[b2 + 2 y + y'] (pair) or lane y k[b2 + y] (single)
  auto rotate = [&](float va, float v1, float v2, float& x1, float& x2) {
    if constexpr (ROTL) {
      x1 = CENTER ? v1 - cx1 : v1;
      x2 = MODE == KR_WIDE ? 0.f : (CENTER ? v2 - cx2 : v2);
      return;
    }
    const float k = CENTER ? va - ca : va;         // d = 16: b1, b2 and c share a row
    const float k1 = k, k2 = k;
    x1 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src1, __builtin_bit_cast(int, k1)));
    x2 = MODE == KR_WIDE ? 0.f
         : __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src2, __builtin_bit_cast(int, k2)));
  };
  // operands and matrix instructions of one step from its components (a = 0 for
  // a key that adds nothing)
  auto compute = [&](float a, float (&u)[NBU], float (&fv)[NF > 0 ? NF : 1], float x1, float x2) {
    float p = 1.f;
    if (CENTER) {
      a -= ca;
#pragma unroll
      for (int y = 0; y < NBU; ++y) u[y] -= cu[y];
#pragma unroll
      for (int f = 0; f < NF; ++f) fv[f] -= cf[f];
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) p *= fv[f];
    return std::make_pair(a, p);
  };
  auto mma = [&](float a, float p, const float (&u)[NBU], float x1, float x2) {
    float A[KR_NA];
    A[0] = kr_bmul<0>(x1, a);
    A[1] = kr_bmul<2>(x1, a);
    A[2] = kr_bmul<4>(x1, a);
    A[3] = kr_bmul<6>(x1, a);
    float B[NBE];
    if constexpr (MODE == KR_WIDE) {
#pragma unroll
      for (int y = 0; y < NBE; ++y) B[y] = u[y];
    } else {
      const float pu = NF > 0 ? u[0] * p : u[0];
      if constexpr (MODE == KR_PAIR) {
        B[0] = kr_bmul<0>(x2, pu);
        B[1] = kr_bmul<2>(x2, pu);
      } else {
        B[0] = kr_bmul<0>(x2, pu);
        B[1] = kr_bmul<1>(x2, pu);
      }
    }
#pragma unroll
    for (int x = 0; x < KR_NA; ++x)
#pragma unroll
      for (int y = 0; y < NBE; ++y) acc[x][y] = mfma32x32x2(A[x], B[y], acc[x][y]);
  };

  // rotations of the current step, issued one step ahead
  float xr1 = 0.f, xr2 = 0.f;
  if (npair > 0) rotate(ra[0], r1[0], r2[0], xr1, xr2);

  auto step = [&](int st, auto slot_c, auto tail_c) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr bool TAIL = decltype(tail_c)::value;     // a step of the last groups
    float u[NBU], fv[NF > 0 ? NF : 1];
    const float a0v = ra[SL];
#pragma unroll
    for (int y = 0; y < NBU; ++y) u[y] = TOP || !usel[y] ? ru[SL][y] : rk2[SL][TOP ? 0 : y];
#pragma unroll
    for (int f = 0; f < NF; ++f) fv[f] = rf[SL][f];
    const float x1 = xr1, x2 = xr2;
    // the loads for step st + KR_PF and the rotations for step st + 1 go out
    // here, ahead of this step's work (the scheduler would otherwise sink them
    // next to their use)
    __builtin_amdgcn_sched_barrier(0);
    fetch(st + KR_PF, (SL + KR_PF) % KR_SLOTS, tail_c);
    constexpr int SN = (SL + 1) % KR_SLOTS;
    rotate(ra[SN], r1[SN], r2[SN], xr1, xr2);
    __builtin_amdgcn_sched_barrier(0);
    auto ap = compute(a0v, u, fv, x1, x2);
    // uniform: steps past the pairs (last groups only) add nothing
    const float a = !TAIL || st < npair ? ap.first : 0.f;
    mma(a, ap.second, u, x1, x2);
  };
  static_assert(KR_PF == 3 && KR_SLOTS == 4 && KR_NA == 4, "the step is written for these sizes");
  // whole groups of KR_SLOTS steps with no branches inside (a merge of ring slots
  // would make the compiler wait for loads just issued): first the groups whose
  // steps and fetches all lie before the last pair, then (at most two) groups that
  // clamp their fetches and zero the A operands of steps past the pairs
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  int st0 = 0;
  for (; st0 + KR_SLOTS + KR_PF <= npair; st0 += KR_SLOTS) {
    step(st0, S0{}, std::false_type{});
    step(st0 + 1, S1{}, std::false_type{});
    step(st0 + 2, S2{}, std::false_type{});
    step(st0 + 3, S3{}, std::false_type{});
  }
  for (; st0 < npair; st0 += KR_SLOTS) {
    step(st0, S0{}, std::true_type{});
    step(st0 + 1, S1{}, std::true_type{});
    step(st0 + 2, S2{}, std::true_type{});
    step(st0 + 3, S3{}, std::true_type{});
  }
  if (nk & 1) {
    // the lone last key: both lane halves read its row, the second half adds nothing
    const long long lastk = nk - 1;
    float va = 0.f, v1 = 0.f, v2 = 0.f, u[NBU], uk[NUK], fv[NF > 0 ? NF : 1];
    load((unsigned)lastk * (4u * d), (unsigned)lastk * (4u * dv), (unsigned)khalf * (4u * d),
         (unsigned)khalf * (4u * dv), va, v1, v2, u, uk, fv);
#pragma unroll
    for (int y = 0; y < NBU; ++y)
      if (!TOP && usel[y]) u[y] = uk[TOP ? 0 : y];
    float x1, x2;
    rotate(va, v1, v2, x1, x2);
    auto ap = compute(va, u, fv, x1, x2);
    mma(khalf == 0 ? ap.first : 0.f, ap.second, u, x1, x2);
  }

  // Epilogue.  Block (x, y), register r: row 8 (r / 4) + 4 khalf + r % 4 =
  // (x' = row / 16, c = 16 rc + row % 16) with b1 = b1 + 2 x + x'; column l32 =
  // (y' = l32 / 16, e = l32 % 16) with b2 = b2 + 2 y + y' (pair), or e in the
  // unit's 32-column chunk with b2 = b2 + y (single), or e in 32-column chunk y
  // of the unit's 64 (wide).
#pragma unroll
  for (int y = 0; y < NBE; ++y) {
    int e, b2;
    if (MODE == KR_PAIR) { e = m; b2 = U.b2 + 2 * y + par; }
    else if (MODE == KR_SINGLE) { e = 32 * U.ct + l32; b2 = U.b2 + y; }
    else { e = 64 * U.ct + 32 * y + l32; b2 = 0; }
    if (e >= U.C) continue;
    // rows above b1: F and b2 for levels >= 3, nothing at level 2
    const long long hi = MODE == KR_WIDE ? 0 : (long long)U.F * d + b2;
#pragma unroll
    for (int x = 0; x < KR_NA; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * khalf + (r & 3);
        const int b1 = U.b1 + 2 * x + (row >> 4);
        const int c = 16 * U.rc + (row & 15);
        const long long a = (hi * d + b1) * d + c;
        float* dst = o + a * U.C + e;
        *dst = accumulate ? *dst + acc[x][y][r] : acc[x][y][r];
      }
  }
  // zeros into the unit's rows of the partial buffers its group does not reach
  // (a plain loop over the same positions: only the lighter groups have any)
#pragma unroll 1
  for (int i = 0; i < nzero * NBE * KR_NA * 16; ++i) {
    const int r = i & 15, x = (i >> 4) % KR_NA, y = (i >> 4) / KR_NA % NBE;
    const int z = 1 + (i >> 4) / (KR_NA * NBE);
    int e, b2;
    if (MODE == KR_PAIR) { e = m; b2 = U.b2 + 2 * y + par; }
    else if (MODE == KR_SINGLE) { e = 32 * U.ct + l32; b2 = U.b2 + y; }
    else { e = 64 * U.ct + 32 * y + l32; b2 = 0; }
    const long long hi = MODE == KR_WIDE ? 0 : (long long)U.F * d + b2;
    const int row = 8 * (r >> 2) + 4 * khalf + (r & 3);
    const long long a = (hi * d + U.b1 + 2 * x + (row >> 4)) * d + 16 * U.rc + (row & 15);
    if (e < U.C) o[z * zstride + a * U.C + e] = 0.f;
  }
}

// Three waves per SIMD (168 registers; measured faster than two with more
// registers).  At d = 32 the loops of units with two or more leading digits
// (levels >= 5) spill a few registers; the others do not.
template <int RT, bool CENTER>
__global__ __launch_bounds__(64 * KR_WAVES, 3)
void sk_update_kr_kernel(const float* __restrict__ K, const float* __restrict__ V,
                         long long n, long long hkeys, int dv,
                         const KrUnit* __restrict__ units, KrSplits P, int nhead,
                         float* __restrict__ out, long long head_stride,
                         long long split_stride, int accumulate,
                         const float* __restrict__ center, PendingReduce red) {
  constexpr int d = 16 * RT;
  const long long per_head = P.item0[P.ngroup];
  const long long nitems = per_head * nhead;
  const long long nwg = (nitems + KR_WAVES - 1) / KR_WAVES;
  if ((long long)blockIdx.x >= nwg) {
    pending_reduce_wg(red, (long long)blockIdx.x - nwg);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // workgroups of one XCD take a contiguous range of items: the items of one key
  // split (all units of a group) read the same key rows from that XCD's L2; with
  // P.rev a head's items run from its last (lightest group, longest waves) down
  const long long item = xcd_remap(blockIdx.x, nwg) * KR_WAVES + wave;
  if (item >= nitems) return;
  const long long head = item / per_head;
  const long long li = P.rev ? per_head - 1 - (item - head * per_head) : item - head * per_head;
  // the item's group (scalar selects: no dynamic index into the argument block)
  long long gbase = P.item0[0], kps = P.kps[0];
  int u0 = P.unit0[0], gn = P.unit0[1] - P.unit0[0], gns = P.ns[0];
#pragma unroll
  for (int g = 1; g < KR_MAXG; ++g)
    if (g < P.ngroup && li >= P.item0[g]) {
      gbase = P.item0[g];
      kps = P.kps[g];
      u0 = P.unit0[g];
      gn = P.unit0[g + 1] - P.unit0[g];
      gns = P.ns[g];
    }
  const long long gi = li - gbase;
  const int unit_id = u0 + (int)(gi % gn);
  const long long split = gi / gn;
  const KrUnit U = units[unit_id];
  // partial buffers split + gns, split + 2 gns, ... below nsplit get zeros here
  const int nzero = accumulate ? 0 : (int)((P.nsplit - 1 - split) / gns);
  const long long zstride = (long long)gns * split_stride;

  const long long k_begin = split * kps;
  long long k_end = k_begin + kps;
  if (k_end > n) k_end = n;
  if (k_end < k_begin) k_end = k_begin;
  const float* Kh = K + head * hkeys * d;
  const float* Vh = V + head * hkeys * dv;
  const float* cen = CENTER ? center + head * d : nullptr;
  float* o = out + split * split_stride + head * head_stride + U.xoff;
  const int m = lane & 15;

  if (U.mode == KR_SMALL) {
    // ---- levels 0 and 1 with v_mfma_f32_16x16x4_f32: lane 16 kk + i supplies
    // A[i][kk] = k[16 r + i] (level 1) or [i == 0] (level 0) and B[kk][i] = u[e]
    const int kk = lane >> 4;
    const int nstep = k_end > k_begin ? (int)((k_end - k_begin + 3) / 4) : 0;
    const int e = 16 * U.ct + m;
    floatx4v acc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r] = floatx4v{0.f, 0.f, 0.f, 0.f};
    // prefetch ring (static slots): key components 16 r + m and the u component
    float sa[KR_PF][RT], su[KR_PF];
    auto sfetch = [&](int st, int sl) {
      const long long key = k_begin + 4LL * st + kk;
      const bool ok = key < k_end;
      const float* krow = Kh + key * d;
#pragma unroll
      for (int r = 0; r < RT; ++r) sa[sl][r] = (ok && U.j == 1) ? krow[16 * r + m] : 0.f;
      su[sl] = kr_u(krow, Vh + key * dv, e, d, dv, U.C, U.top, ok);
    };
#pragma unroll
    for (int s2 = 0; s2 < KR_PF; ++s2)
      if (s2 < nstep) sfetch(s2, s2);
    auto sstep = [&](int st, auto slot_c) {
      constexpr int SL = decltype(slot_c)::value;
      const bool ok = k_begin + 4LL * st + kk < k_end;
      float u = su[SL], a[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) a[r] = sa[SL][r];
      if (st + KR_PF < nstep) sfetch(st + KR_PF, SL);
      if (CENTER && ok && !U.top && e < d) u -= cen[e];
      if (U.j == 1) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          if (CENTER && ok) a[r] -= cen[16 * r + m];
          acc[r] = mfma16x16x4(a[r], u, acc[r]);
        }
      } else {
        acc[0] = mfma16x16x4(m == 0 ? 1.f : 0.f, u, acc[0]);
      }
    };
    for (int st0 = 0; st0 < nstep; st0 += KR_PF) {
      sstep(st0, std::integral_constant<int, 0>{});
      if (st0 + 1 < nstep) sstep(st0 + 1, std::integral_constant<int, 1>{});
      if (st0 + 2 < nstep) sstep(st0 + 2, std::integral_constant<int, 2>{});
    }
    if (e >= U.C) return;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 16 * r + 4 * kk + q;       // row of level 1, or 0 at level 0
        const bool keep = U.j == 1 ? true : (r == 0 && c == 0);
        if (keep) {
          float* dst = o + (long long)c * U.C + e;
          *dst = accumulate ? *dst + acc[r][q] : acc[r][q];
          for (int z = 1; z <= nzero; ++z) dst[z * zstride] = 0.f;
        }
      }
    return;
  }

  // ---- levels >= 2 with v_mfma_f32_32x32x2_f32: a loop specialised per mode,
  // number of blocks and number of leading digits
  const int nbe = U.mode == KR_WIDE ? (U.C - 64 * U.ct > 32 ? 2 : 1) : KR_NB;
  const int nf = U.mode == KR_WIDE ? 0 : U.j - 3;
#define KR_CALL(MODE, NBE, NF, TOP)                                                         \
  kr_body<RT, CENTER, MODE, NBE, NF, TOP>(U, Kh, Vh, dv, k_begin, k_end, cen, o, accumulate, \
                                          nzero, zstride)
#define KR_NF(MODE, TOP)                          \
  switch (nf) {                                   \
    case 0: KR_CALL(MODE, 2, 0, TOP); break;      \
    case 1: KR_CALL(MODE, 2, 1, TOP); break;      \
    case 2: KR_CALL(MODE, 2, 2, TOP); break;      \
    case 3: KR_CALL(MODE, 2, 3, TOP); break;      \
    default: KR_CALL(MODE, 2, 4, TOP); break;     \
  }
  if (U.mode == KR_WIDE) {
    if (U.top) {
      if (nbe == 2) KR_CALL(KR_WIDE, 2, 0, true); else KR_CALL(KR_WIDE, 1, 0, true);
    } else {
      if (nbe == 2) KR_CALL(KR_WIDE, 2, 0, false); else KR_CALL(KR_WIDE, 1, 0, false);
    }
  } else if (U.mode == KR_PAIR) {
    KR_NF(KR_PAIR, true)                  // C <= 16 < d + dv: only the top level
  } else if (U.top) {
    KR_NF(KR_SINGLE, true)
  } else {
    KR_NF(KR_SINGLE, false)
  }
#undef KR_NF
#undef KR_CALL
}
