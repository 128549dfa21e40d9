// Exact streaming path: Z(q) = sum_i exp(<q, k_i>), o(q) = sum_i exp(<q,k_i>) v_i / Z.
// Source: "Rumo a Limites Estritos para Atenção em Streaming", "Definição do
// Problema" (the naive answer that keeps every key/value pair).
//
// Keys are split into slices; each slice keeps a running maximum mu, the sum
// l = sum e^(s - mu) and acc = sum e^(s - mu) v (online softmax).  Two slices
// (mu, l, acc) and (mu', l', acc') combine as mu* = max(mu, mu'),
// l* = l e^(mu - mu*) + l' e^(mu' - mu*), acc* likewise; at the end
// Z = e^mu l and o = acc / l.  Every combine runs in a fixed order.
//
// sk_exact_decode  (few queries per head): HBM-streaming.  G = B/4 lanes share a
//   key row, each loading one float4 of K and one of V; the dot product is
//   reduced across the G lanes with xor shuffles.  Each group walks U keys per
//   step so that many 128-bit loads are in flight.
// sk_exact_mfma    (many queries per head, d or dv >= 16): fp32 MFMA for both
//   products (queries x keys, then values x keys), online softmax in between.
// sk_exact_tiled   (many queries per head, d, dv <= 8): one thread per query, key
//   and value rows staged through LDS and read as broadcasts; per stage of 32
//   keys one rescale.
// sk_exact_combine: folds the slice partials of each (head, query).
#pragma once

#include "sk_common.h"

#include <type_traits>

#ifndef SK_EX_U
#define SK_EX_U 8          // keys per group in flight per step (decode)
#endif

__device__ __forceinline__ float4 ld_stream(const float* p) {
  const floatx4v v = __builtin_nontemporal_load(reinterpret_cast<const floatx4v*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// The fold of one (head, query)'s slice records P[nsplit][2 + dv] by one
// workgroup of NT threads, in one pass over the records: thread (g, slot) walks
// slices g, g + G, g + 2G, ... (G = NT / (1 + dv) groups) keeping its own
// running maximum m and the sum of slot 0 (l) or slot 1 + c (acc[c]) rescaled to
// it; the records come in blocks of sixteen (each block's terms rescaled to the
// block's new maximum at once), the next block's loads issued before the current
// block is added (the records were written on other XCDs, so each load is a
// long round trip).
// Then the largest m of the workgroup is found, every thread's sum is rescaled
// to it, and the G group sums are added in group order.  Fixed order
// throughout, so the result does not depend on timing.  red: NT floats of LDS,
// lsum: one.
template <int NT>
__device__ __forceinline__ void exact_fold(const float* __restrict__ P, int nsplit, int dv,
                                           float* __restrict__ o, float* __restrict__ z,
                                           float* red, float* lsum) {
  constexpr int FB = 16;                       // records per block
  const int tid = threadIdx.x;
  const int rec = 2 + dv;
  const int slots = 1 + dv;
  const int groups = NT / slots > 0 ? NT / slots : 1;
  const int g = tid / slots, slot = tid - g * slots;
  float m = -INFINITY, acc = 0.f;
  // slices of this thread: g + G t for t < nt
  const int nt = g < groups && g < nsplit ? (nsplit - g + groups - 1) / groups : 0;
  auto load = [&](int t0, float (&mu)[FB], float (&x)[FB]) {
#pragma unroll
    for (int u = 0; u < FB; ++u) {
      // past the last slice: re-read this thread's first one, ignored when added
      const int t = t0 + u < nt ? t0 + u : 0;
      const float* r = P + (long long)(g + t * groups) * rec;
      mu[u] = r[0];
      x[u] = r[1 + slot];
    }
  };
  // a block: its largest maximum first, then its terms rescaled to the new
  // running maximum (independent exponentials) and the running sum once
  auto add = [&](int t0, const float (&mu)[FB], const float (&x)[FB]) {
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < FB; ++u)
      if (t0 + u < nt) bm = fmaxf(bm, mu[u]);
    if (bm == -INFINITY) return;
    const float nm = fmaxf(m, bm);
    float sb = 0.f;
#pragma unroll
    for (int u = 0; u < FB; ++u)
      if (t0 + u < nt) sb += x[u] * expf(mu[u] - nm);
    acc = acc * expf(m - nm) + sb;
    m = nm;
  };
  if (nt > 0) {
    float mu0[FB], x0[FB], mu1[FB], x1[FB];
    load(0, mu0, x0);
    for (int t0 = 0; t0 < nt; t0 += 2 * FB) {
      if (t0 + FB < nt) load(t0 + FB, mu1, x1);
      add(t0, mu0, x0);
      if (t0 + FB < nt) {
        if (t0 + 2 * FB < nt) load(t0 + 2 * FB, mu0, x0);
        add(t0 + FB, mu1, x1);
      }
    }
  }
  red[tid] = m;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float ms = red[0];
  __syncthreads();
  red[tid] = (m == -INFINITY) ? 0.f : acc * expf(m - ms);
  __syncthreads();
  float sum = 0.f;
  if (tid < slots) {
    for (int gg = 0; gg < groups; ++gg) sum += red[gg * slots + tid];
    if (tid == 0) *lsum = sum;
  }
  __syncthreads();
  if (tid == 0) *z = (ms == -INFINITY) ? 0.f : expf(ms) * *lsum;
  else if (tid < slots) o[tid - 1] = sum / *lsum;
  __syncthreads();
}

// sk_exact_mfma (many queries per head): one workgroup = 4 waves x 32 queries,
// one key slice; per stage of 32 keys (K and V rows staged in LDS):
//   S^T = K Q^T         v_mfma_f32_32x32x2_f32, rows = keys, columns = queries;
//                       the lane's query components stay in registers
//   online softmax      in base 2 (queries prescaled by log2 e, p = 2^{s - ref});
//                       the stage's row maximum of a query is the larger of its
//                       two lanes' 16 entries (one cross-lane exchange); the
//                       reference ref is raised, and the sums rescaled by
//                       2^{ref_old - ref}, only when a stage maximum exceeds it by
//                       more than SK_XTAU (p <= 2^SK_XTAU otherwise), a branch
//                       the whole wave takes or skips
//   O^T += V^T P^T      the same MFMA with P taken straight from the first
//                       product's accumulator registers: an MFMA sums over its K
//                       index in any order, so at k-step t each lane half uses
//                       the key its register t holds, and reads that key's value
//                       row from LDS as the other operand.
// K rows sit in LDS with a stride of D + 2 floats: the two lane halves of a
// k-step read neighbouring features of 32 rows, which then fall in distinct
// banks for every D (D + 1 made the halves collide at D >= 64).
// The partial record per (head, query, slice) is the one of sk_exact_decode
// (mu = ref in natural-log units).
#define SK_XQ 128          // queries per workgroup (4 waves x 32)
#define SK_XTAU 8.f        // reference slack of the base-2 online softmax
#define SK_XK 32           // keys per stage
// Waves per SIMD the register allocation of sk_exact_mfma<D, NCB> keeps room for:
// three where the accumulators and the query leave space for the next stage's
// rows (measured with those rows in flight: 0.59 -> 0.64 of the fp32 peak at
// d = dv = 64, 0.58 -> 0.59 at d = dv = 32), the compiler's choice otherwise.
template <int D, int NCB>
struct XmWaves {
  static constexpr int v = (D / 2 + 16 * NCB <= 64) ? 3 : 1;
};
template <int D, int NCB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(XmWaves<D, NCB>::v)))
void sk_exact_mfma(const float* __restrict__ K, const float* __restrict__ V,
                   long long n, int dv, const float* __restrict__ Q, long long m,
                   long long keys_per_split, int nsplit, float* __restrict__ parts) {
  constexpr int LDKE = D + 2;               // K stage row stride (keys x D)
  constexpr float LOG2E = 1.4426950408889634f;
  constexpr float LN2 = 0.6931471805599453f;
  constexpr int DVP = 32 * NCB;             // value columns, padded to 32
  constexpr int LDV = DVP + 8;              // the two lane halves' rows 32 banks apart
  __shared__ float Ks[SK_XK * LDKE];
  __shared__ float Vs[SK_XK * LDV];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const long long split = blockIdx.x % nsplit;
  const long long qt = blockIdx.x / nsplit;
  const long long head = blockIdx.y;
  const long long q = qt * SK_XQ + wave * 32 + l32;
  const bool qok = q < m;
  const long long k_begin = split * keys_per_split;
  long long k_end = k_begin + keys_per_split;
  if (k_end > n) k_end = n;
  const float* Kh = K + head * n * D;
  const float* Vh = V + head * n * dv;

  float qreg[D / 2];                        // Q[q][2 st + g] * log2 e
#pragma unroll
  for (int st = 0; st < D / 2; ++st)
    qreg[st] = qok ? Q[(head * m + q) * D + 2 * st + g] * LOG2E : 0.f;

  float mu = -INFINITY, l = 0.f;
  floatx16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = floatx16{0.f};

  // a stage's K and V rows: KT and VT float4 per thread, fetched into registers
  // one stage ahead (their loads run under the current stage's MFMAs), zeros
  // past the slice's last key and past dv
  constexpr int KT = (SK_XK * D / 4 + 255) / 256;
  constexpr int VT = (SK_XK * DVP / 4 + 255) / 256;
  float4 kx[KT], vx[VT];
  auto fetch = [&](long long k0) {
    const long long left = k_end - k0;
    const int nk = left < SK_XK ? (int)left : SK_XK;
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      const int i = tid + 256 * u;
      const int key = i / (D / 4), e = 4 * (i - key * (D / 4));
      kx[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < SK_XK * D / 4 && key < nk)
        kx[u] = *reinterpret_cast<const float4*>(Kh + (k0 + key) * D + e);
    }
#pragma unroll
    for (int u = 0; u < VT; ++u) {
      const int i = tid + 256 * u;
      const int key = i / (DVP / 4), c = 4 * (i - key * (DVP / 4));
      vx[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < SK_XK * DVP / 4 && key < nk && c < dv)
        vx[u] = *reinterpret_cast<const float4*>(Vh + (k0 + key) * dv + c);
    }
  };
  if (k_begin < k_end) fetch(k_begin);

  for (long long kb = k_begin; kb < k_end; kb += SK_XK) {
    const long long left = k_end - kb;
    const int nk = left < SK_XK ? (int)left : SK_XK;
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      const int i = tid + 256 * u;
      const int key = i / (D / 4), e = 4 * (i - key * (D / 4));
      if (i < SK_XK * D / 4) {
        float2* dst = reinterpret_cast<float2*>(Ks + key * LDKE + e);
        dst[0] = make_float2(kx[u].x, kx[u].y);
        dst[1] = make_float2(kx[u].z, kx[u].w);
      }
    }
#pragma unroll
    for (int u = 0; u < VT; ++u) {
      const int i = tid + 256 * u;
      const int key = i / (DVP / 4), c = 4 * (i - key * (DVP / 4));
      if (i < SK_XK * DVP / 4) *reinterpret_cast<float4*>(Vs + key * LDV + c) = vx[u];
    }
    __syncthreads();
    if (kb + SK_XK < k_end) fetch(kb + SK_XK);
    floatx16 s = {0.f};
#pragma unroll
    for (int st = 0; st < D / 2; ++st)
      s = mfma32x32x2(Ks[l32 * LDKE + 2 * st + g], qreg[st], s);
    // s[r] = <q, k_key>, key = acc_row(r, lane) of the stage
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (acc_row(r, lane) >= nk) s[r] = -INFINITY;
      mloc = fmaxf(mloc, s[r]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    if (__any(mloc > mu + SK_XTAU)) {       // also the first stage (mu = -inf)
      const float mnew = fmaxf(mu, mloc);   // finite: every stage has a key
      const float alpha = __builtin_amdgcn_exp2f(mu - mnew);   // 0 the first time
      l *= alpha;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
      mu = mnew;
    }
    float p[16];
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(s[r] - mu);   // 0 for keys past the slice
      lsum += p[r];
    }
    l += lsum;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int t = 0; t < 16; ++t)
        acc[cb] = mfma32x32x2(Vs[acc_row(t, lane) * LDV + 32 * cb + l32], p[t], acc[cb]);
    }
    __syncthreads();
  }
  l += __shfl_xor(l, 32, 64);               // the query's two lane halves
  if (qok) {
    float* P = parts + ((head * m + q) * nsplit + split) * (2 + dv);
    if (g == 0) {
      P[0] = mu * LN2;
      P[1] = l;
    }
    // acc[cb][r] = sum_i p_i v_i[c], c = 32 cb + acc_row(r, lane)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * cb + acc_row(r, lane);
        if (c < dv) P[2 + c] = acc[cb][r];
      }
  }
}

// sk_exact_mfma16 (many queries per head, value width a multiple of 16 that is
// not one of 32): the same online softmax with v_mfma_f32_16x16x4_f32 for both
// products, so 16 value columns fill the instruction (the 32x32 form pads them
// to 32).  One workgroup = 4 waves x 16 QB queries (QB 16-query blocks per wave:
// 4 up to d = 32, 2 at d = 64 for registers), one key slice; per stage of 32 keys (two 16-key blocks) each wave loads its
// operands straight from memory into registers, one stage ahead (buffer loads:
// fixed lane offsets, the stage's offset in a scalar register; the rows of a
// stage are shared by the workgroup's waves through L1/L2): no LDS, no barrier.
//   S^T block (16 keys x 16 queries): D/4 instructions, A = key rows, B = the
//       query components (registers); lane l, register r holds S[key 4 (l/16) +
//       r][query l % 16]
//   softmax in base 2 (queries prescaled by log2 e, p = 2^{s - ref}) against a
//       reference ref per query that is raised, and the sums rescaled by
//       2^{ref_old - ref}, only when a stage maximum exceeds it by more than
//       SK_XTAU (p <= 2^SK_XTAU otherwise); the decision is per wave, so the
//       rescale is a branch the whole wave takes or skips.  A stage maximum is
//       the largest of the lane's 8 entries and of its 4 lane groups.
//   O^T block (16 value columns x 16 queries): per key block 4 instructions,
//       instruction r taking keys 4 k + r (k = lane / 16) with B = P straight
//       from S's register r and A = those keys' value rows.
// The partial record is the one of sk_exact_decode (mu = ref in natural-log units).
template <int D, int DV, int QB>
__global__ __launch_bounds__(256)
void sk_exact_mfma16(const float* __restrict__ K, const float* __restrict__ V,
                     long long n, const float* __restrict__ Q, long long m,
                     long long keys_per_split, int nsplit, float* __restrict__ parts) {
  static_assert(D % 16 == 0 && DV % 16 == 0, "widths in blocks of 16");
  constexpr int QW = 16 * QB;               // queries per wave
  constexpr int XQ = 4 * QW;                // queries per workgroup
  constexpr int NKK = D / 4;                // k-steps of the first product
  constexpr int NCB = DV / 16;              // value column blocks
  constexpr float LOG2E = 1.4426950408889634f;
  constexpr float LN2 = 0.6931471805599453f;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const long long split = blockIdx.x % nsplit;
  const long long qt = blockIdx.x / nsplit;
  const long long head = blockIdx.y;
  const long long k_begin = split * keys_per_split;
  long long k_end = k_begin + keys_per_split;
  if (k_end > n) k_end = n;
  const int nkeys = (int)(k_end > k_begin ? k_end - k_begin : 0);   // < 2^31 / (4 max(D, DV))

  // B operands of the first product: Q[query][4 kk + g] * log2 e
  float qop[QB][NKK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const long long q = qt * XQ + wave * QW + qb * 16 + i16;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qop[qb][kk] = q < m ? Q[(head * m + q) * D + 4 * kk + g] * LOG2E : 0.f;
  }

  // resources at the slice's first key and value rows
  const __amdgpu_buffer_rsrc_t rk = sk_rsrc(K + (head * n + k_begin) * D);
  const __amdgpu_buffer_rsrc_t rv = sk_rsrc(V + (head * n + k_begin) * DV);
  // operands of one stage: key rows (A of the first product) and value rows (A of
  // the second); in the last, partial stage rows past the slice are clamped to
  // its last row (their p is 0)
  float kop[2][2][NKK], vop[2][2][4][NCB];
  auto fetch = [&](int kb0, int buf, auto part_c) {   // kb0: the stage's first key in the slice
    constexpr bool part = decltype(part_c)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int krow = 16 * kb + i16;
      int vrow[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) vrow[r] = 16 * kb + 4 * g + r;
      if constexpr (part) {
        const int last = nkeys - 1 - kb0;
        krow = krow < last ? krow : last;
#pragma unroll
        for (int r = 0; r < 4; ++r) vrow[r] = vrow[r] < last ? vrow[r] : last;
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kop[buf][kb][kk] = sk_ld(rk, 4u * (unsigned)(krow * D + 4 * kk + g), 4u * (unsigned)kb0 * D);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          vop[buf][kb][r][cb] =
              sk_ld(rv, 4u * (unsigned)(vrow[r] * DV + 16 * cb + i16), 4u * (unsigned)kb0 * DV);
    }
  };

  float ref[QB], l[QB];
  floatx4v acc[QB][NCB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    ref[qb] = -INFINITY;
    l[qb] = 0.f;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[qb][cb] = floatx4v{0.f, 0.f, 0.f, 0.f};

  auto stage = [&](int kb0, int buf, auto part_c) {
    constexpr bool part = decltype(part_c)::value;
    const int nk = nkeys - kb0 < SK_XK ? nkeys - kb0 : SK_XK;
    floatx4v sc[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[qb][kb] = floatx4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          sc[qb][kb] = mfma16x16x4(kop[buf][kb][kk], qop[qb][kk], sc[qb][kb]);
      }
    if constexpr (part) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + 4 * g + r >= nk) sc[qb][kb][r] = -INFINITY;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, sc[qb][kb][r]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      if (__any(mloc > ref[qb] + SK_XTAU)) {   // also the first stage (ref = -inf)
        const float rnew = fmaxf(ref[qb], mloc);   // finite: every stage has a key
        const float alpha = __builtin_amdgcn_exp2f(ref[qb] - rnew);   // 0 the first time
        l[qb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[qb][cb] *= alpha;
        ref[qb] = rnew;
      }
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = __builtin_amdgcn_exp2f(sc[qb][kb][r] - ref[qb]);
          sc[qb][kb][r] = pv;
          lsum += pv;
        }
      l[qb] += lsum;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[qb][cb] = mfma16x16x4(vop[buf][kb][r][cb], sc[qb][kb][r], acc[qb][cb]);
    }
  };

  // full stages in pairs (static buffer indices), each fetching the next one
  // ahead; the last, partial stage (if any) clamps its rows and masks its keys
  using Full = std::false_type;
  using Part = std::true_type;
  const int nfull = nkeys / SK_XK;
  const bool tail = nkeys % SK_XK != 0;
  if (nfull > 0) fetch(0, 0, Full{});
  else if (tail) fetch(0, 0, Part{});
  int st = 0;
  for (; st + 2 <= nfull; st += 2) {
    fetch((st + 1) * SK_XK, 1, Full{});
    stage(st * SK_XK, 0, Full{});
    if (st + 2 < nfull) fetch((st + 2) * SK_XK, 0, Full{});
    else if (tail) fetch((st + 2) * SK_XK, 0, Part{});
    stage((st + 1) * SK_XK, 1, Full{});
  }
  if (st < nfull) {                         // one full stage left, in buffer 0
    if (tail) fetch((st + 1) * SK_XK, 1, Part{});
    stage(st * SK_XK, 0, Full{});
    if (tail) stage((st + 1) * SK_XK, 1, Part{});
  } else if (tail) {
    stage(st * SK_XK, 0, Part{});
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float lt = l[qb] + __shfl_xor(l[qb], 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const long long q = qt * XQ + wave * QW + qb * 16 + i16;
    if (q < m) {
      float* P = parts + ((head * m + q) * nsplit + split) * (2 + DV);
      if (g == 0) {
        P[0] = ref[qb] * LN2;
        P[1] = lt;
      }
      // acc[qb][cb][r] = sum_i p_i v_i[c], c = 16 cb + 4 g + r
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) P[2 + 16 * cb + 4 * g + r] = acc[qb][cb][r];
    }
  }
}

// partial record per (head, query, slice): [mu, l, acc[dv]]
template <int B, int MQ>
__global__ __launch_bounds__(256)
void sk_exact_decode(const float* __restrict__ K, const float* __restrict__ V,
                     long long n, int d, int dv,
                     const float* __restrict__ Q, long long m,
                     long long keys_per_split, int nsplit,
                     float* __restrict__ parts) {
  constexpr int G = B / 4;            // lanes per key row
  constexpr int NG = 256 / G;         // key groups per workgroup
  __shared__ float sm_mu[MQ][NG];
  __shared__ float sm_l[MQ][NG];
  __shared__ float sm_acc[MQ][NG * B];

  const int tid = threadIdx.x;
  const int gl = tid % G;             // lane within the group
  const int grp = tid / G;
  const int c4 = gl * 4;
  const bool kin = c4 < d, vin = c4 < dv;
  const long long split = blockIdx.x;
  const long long head = blockIdx.y;
  const long long k_begin = split * keys_per_split;
  long long k_end = k_begin + keys_per_split;
  if (k_end > n) k_end = n;

  const float* Kh = K + head * n * d;
  const float* Vh = V + head * n * dv;

  // base-2 softmax: queries prescaled by log2 e, maxima in log2 units until the
  // record
  constexpr float LOG2E = 1.4426950408889634f;
  constexpr float LN2 = 0.6931471805599453f;
  float4 q4[MQ];
  float mu[MQ], l[MQ];
  float4 acc[MQ];
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    q4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < m && kin) {
      q4[i] = *reinterpret_cast<const float4*>(Q + (head * m + i) * d + c4);
      q4[i].x *= LOG2E; q4[i].y *= LOG2E; q4[i].z *= LOG2E; q4[i].w *= LOG2E;
    }
    mu[i] = -INFINITY;
    l[i] = 0.f;
    acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  for (long long kb = k_begin + grp; kb < k_end; kb += (long long)NG * SK_EX_U) {
    float4 k4[SK_EX_U], v4[SK_EX_U];
    bool ok[SK_EX_U];
#pragma unroll
    for (int u = 0; u < SK_EX_U; ++u) {
      const long long key = kb + (long long)u * NG;
      ok[u] = key < k_end;
      k4[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      v4[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      // streamed once: non-temporal loads
      if (ok[u] && kin) k4[u] = ld_stream(Kh + key * d + c4);
      if (ok[u] && vin) v4[u] = ld_stream(Vh + key * dv + c4);
    }
#pragma unroll
    for (int i = 0; i < MQ; ++i) {
      if (i >= m) break;
      float s[SK_EX_U];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < SK_EX_U; ++u) {
        float p = q4[i].x * k4[u].x + q4[i].y * k4[u].y + q4[i].z * k4[u].z +
                  q4[i].w * k4[u].w;
        p = group_sum<G>(p);
        s[u] = ok[u] ? p : -INFINITY;
        mx = fmaxf(mx, s[u]);
      }
      if (mx == -INFINITY) continue;
      const float mnew = fmaxf(mu[i], mx);
      const float alpha = __builtin_amdgcn_exp2f(mu[i] - mnew);
      float lb = 0.f;
      float4 ab = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < SK_EX_U; ++u) {
        const float w = __builtin_amdgcn_exp2f(s[u] - mnew);   // 2^-inf = 0 for missing keys
        lb += w;
        ab.x += w * v4[u].x; ab.y += w * v4[u].y;
        ab.z += w * v4[u].z; ab.w += w * v4[u].w;
      }
      l[i] = l[i] * alpha + lb;
      acc[i].x = acc[i].x * alpha + ab.x; acc[i].y = acc[i].y * alpha + ab.y;
      acc[i].z = acc[i].z * alpha + ab.z; acc[i].w = acc[i].w * alpha + ab.w;
      mu[i] = mnew;
    }
  }

  // fold the NG groups of this workgroup, in group order
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    if (gl == 0) { sm_mu[i][grp] = mu[i]; sm_l[i][grp] = l[i]; }
    sm_acc[i][grp * B + c4 + 0] = acc[i].x;
    sm_acc[i][grp * B + c4 + 1] = acc[i].y;
    sm_acc[i][grp * B + c4 + 2] = acc[i].z;
    sm_acc[i][grp * B + c4 + 3] = acc[i].w;
  }
  __syncthreads();
  for (int i = 0; i < MQ && i < m; ++i) {
    float ms = -INFINITY;
    for (int g = 0; g < NG; ++g) ms = fmaxf(ms, sm_mu[i][g]);
    float* P = parts + ((head * m + i) * nsplit + split) * (2 + dv);
    if (tid <= dv) {
      float sum = 0.f;
      if (ms != -INFINITY) {
        for (int g = 0; g < NG; ++g) {
          const float sc = __builtin_amdgcn_exp2f(sm_mu[i][g] - ms);
          sum += (tid == 0 ? sm_l[i][g] : sm_acc[i][g * B + tid - 1]) * sc;
        }
      }
      if (tid == 0) { P[0] = ms * LN2; P[1] = sum; }
      else P[1 + tid] = sum;
    }
  }
}

template <int B, int KS>
__global__ __launch_bounds__(256)
void sk_exact_tiled(const float* __restrict__ K, const float* __restrict__ V,
                    long long n, int d, int dv,
                    const float* __restrict__ Q, long long m,
                    long long keys_per_split, int nsplit,
                    float* __restrict__ parts) {
  __shared__ float4 Ks4[KS * B / 4];
  __shared__ float4 Vs4[KS * B / 4];
  const float* Ks = reinterpret_cast<const float*>(Ks4);
  const float* Vs = reinterpret_cast<const float*>(Vs4);
  const int tid = threadIdx.x;
  const long long split = blockIdx.x % nsplit;
  const long long qt = blockIdx.x / nsplit;
  const long long head = blockIdx.y;
  const long long q = qt * 256 + tid;
  const bool qok = q < m;

  const long long k_begin = split * keys_per_split;
  long long k_end = k_begin + keys_per_split;
  if (k_end > n) k_end = n;
  const float* Kh = K + head * n * d;
  const float* Vh = V + head * n * dv;

  // base-2 softmax: query prescaled by log2 e, mu in log2 units until the record
  constexpr float LOG2E = 1.4426950408889634f;
  constexpr float LN2 = 0.6931471805599453f;
  float qr[B], acc[B];
#pragma unroll
  for (int c = 0; c < B; ++c) {
    qr[c] = (qok && c < d) ? Q[(head * m + q) * d + c] * LOG2E : 0.f;
    acc[c] = 0.f;
  }
  float mu = -INFINITY, l = 0.f;
  const int d4 = d >> 2, dv4 = dv >> 2;

  for (long long kb0 = k_begin; kb0 < k_end; kb0 += KS) {
    const long long left = k_end - kb0;
    const int nk = left < KS ? (int)left : KS;
    __syncthreads();
    for (int i = tid; i < KS * (B / 4); i += 256) {
      const int kk = i / (B / 4), c4 = i % (B / 4);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
      if (kk < nk) {
        if (c4 < d4) x = *reinterpret_cast<const float4*>(Kh + (kb0 + kk) * d + 4 * c4);
        if (c4 < dv4) y = *reinterpret_cast<const float4*>(Vh + (kb0 + kk) * dv + 4 * c4);
      }
      Ks4[i] = x;
      Vs4[i] = y;
    }
    __syncthreads();
    float s[KS];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < B; ++c) a += qr[c] * Ks[kk * B + c];
      s[kk] = kk < nk ? a : -INFINITY;
      mx = fmaxf(mx, s[kk]);
    }
    const float mnew = fmaxf(mu, mx);
    const float alpha = __builtin_amdgcn_exp2f(mu - mnew);
    float lb = 0.f;
    // Per-stage sums first (two-level summation); at B = 128 the stage sum of
    // the values would not fit in registers, so the values go straight in.
    constexpr bool kStage = B <= 64;
    float ab[kStage ? B : 1];
#pragma unroll
    for (int c = 0; c < B; ++c) {
      if (kStage) ab[c] = 0.f;
      else acc[c] *= alpha;
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const float w = __builtin_amdgcn_exp2f(s[kk] - mnew);
      lb += w;
#pragma unroll
      for (int c = 0; c < B; ++c) {
        if (kStage) ab[c] += w * Vs[kk * B + c];
        else acc[c] += w * Vs[kk * B + c];
      }
    }
    l = l * alpha + lb;
    if (kStage) {
#pragma unroll
      for (int c = 0; c < B; ++c) acc[c] = acc[c] * alpha + ab[kStage ? c : 0];
    }
    mu = mnew;
  }
  if (qok) {
    float* P = parts + ((head * m + q) * nsplit + split) * (2 + dv);
    P[0] = mu * LN2;
    P[1] = l;
#pragma unroll
    for (int c = 0; c < B; ++c)
      if (c < dv) P[2 + c] = acc[c];
  }
}

// One workgroup per (head, query): exact_fold of its slice records.  (1024
// threads, for two rounds of loads over the 512 slices of a 1M-key head instead
// of five, measured the same: 52.4 us per decode call.)
__global__ __launch_bounds__(256)
void sk_exact_combine(const float* __restrict__ parts, int nsplit, long long m, int dv,
                      int h, float* __restrict__ out, float* __restrict__ Z) {
  __shared__ float red[256];
  __shared__ float lsum;
  const long long hq = blockIdx.x;
  exact_fold<256>(parts + hq * (long long)nsplit * (2 + dv), nsplit, dv, out + hq * dv, Z + hq,
                  red, &lsum);
}
