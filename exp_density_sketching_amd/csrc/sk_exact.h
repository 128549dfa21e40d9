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
// sk_exact_tiled   (many queries per head): one thread per query, key and value
//   rows staged through LDS and read as broadcasts; per stage of 32 keys one
//   rescale.
// sk_exact_combine: folds the slice partials of each (head, query).
#pragma once

#include "sk_common.h"

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

  float4 q4[MQ];
  float mu[MQ], l[MQ];
  float4 acc[MQ];
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    q4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < m && kin) q4[i] = *reinterpret_cast<const float4*>(Q + (head * m + i) * d + c4);
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
      const float alpha = expf(mu[i] - mnew);
      float lb = 0.f;
      float4 ab = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < SK_EX_U; ++u) {
        const float w = expf(s[u] - mnew);   // exp(-inf) = 0 for missing keys
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
          const float sc = expf(sm_mu[i][g] - ms);
          sum += (tid == 0 ? sm_l[i][g] : sm_acc[i][g * B + tid - 1]) * sc;
        }
      }
      if (tid == 0) { P[0] = ms; P[1] = sum; }
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

  float qr[B], acc[B];
#pragma unroll
  for (int c = 0; c < B; ++c) {
    qr[c] = (qok && c < d) ? Q[(head * m + q) * d + c] : 0.f;
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
    const float alpha = expf(mu - mnew);
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
      const float w = expf(s[kk] - mnew);
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
    P[0] = mu;
    P[1] = l;
#pragma unroll
    for (int c = 0; c < B; ++c)
      if (c < dv) P[2 + c] = acc[c];
  }
}

// One workgroup per (head, query).  The slices' maxima are reduced first; then
// thread (g, slot) sums slot 0 (l) or slot 1 + c (acc[c]) over slices g, g + G,
// ... with the rescale e^(mu_s - mu*), and the G group sums are added in group
// order.  Fixed order throughout, so the result does not depend on timing.
__global__ __launch_bounds__(256)
void sk_exact_combine(const float* __restrict__ parts, int nsplit, long long m, int dv,
                      int h, float* __restrict__ out, float* __restrict__ Z) {
  __shared__ float red[256];
  __shared__ float lsum;
  const long long hq = blockIdx.x;
  const int tid = threadIdx.x;
  const int rec = 2 + dv;
  const float* P = parts + hq * (long long)nsplit * rec;
  float mx = -INFINITY;
  for (int sp = tid; sp < nsplit; sp += 256) mx = fmaxf(mx, P[(long long)sp * rec]);
  red[tid] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float ms = red[0];
  __syncthreads();
  const int slots = 1 + dv;
  const int groups = 256 / slots > 0 ? 256 / slots : 1;
  const int g = tid / slots, slot = tid - g * slots;
  float acc = 0.f;
  if (g < groups && ms != -INFINITY) {
    for (int sp = g; sp < nsplit; sp += groups) {
      const float* r = P + (long long)sp * rec;
      acc += r[1 + slot] * expf(r[0] - ms);
    }
  }
  red[tid] = acc;
  __syncthreads();
  float sum = 0.f;
  if (tid < slots) {
    for (int gg = 0; gg < groups; ++gg) sum += red[gg * slots + tid];
    if (tid == 0) lsum = sum;
  }
  __syncthreads();
  if (tid == 0) Z[hq] = (ms == -INFINITY) ? 0.f : expf(ms) * lsum;
  else if (tid < slots) out[hq * dv + (tid - 1)] = sum / lsum;
}
