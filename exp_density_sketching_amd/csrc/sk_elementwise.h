// Elementwise kernels over the state: merge, split-K reduction, zero fill, and the
// canonical [M | N] view.
#pragma once

#include "sk_common.h"
#include "sk_reduce.h"

#define SK_MAXLEV 17

// dst += src over `count4` float4s (merge of two sketches: moments add; the
// Merge step of Merge-and-Reduce, "Rumo a Limites Estritos para Atenção em
// Streaming", "Metodologia", closing paragraph).
__global__ __launch_bounds__(256)
void sk_add_kernel(float4* __restrict__ dst, const float4* __restrict__ src, long long count4) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < count4;
       i += (long long)gridDim.x * blockDim.x) {
    float4 a = dst[i];
    const float4 b = src[i];
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    dst[i] = a;
  }
}

__global__ __launch_bounds__(256)
void sk_split_reduce_kernel(float4* __restrict__ state, const float4* __restrict__ parts,
                            long long count4, int nsplit, long long split_stride4) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < count4;
       i += (long long)gridDim.x * blockDim.x)
    split_reduce_one(state, parts, i, nsplit, split_stride4);
}

// Appends one call's keys and values to the staging buffers: the n rows of head
// hh of K (d4 float4 each) and of V (dv4 float4 each) go to rows [off, off + n)
// of that head's block of cap rows.  Workgroup w copies part w % nb of segment
// w / nb, segment 2 hh being head hh's K rows and 2 hh + 1 its V rows, so one
// launch moves both, 128 bits per thread.
__global__ __launch_bounds__(256)
void sk_stage_copy_kernel(const float4* __restrict__ K, const float4* __restrict__ V,
                          long long n, int d4, int dv4, int nb,
                          float4* __restrict__ sk, float4* __restrict__ sv,
                          long long cap, long long off) {
  const long long seg = blockIdx.x / nb;
  const int part = (int)(blockIdx.x - seg * nb);
  const long long hh = seg >> 1;
  const bool isv = (seg & 1) != 0;
  const int w4 = isv ? dv4 : d4;
  const long long cnt = n * w4;
  const float4* src = (isv ? V : K) + hh * cnt;
  float4* dst = (isv ? sv : sk) + (hh * cap + off) * w4;
  for (long long i = (long long)part * blockDim.x + threadIdx.x; i < cnt;
       i += (long long)nb * blockDim.x)
    dst[i] = src[i];
}

__global__ __launch_bounds__(256)
void sk_fill_zero_kernel(float4* __restrict__ p, long long count4) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < count4;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

struct LevelTable {
  long long row_start[SK_MAXLEV];  // first canonical row of level j
  long long xoff[SK_MAXLEV];       // offset of X_j in the level-fold layout
  int C[SK_MAXLEV];                // row width of X_j
  int p;
};

// Canonical [M | N] (per head [D][1 + dv]) from the level-fold layout.
// Row r of level j (local index a): column 0 is M_j[a] (the count for j = 0,
// else X_{j-1}[a / d][a % d]); column 1 + c is N_j[a][c] (X_j[a][d + c] below
// the top level, X_p[a][c] at the top).
__global__ __launch_bounds__(256)
void sk_export_kernel(const float* __restrict__ X, long long head_stride, LevelTable lt,
                      long long D, int d, int logd, int dv, float count,
                      float* __restrict__ dst, long long total) {
  const int cols = 1 + dv;
  for (long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (long long)gridDim.x * blockDim.x) {
    const long long head = g / (D * cols);
    const long long rem = g - head * D * cols;
    const long long r = rem / cols;
    const int c = (int)(rem - r * cols);
    int j = 0;
    while (j < lt.p && r >= lt.row_start[j + 1]) ++j;
    const long long a = r - lt.row_start[j];
    const float* Xh = X + head * head_stride;
    float v;
    if (c == 0) {
      if (j == 0) v = count;
      else v = Xh[lt.xoff[j - 1] + (a >> logd) * lt.C[j - 1] + (a & (d - 1))];
    } else {
      if (j < lt.p) v = Xh[lt.xoff[j] + a * lt.C[j] + d + (c - 1)];
      else v = Xh[lt.xoff[j] + a * lt.C[j] + (c - 1)];
    }
    dst[g] = v;
  }
}
