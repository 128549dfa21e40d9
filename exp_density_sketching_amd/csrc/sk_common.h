// Common device-side definitions for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4v __attribute__((ext_vector_type(4)));

#define SK_WG 256          // threads per workgroup in every GEMM-shaped kernel
#define SK_KB 32           // keys (update) or feature rows (query) per LDS stage
#define SK_PAD 32          // LDS row padding: lanes 32..63 land on other banks
#define SK_MAXDIG 8        // max Kronecker digits on either side of a level split

// v_mfma_f32_32x32x2_f32: D(32x32) += A(32x2) * B(2x32), fp32 in and out.
// Lane l supplies A[l%32][l/32] and B[l/32][l%32]; accumulator register r of
// lane l holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ floatx16 mfma32x32x2(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x4_f32: D(16x16) += A(16x4) * B(4x16), fp32 in and out.
// Lane l supplies A[l%16][l/16] and B[l/16][l%16]; accumulator register r of lane
// l holds D[4*(l/16) + r][l%16].
__device__ __forceinline__ floatx4v mfma16x16x4(float a, float b, floatx4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Raw buffer loads: a resource for a wave-uniform base (scalar registers), a
// byte offset per lane in a vector register and a wave-uniform byte offset in a
// scalar register; no per-lane 64-bit address arithmetic.  Callers keep every
// offset in bounds (the resource's range is only an upper limit).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const float* base) {
  // raw buffer: stride 0, the largest range, the gfx9 format word of 32-bit data
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}
__device__ __forceinline__ float sk_ld(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.
// Map dispatch index p to a logical index so that every XCD works through one
// contiguous range of logical indices: neighbours in logical order (tiles that
// read the same keys, or the same state rows) then share an L2.
#define SK_NXCD 8
__device__ __forceinline__ long long xcd_remap(long long p, long long total) {
  const long long x = p % SK_NXCD, i = p / SK_NXCD;
  const long long q = total / SK_NXCD, rem = total % SK_NXCD;
  return (x < rem) ? x * (q + 1) + i : rem * (q + 1) + (x - rem) * q + i;
}

// Tile descriptor of the moment update: one (level, row tile, column tile) of the
// level's GEMM  X_j[a_hi][(a_lo, e)] += sum_keys L[a_hi](k) * R[(a_lo, e)](k, v)
// with L = k^(x)s (s leading digits) and R = k^(x)t (x) u, u = [k, v] below the
// top level and u = v at the top level.
struct UpdTile {
  long long xoff;   // float offset of level j inside one head's state
  int level;
  int s, t;         // digits on the row side and on the column side (s + t = j)
  int C;            // the level's row width (d + dv, or dv at the top)
  int top;          // 1 at j == p
  int M, N;         // GEMM rows (d^s) and columns (d^t * C)
  int row0, col0;   // tile origin inside the level GEMM
  int wc;           // waves along the column side: 1, 2 or 4 (tile 256/wc x 64*wc)
  int pad_;
};

// Tile descriptor of the query of level j.  The level's Kronecker index is split
// into s leading digits a_hi (the GEMM's reduction index) and t trailing digits
// a_lo; the GEMM is
//     Y[q][(a_lo, e)] = sum_{a_hi in [a0, a1)} q^(x)s[a_hi] * X_j[a_hi][(a_lo, e)]
// over N = d^t * C columns, one tile owning 128 of them; the epilogue then folds
// a_lo with the weights q^(x)t[a_lo].
struct QryTile {
  long long xoff;   // float offset of level j inside one head's state
  long long a0, a1; // a_hi range
  long long pofs;   // offset of this tile's [128][C] partial in a query-tile block
  int level;
  int C;            // row width of the level
  int top;
  int s, t;
  int N;            // d^t * C
  int col0;         // first GEMM column of the tile
  int alo0, nalo;   // a_lo values the tile's columns touch
  float wz, wn;     // 1/(j+1)! (weights of M_{j+1}), 1/j! (weights of N_j)
  int fc0, fw;      // the partial holds columns fc0 .. fc0 + fw - 1 of the level: [128][fw]
};
