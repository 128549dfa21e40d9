// Device-side pieces of the fixed-order split reduction, shared by the
// elementwise kernels and the update kernels.
#pragma once

#include "sk_common.h"

// state[i] += (part_0 + part_1 + ... + part_{ns-1})[i], partials summed in split
// order (the one order every path uses, so results do not depend on the path).
__device__ __forceinline__ void split_reduce_one(float4* __restrict__ state,
                                                 const float4* __restrict__ parts,
                                                 long long i, int nsplit,
                                                 long long split_stride4) {
  float4 t = parts[i];
#pragma unroll 8
  for (int sp = 1; sp < nsplit; ++sp) {
    const float4 b = parts[sp * split_stride4 + i];
    t.x += b.x; t.y += b.y; t.z += b.z; t.w += b.w;
  }
  float4 a = state[i];
  a.x += t.x; a.y += t.y; a.z += t.z; a.w += t.w;
  state[i] = a;
}

// The previous update call's split partials, added into the state by extra
// workgroups of the next update launch (queued after its tiles, so they run in
// the launch's tail).  Workgroup w of them takes float4 [w * SK_RED4, (w + 1) *
// SK_RED4), one per thread, so small states still spread over many workgroups.
// The launch's own tiles write the other partials buffer, never the state, so
// the two do not touch the same memory.
#define SK_RED4 256
struct PendingReduce {
  float4* state;
  const float4* parts;   // null: nothing pending
  long long count4;      // float4 of the state (all heads)
  int nsplit;
  int pad_;
};
__device__ __forceinline__ void pending_reduce_wg(const PendingReduce& r, long long w) {
  const long long i0 = w * SK_RED4;
  for (long long i = i0 + threadIdx.x; i < i0 + SK_RED4 && i < r.count4; i += blockDim.x)
    split_reduce_one(r.state, r.parts, i, r.nsplit, r.count4);
}
