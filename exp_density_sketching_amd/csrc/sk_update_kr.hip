// One instantiation of the digit-organised update kernel (sk_update_kr.h) per
// object file: the build compiles this file once per (KR_RT, KR_CENTER), in
// parallel, and expsketch.hip declares the instantiations extern.
#include <hip/hip_runtime.h>

#include "sk_update_kr.h"

#if !defined(KR_RT) || !defined(KR_CENTER)
#error "compile with -DKR_RT=<1|2|4> -DKR_CENTER=<0|1>"
#endif

template __global__ void sk_update_kr_kernel<KR_RT, (KR_CENTER != 0)>(
    const float*, const float*, long long, long long, int, const KrUnit*, KrSplits, int, float*,
    long long, long long, int, const float*, PendingReduce);
