// Host side of libexpsketch: argument checks, launch planning, state ownership.
// The C ABI is declared (with the passages each call follows) in expsketch.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "expsketch.h"
#include "sk_common.h"
#include "sk_elementwise.h"
#include "sk_exact.h"
#include "sk_query.h"
#include "sk_update.h"

namespace {

#define SK_TRY(expr)                               \
  do {                                             \
    if ((expr) != hipSuccess) return SK_EHIP;      \
  } while (0)

constexpr int kMaxP = 16;
// a_hi rows per query tile (EXPSKETCH_QUERY_ROWS overrides, tuning aid)
long long query_rows_per_tile() {
  static const long long v = [] {
    const char* e = std::getenv("EXPSKETCH_QUERY_ROWS");
    const long long r = e ? std::atoll(e) : 0;
    return r >= SK_KB ? r / SK_KB * SK_KB : 512LL;
  }();
  return v;
}

bool is_pow2_in(int x, int lo, int hi) {
  return x >= lo && x <= hi && (x & (x - 1)) == 0;
}
int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct DeviceInfo {
  int num_cu = 0;
  int max_lds = 0;
  bool pool_ready = false;
};

std::mutex g_dev_mutex;
std::vector<DeviceInfo> g_dev;

int device_info(int dev, DeviceInfo* out) {
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  DeviceInfo& di = g_dev[dev];
  if (di.num_cu == 0) {
    SK_TRY(hipDeviceGetAttribute(&di.num_cu, hipDeviceAttributeMultiprocessorCount, dev));
    SK_TRY(hipDeviceGetAttribute(&di.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    // Keep freed stream-ordered allocations in the pool: the per-call
    // workspaces are re-taken on every call.
    hipMemPool_t pool;
    if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
      uint64_t thr = UINT64_MAX;
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
    }
    (void)hipGetLastError();
    di.pool_ready = true;
  }
  *out = di;
  return SK_OK;
}

int current_device(int* dev) {
  SK_TRY(hipGetDevice(dev));
  return SK_OK;
}

size_t update_lds_bytes(int d, int dv) {
  // Ks + Vs (transposed, stride SK_KB + 1) + Lt + Rt with (TM + TN + 2 * pad) <= 384
  return sizeof(float) * ((size_t)(SK_KB + 1) * (d + dv) + (size_t)SK_KB * 384);
}
size_t query_lds_bytes(int d) {
  // Qs + max(At + Bt, Ys)
  const size_t ab = (size_t)SK_KB * (SK_TMQ + SK_PAD) + (size_t)SK_KB * (SK_TNQ + SK_PAD);
  const size_t ys = (size_t)64 * (SK_TNQ + 1);
  return sizeof(float) * ((size_t)d * (SK_TMQ + 1) + std::max(ab, ys));
}

// The query kernel is instantiated per log2(d) (d = 4 .. 128).
using QueryKernel = void (*)(const float*, long long, const float*, long long,
                             const QryTile*, int, int, long long, float*);
QueryKernel query_kernel_for(int logd) {
  switch (logd) {
    case 2: return sk_query_kernel<2>;
    case 3: return sk_query_kernel<3>;
    case 4: return sk_query_kernel<4>;
    case 5: return sk_query_kernel<5>;
    case 6: return sk_query_kernel<6>;
    case 7: return sk_query_kernel<7>;
    default: return nullptr;
  }
}

}  // namespace

struct sk_sketch {
  int d = 0, dv = 0, p = 0, h = 0, logd = 0;
  int device = 0;
  long long D = 0;          // sum_{j<=p} d^j
  long long XS = 0;         // floats per head in the level-fold layout
  int64_t count = 0;        // keys per head ingested (M_0)
  hipStream_t stream = nullptr;
  float* state = nullptr;   // [h][XS]
  std::vector<long long> xoff, rows;
  std::vector<int> C;
  std::vector<UpdTile> utiles;
  std::vector<QryTile> qtiles;
  UpdTile* d_utiles = nullptr;
  QryTile* d_qtiles = nullptr;
  long long qpb = 0;        // floats of query partials per (head, query tile)
  float* view = nullptr;    // canonical view buffer
  bool timing = false;      // kernel timing (sketch_timing)
  std::vector<hipEvent_t> tev[2][2];   // [kind][start, stop], created on first use
  int trec[2] = {0, 0};     // pairs recorded per kind
  size_t view_bytes = 0;
  DeviceInfo dev;
};

namespace {

constexpr int kTimingPairs = 256;

// Records the start (stop = false) or stop event of the current pair of `kind`.
void timing_mark(sk_sketch* s, int kind, bool stop) {
  if (!s->timing || s->trec[kind] >= (int)s->tev[kind][0].size()) return;
  (void)hipEventRecord(s->tev[kind][stop ? 1 : 0][s->trec[kind]], s->stream);
  if (stop) ++s->trec[kind];
}

// Level split and tile shape of the update GEMM for one level: fewest tiles.
void plan_update_level(sk_sketch* s, int j, std::vector<UpdTile>* out) {
  const int d = s->d, C = s->C[j];
  long long best_tiles = -1;
  UpdTile best{};
  const int wcs[3] = {2, 1, 4};
  for (int wi = 0; wi < 3; ++wi) {
    const int wc = wcs[wi];
    const int TM = SK_WG / wc, TN = 64 * wc;
    for (int ss = 0; ss <= j; ++ss) {
      const int tt = j - ss;
      if (ss > SK_MAXDIG || tt > SK_MAXDIG) continue;
      const double Md = std::pow((double)d, ss);
      const double Nd = std::pow((double)d, tt) * C;
      if (Md >= (double)(1 << 30) || Nd >= (double)(1 << 30)) continue;
      const long long M = (long long)Md, N = (long long)Nd;
      const long long tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
      if (best_tiles < 0 || tiles < best_tiles) {
        best_tiles = tiles;
        best = UpdTile{};
        best.xoff = s->xoff[j];
        best.level = j;
        best.s = ss;
        best.t = tt;
        best.C = C;
        best.top = (j == s->p);
        best.M = (int)M;
        best.N = (int)N;
        best.wc = wc;
      }
    }
  }
  const int TM = SK_WG / best.wc, TN = 64 * best.wc;
  for (int r0 = 0; r0 < best.M; r0 += TM)
    for (int c0 = 0; c0 < best.N; c0 += TN) {
      UpdTile t = best;
      t.row0 = r0;
      t.col0 = c0;
      out->push_back(t);
    }
}

// Query tiles of level j: t trailing digits in the columns (the fewest giving at
// least SK_TNQ columns), 128-column tiles, a_hi ranges of query_rows_per_tile().
void plan_query_level(sk_sketch* s, int j, std::vector<QryTile>* out, long long* pb) {
  const int d = s->d, C = s->C[j];
  int t = j;
  for (int tt = 0; tt <= j; ++tt) {
    if (std::pow((double)d, tt) * C >= SK_TNQ) { t = tt; break; }
  }
  while (t > SK_MAXDIG) --t;
  const int sd = j - t;
  const long long N = (long long)std::llround(std::pow((double)d, t)) * C;
  const long long Kr = (long long)std::llround(std::pow((double)d, sd));
  double fj = 1.0;
  for (int i = 2; i <= j; ++i) fj *= i;
  for (long long col0 = 0; col0 < N; col0 += SK_TNQ) {
    const long long last = std::min(N, col0 + SK_TNQ) - 1;
    for (long long a0 = 0; a0 < Kr; a0 += query_rows_per_tile()) {
      QryTile q{};
      q.xoff = s->xoff[j];
      q.a0 = a0;
      q.a1 = std::min(Kr, a0 + query_rows_per_tile());
      q.pofs = *pb;
      q.level = j;
      q.C = C;
      q.top = (j == s->p);
      q.s = sd;
      q.t = t;
      q.N = (int)N;
      q.col0 = (int)col0;
      q.alo0 = (int)(col0 / C);
      q.nalo = (int)(last / C - col0 / C + 1);
      q.wz = (float)(1.0 / (fj * (j + 1)));
      q.wn = (float)(1.0 / fj);
      *pb += (long long)SK_TMQ * C;
      out->push_back(q);
    }
  }
}

int choose_update_splits(const sk_sketch* s, long long n) {
  // EXPSKETCH_UPDATE_SPLITS=<k> fixes the number of key splits (tuning aid).
  static const int forced = [] {
    const char* v = std::getenv("EXPSKETCH_UPDATE_SPLITS");
    return v ? std::max(0, std::atoi(v)) : 0;
  }();
  if (forced > 0) return (int)std::max(1LL, std::min<long long>(forced, (n + SK_KB - 1) / SK_KB));
  const long long base = (long long)s->utiles.size() * s->h;
  const long long slots = 2LL * std::max(1, s->dev.num_cu);
  const long long max_ns = std::max(1LL, std::min(64LL, n / 256));
  int best = 1;
  double best_score = -1.0;
  for (long long ns = 1; ns <= max_ns; ++ns) {
    const long long wgs = base * ns;
    const long long waves = (wgs + slots - 1) / slots;
    const double eff = (double)wgs / (double)(waves * slots);
    const double score = eff - 0.005 * (double)ns;
    if (score > best_score + 1e-9) {
      best_score = score;
      best = (int)ns;
    }
  }
  return best;
}

int launch_fill_zero(float* p, long long count, hipStream_t st) {
  const long long c4 = count / 4;
  if (c4 == 0) return SK_OK;
  const int grid = (int)std::min<long long>((c4 + 255) / 256, 8192);
  hipLaunchKernelGGL(sk_fill_zero_kernel, dim3(grid), dim3(256), 0, st,
                     reinterpret_cast<float4*>(p), c4);
  SK_TRY(hipGetLastError());
  return SK_OK;
}

}  // namespace

extern "C" {

int sk_version(void) { return 100; }

const char* sk_strerror(int code) {
  switch (code) {
    case SK_OK: return "ok";
    case SK_EINVAL: return "invalid argument";
    case SK_ENOMEM: return "out of device memory";
    case SK_EMISMATCH: return "sketch shapes differ";
    case SK_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int sketch_create(int d, int dv, int p, int h, void* hip_stream, sk_handle* out) {
  if (out == nullptr) return SK_EINVAL;
  *out = nullptr;
  if (!is_pow2_in(d, 4, 128) || !is_pow2_in(dv, 4, 128) || p < 0 || p > kMaxP || h < 1)
    return SK_EINVAL;
  // sizes, with overflow checks in floating point first
  double XSd = 0.0;
  for (int j = 0; j <= p; ++j) {
    const double r = std::pow((double)d, j);
    XSd += r * (double)(j < p ? d + dv : dv);
  }
  if (XSd * (double)h * 4.0 > 1.0e15) return SK_ENOMEM;

  sk_sketch* s = new (std::nothrow) sk_sketch();
  if (s == nullptr) return SK_ENOMEM;
  s->d = d; s->dv = dv; s->p = p; s->h = h; s->logd = ilog2(d);
  s->stream = reinterpret_cast<hipStream_t>(hip_stream);
  int rc = current_device(&s->device);
  if (rc == SK_OK) rc = device_info(s->device, &s->dev);
  if (rc != SK_OK) { delete s; return rc; }
  long long off = 0, r = 1, D = 0;
  for (int j = 0; j <= p; ++j) {
    s->rows.push_back(r);
    s->C.push_back(j < p ? d + dv : dv);
    s->xoff.push_back(off);
    off += r * s->C[j];
    D += r;
    r *= d;
  }
  s->D = D;
  s->XS = off;   // a multiple of 4: every term is
  if (update_lds_bytes(d, dv) > (size_t)s->dev.max_lds ||
      query_lds_bytes(d) > (size_t)s->dev.max_lds) {
    delete s;
    return SK_EINVAL;
  }
  for (int j = 0; j <= p; ++j) plan_update_level(s, j, &s->utiles);

  for (int j = 0; j <= p; ++j) plan_query_level(s, j, &s->qtiles, &s->qpb);

  const size_t state_bytes = sizeof(float) * (size_t)s->XS * (size_t)h;
  if (hipMalloc(&s->state, state_bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete s;
    return SK_ENOMEM;
  }
  bool ok = hipMalloc(&s->d_utiles, sizeof(UpdTile) * s->utiles.size()) == hipSuccess &&
            hipMalloc(&s->d_qtiles, sizeof(QryTile) * s->qtiles.size()) == hipSuccess;
  if (ok)
    ok = hipMemcpy(s->d_utiles, s->utiles.data(), sizeof(UpdTile) * s->utiles.size(),
                   hipMemcpyHostToDevice) == hipSuccess &&
         hipMemcpy(s->d_qtiles, s->qtiles.data(), sizeof(QryTile) * s->qtiles.size(),
                   hipMemcpyHostToDevice) == hipSuccess;
  if (ok) {
    const size_t ul = update_lds_bytes(d, dv), ql = query_lds_bytes(d);
    ok = hipFuncSetAttribute((const void*)sk_update_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ul) == hipSuccess &&
         hipFuncSetAttribute((const void*)query_kernel_for(s->logd),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ql) == hipSuccess;
  }
  if (ok) ok = launch_fill_zero(s->state, s->XS * h, s->stream) == SK_OK;
  if (!ok) {
    (void)hipGetLastError();
    (void)hipFree(s->state); (void)hipFree(s->d_utiles); (void)hipFree(s->d_qtiles);
    delete s;
    return SK_EHIP;
  }
  *out = s;
  return SK_OK;
}

int sketch_destroy(sk_handle s) {
  if (s == nullptr) return SK_OK;
  int rc = SK_OK;
  if (hipStreamSynchronize(s->stream) != hipSuccess) rc = SK_EHIP;
  (void)hipFree(s->state);
  (void)hipFree(s->d_utiles);
  (void)hipFree(s->d_qtiles);
  (void)hipFree(s->view);
  for (int k = 0; k < 2; ++k)
    for (int w = 0; w < 2; ++w)
      for (hipEvent_t e : s->tev[k][w]) (void)hipEventDestroy(e);
  delete s;
  return rc;
}

int sketch_set_stream(sk_handle s, void* hip_stream) {
  if (s == nullptr) return SK_EINVAL;
  s->stream = reinterpret_cast<hipStream_t>(hip_stream);
  return SK_OK;
}

int sketch_reset(sk_handle s) {
  if (s == nullptr) return SK_EINVAL;
  s->count = 0;
  return launch_fill_zero(s->state, s->XS * s->h, s->stream);
}

int sketch_info(sk_handle s, int* d, int* dv, int* p, int* h, int64_t* D, int64_t* count) {
  if (s == nullptr) return SK_EINVAL;
  if (d) *d = s->d;
  if (dv) *dv = s->dv;
  if (p) *p = s->p;
  if (h) *h = s->h;
  if (D) *D = s->D;
  if (count) *count = s->count;
  return SK_OK;
}

int sketch_update(sk_handle s, const float* K, const float* V, int64_t n) {
  if (s == nullptr || n < 0) return SK_EINVAL;
  if (n == 0) return SK_OK;
  if (K == nullptr || V == nullptr || !aligned16(K) || !aligned16(V)) return SK_EINVAL;
  const int ns = choose_update_splits(s, n);
  long long kps = (n + ns - 1) / ns;
  kps = (kps + SK_KB - 1) / SK_KB * SK_KB;
  const int nsplit = (int)((n + kps - 1) / kps);
  const int ntiles = (int)s->utiles.size();
  if ((long long)ntiles * nsplit * s->h > 0x7fffffffLL) return SK_EINVAL;
  const size_t lds = update_lds_bytes(s->d, s->dv);
  const long long total = s->XS * s->h;
  float* parts = nullptr;
  if (nsplit > 1 &&
      hipMallocAsync((void**)&parts, sizeof(float) * (size_t)total * nsplit, s->stream) !=
          hipSuccess) {
    (void)hipGetLastError();
    return SK_ENOMEM;
  }
  float* dst = nsplit > 1 ? parts : s->state;
  const long long sstride = nsplit > 1 ? total : 0;
  const int acc = nsplit > 1 ? 0 : 1;
  hipError_t err = hipSuccess;
  timing_mark(s, 0, false);
  hipLaunchKernelGGL(sk_update_kernel, dim3((unsigned)((long long)ntiles * nsplit * s->h)),
                     dim3(SK_WG), lds, s->stream, K, V, (long long)n, s->d, s->dv, s->logd,
                     s->d_utiles, ntiles, kps, nsplit, s->h, dst, s->XS, sstride, acc);
  err = hipGetLastError();
  timing_mark(s, 0, true);
  if (nsplit > 1) {
    const long long c4 = total / 4;
    const int grid = (int)std::min<long long>((c4 + 255) / 256, 16384);
    hipLaunchKernelGGL(sk_split_reduce_kernel, dim3(grid), dim3(256), 0, s->stream,
                       reinterpret_cast<float4*>(s->state),
                       reinterpret_cast<const float4*>(parts), c4, nsplit, c4);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) err = e;
    (void)hipFreeAsync(parts, s->stream);
  }
  if (err != hipSuccess) return SK_EHIP;
  s->count += n;
  return SK_OK;
}

int sketch_merge(sk_handle dst, sk_handle src) {
  if (dst == nullptr || src == nullptr || dst == src) return SK_EINVAL;
  if (dst->d != src->d || dst->dv != src->dv || dst->p != src->p || dst->h != src->h)
    return SK_EMISMATCH;
  const long long c4 = dst->XS * dst->h / 4;
  const int grid = (int)std::min<long long>((c4 + 255) / 256, 16384);
  hipLaunchKernelGGL(sk_add_kernel, dim3(grid), dim3(256), 0, dst->stream,
                     reinterpret_cast<float4*>(dst->state),
                     reinterpret_cast<const float4*>(src->state), c4);
  SK_TRY(hipGetLastError());
  dst->count += src->count;
  return SK_OK;
}

int sketch_query(sk_handle s, const float* Q, int64_t m, float* out, float* Z) {
  if (s == nullptr || m < 0) return SK_EINVAL;
  if (m == 0) return SK_OK;
  if (Q == nullptr || out == nullptr || Z == nullptr || !aligned16(Q)) return SK_EINVAL;
  const int ntiles = (int)s->qtiles.size();
  const long long nqt = (m + SK_TMQ - 1) / SK_TMQ;
  if (nqt * std::max<long long>(ntiles, SK_TMQ) * s->h > 0x7fffffffLL) return SK_EINVAL;
  const size_t pbytes = sizeof(float) * (size_t)s->h * nqt * s->qpb;
  float* parts = nullptr;
  if (hipMallocAsync((void**)&parts, pbytes, s->stream) != hipSuccess) {
    (void)hipGetLastError();
    return SK_ENOMEM;
  }
  timing_mark(s, 1, false);
  hipLaunchKernelGGL(query_kernel_for(s->logd), dim3((unsigned)(ntiles * nqt * s->h)),
                     dim3(SK_WG), query_lds_bytes(s->d), s->stream, Q, (long long)m,
                     s->state, s->XS, s->d_qtiles, ntiles, (int)nqt, s->qpb, parts);
  hipError_t e1 = hipGetLastError();
  timing_mark(s, 1, true);
  // queries per finishing workgroup: a power of two with qg * (d + dv) <= 256
  int qg = 1;
  while (qg < SK_TMQ && 2 * qg * (s->d + s->dv) <= 256) qg *= 2;
  hipLaunchKernelGGL(sk_query_finish, dim3((unsigned)(nqt * (SK_TMQ / qg) * s->h)),
                     dim3(256), 0, s->stream,
                     parts, s->d_qtiles, ntiles, (int)nqt, s->qpb, (long long)m, s->d,
                     s->dv, qg, (float)s->count, out, Z);
  hipError_t e2 = hipGetLastError();
  (void)hipFreeAsync(parts, s->stream);
  if (e1 != hipSuccess || e2 != hipSuccess) return SK_EHIP;
  return SK_OK;
}

int sketch_timing(sk_handle s, int enable) {
  if (s == nullptr) return SK_EINVAL;
  if (enable && s->tev[0][0].empty()) {
    for (int k = 0; k < 2; ++k)
      for (int w = 0; w < 2; ++w) {
        s->tev[k][w].resize(kTimingPairs);
        for (int i = 0; i < kTimingPairs; ++i) SK_TRY(hipEventCreate(&s->tev[k][w][i]));
      }
  }
  s->timing = enable != 0;
  s->trec[0] = s->trec[1] = 0;
  return SK_OK;
}

int sketch_kernel_times(sk_handle s, int kind, float* ms, int cap, int* count) {
  if (s == nullptr || kind < 0 || kind > 1 || cap < 0 || (ms == nullptr && cap > 0))
    return SK_EINVAL;
  const int nrec = s->trec[kind];
  if (count) *count = nrec;
  if (nrec > 0) {
    SK_TRY(hipEventSynchronize(s->tev[kind][1][nrec - 1]));
    for (int i = 0; i < nrec && i < cap; ++i)
      SK_TRY(hipEventElapsedTime(&ms[i], s->tev[kind][0][i], s->tev[kind][1][i]));
  }
  s->trec[kind] = 0;
  return SK_OK;
}

int sketch_export(sk_handle s, float* dst) {
  if (s == nullptr || dst == nullptr || !aligned16(dst)) return SK_EINVAL;
  const long long total = s->D * (1 + s->dv) * s->h;
  LevelTable lt{};
  lt.p = s->p;
  long long start = 0;
  for (int j = 0; j <= s->p; ++j) {
    lt.row_start[j] = start;
    lt.xoff[j] = s->xoff[j];
    lt.C[j] = s->C[j];
    start += s->rows[j];
  }
  if (s->p + 1 < SK_MAXLEV) lt.row_start[s->p + 1] = start;
  const int grid = (int)std::min<long long>((total + 255) / 256, 16384);
  hipLaunchKernelGGL(sk_export_kernel, dim3(grid), dim3(256), 0, s->stream, s->state,
                     s->XS, lt, s->D, s->d, s->logd, s->dv, (float)s->count, dst, total);
  SK_TRY(hipGetLastError());
  return SK_OK;
}

int sketch_state(sk_handle s, const float** dev_state, int64_t* rows_D, int* cols,
                 int64_t* count) {
  if (s == nullptr) return SK_EINVAL;
  const size_t bytes = sizeof(float) * (size_t)(s->D * (1 + s->dv) * s->h);
  if (s->view_bytes < bytes) {
    SK_TRY(hipStreamSynchronize(s->stream));
    (void)hipFree(s->view);
    s->view = nullptr;
    s->view_bytes = 0;
    if (hipMalloc(&s->view, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return SK_ENOMEM;
    }
    s->view_bytes = bytes;
  }
  const int rc = sketch_export(s, s->view);
  if (rc != SK_OK) return rc;
  SK_TRY(hipStreamSynchronize(s->stream));
  if (dev_state) *dev_state = s->view;
  if (rows_D) *rows_D = s->D;
  if (cols) *cols = 1 + s->dv;
  if (count) *count = s->count;
  return SK_OK;
}

int exact_attend(const float* K, const float* V, int64_t n, int d, int dv, int h,
                 const float* Q, int64_t m, float* out, float* Z, void* hip_stream) {
  if (!is_pow2_in(d, 4, 128) || !is_pow2_in(dv, 4, 128) || h < 1 || n < 0 || m < 0)
    return SK_EINVAL;
  if (m == 0) return SK_OK;
  if (Q == nullptr || out == nullptr || Z == nullptr || !aligned16(Q)) return SK_EINVAL;
  if (n > 0 && (K == nullptr || V == nullptr || !aligned16(K) || !aligned16(V)))
    return SK_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  int dev = 0;
  DeviceInfo di;
  int rc = current_device(&dev);
  if (rc == SK_OK) rc = device_info(dev, &di);
  if (rc != SK_OK) return rc;
  const int bmax = std::max(d, dv);
  const bool decode = m <= 8;
  const long long nqt = decode ? 1 : (m + 255) / 256;
  // EXPSKETCH_EXACT_MINKEYS=<k> sets the fewest keys per slice (tuning aid).
  static const long long min_keys_env = [] {
    const char* v = std::getenv("EXPSKETCH_EXACT_MINKEYS");
    return v ? std::max(0LL, std::atoll(v)) : 0LL;
  }();
  // Decode streams K/V once: about two long (>= 4096-key) slices per CU keep HBM
  // busiest, but never fewer slices than one per CU while slices stay >= 512
  // keys.  The batched kernel is compute-bound: more, shorter slices.
  const long long hq = h * nqt;
  long long ns;
  if (decode) {
    const long long lk = min_keys_env > 0 ? min_keys_env : 4096;
    const long long nn = n;
    const long long ns_long = std::min((2LL * di.num_cu + hq - 1) / hq, (nn + lk - 1) / lk);
    const long long ns_fill = std::min(((long long)di.num_cu + hq - 1) / hq, (nn + 511) / 512);
    ns = std::max(ns_long, ns_fill);
  } else {
    const long long lk = min_keys_env > 0 ? min_keys_env : 512;
    ns = std::min((8LL * di.num_cu + hq - 1) / hq, ((long long)n + lk - 1) / lk);
  }
  ns = std::max(1LL, ns);
  long long kps = n > 0 ? (n + ns - 1) / ns : 0;
  kps = (kps + 31) / 32 * 32;
  const int nsplit = kps > 0 ? (int)((n + kps - 1) / kps) : 1;
  const size_t pbytes = sizeof(float) * (size_t)h * m * nsplit * (2 + dv);
  float* parts = nullptr;
  if (hipMallocAsync((void**)&parts, pbytes, st) != hipSuccess) {
    (void)hipGetLastError();
    return SK_ENOMEM;
  }
  const long long nn = n;
  const long long mm = m;
  if (decode) {
    const int mq = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8;
    dim3 grid(nsplit, h), blk(256);
#define SK_DEC(BB, MQ)                                                              \
  hipLaunchKernelGGL((sk_exact_decode<BB, MQ>), grid, blk, 0, st, K, V, nn, d, dv, Q, \
                     mm, kps, nsplit, parts)
#define SK_DEC_B(BB)              \
  switch (mq) {                   \
    case 1: SK_DEC(BB, 1); break; \
    case 2: SK_DEC(BB, 2); break; \
    case 4: SK_DEC(BB, 4); break; \
    default: SK_DEC(BB, 8); break; \
  }
    switch (bmax) {
      case 4: SK_DEC_B(4); break;
      case 8: SK_DEC_B(8); break;
      case 16: SK_DEC_B(16); break;
      case 32: SK_DEC_B(32); break;
      case 64: SK_DEC_B(64); break;
      default: SK_DEC_B(128); break;
    }
#undef SK_DEC_B
#undef SK_DEC
  } else {
    dim3 grid((unsigned)(nsplit * nqt), h), blk(256);
#define SK_TIL(BB, KS)                                                                 \
  hipLaunchKernelGGL((sk_exact_tiled<BB, KS>), grid, blk, 0, st, K, V, nn, d, dv, Q, mm, \
                     kps, nsplit, parts)
    switch (bmax) {
      case 4: SK_TIL(4, 32); break;
      case 8: SK_TIL(8, 32); break;
      case 16: SK_TIL(16, 32); break;
      case 32: SK_TIL(32, 32); break;
      case 64: SK_TIL(64, 32); break;
      default: SK_TIL(128, 16); break;
    }
#undef SK_TIL
  }
  hipError_t e1 = hipGetLastError();
  hipLaunchKernelGGL(sk_exact_combine, dim3((unsigned)(h * m)), dim3(256), 0, st, parts,
                     nsplit, mm, dv, h, out, Z);
  hipError_t e2 = hipGetLastError();
  (void)hipFreeAsync(parts, st);
  if (e1 != hipSuccess || e2 != hipSuccess) return SK_EHIP;
  return SK_OK;
}

}  // extern "C"
