// Host side of libexpsketch: argument checks, launch planning, state ownership.
// The C ABI is declared (with the passages each call follows) in expsketch.h.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <numeric>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "expsketch.h"
#include "sk_common.h"
#include "sk_elementwise.h"
#include "sk_exact.h"
#include "sk_query.h"
#include "sk_query_dg.h"
#include "sk_step.h"
#include "sk_sym.h"
#include "sk_sym_dg.h"
#include "sk_update.h"
#include "sk_update_kr.h"

// the digit kernel's instantiations live in their own objects (sk_update_kr.hip)
#define KR_EXTERN(RT, CENTER)                                                                  \
  extern template __global__ void sk_update_kr_kernel<RT, CENTER>(                             \
      const float*, const float*, long long, long long, int, const KrUnit*, KrSplits, int,     \
      float*, long long, long long, int, const float*, PendingReduce);
KR_EXTERN(1, false)
KR_EXTERN(1, true)
KR_EXTERN(2, false)
KR_EXTERN(2, true)
KR_EXTERN(4, false)
KR_EXTERN(4, true)
#undef KR_EXTERN

// Scratch of the allocation-free exact path (exact_attend_noalloc): one array per
// device (each GPU the library runs on holds its own copy until the process
// ends).  Host code never uses the array's name as an address: its device
// address is taken once per device with hipGetSymbolAddress (scratch_on_device).
constexpr long long kScratchFloats = 4LL << 20;   // 16 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

#define SK_TRY(expr)                               \
  do {                                             \
    if ((expr) != hipSuccess) return SK_EHIP;      \
  } while (0)

// A kernel launch that, when given timing events, has the launch itself record
// them (hipExtLaunchKernel: the start event takes the kernel's start time, the
// stop event its end), so that a timed pair brackets exactly the kernels of a
// region and not the queue around them.  Without events: a plain launch.
template <typename F, typename... Args>
void launch_ev(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, hipEvent_t ev0,
               hipEvent_t ev1, Args... args) {
  if (ev0 == nullptr && ev1 == nullptr)
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  else
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)lds, st, ev0, ev1, 0u, args...);
}

constexpr int kMaxP = 16;
// a_hi rows per query tile: the full layout keeps plans of 512, 256 and 128 rows
// and a query takes the longest whose launch fills the GPU (query_plan_for);
// EXPSKETCH_QUERY_ROWS fixes one length instead (a multiple of 64 up to 4096, so a
// tile's rows stay within a 32-bit buffer range; tuning aid)
long long query_rows_fixed() {
  static const long long v = [] {
    const char* e = std::getenv("EXPSKETCH_QUERY_ROWS");
    const long long r = e ? std::min(std::atoll(e), 4096LL) : 0;
    return r >= 64 ? r / 64 * 64 : 0LL;
  }();
  return v;
}

// a level's query split keeps the fewest trailing digits whose columns (d^t C)
// reach this count (EXPSKETCH_QUERY_MINCOLS overrides, tuning aid)
long long query_min_cols() {
  static const long long v = [] {
    const char* e = std::getenv("EXPSKETCH_QUERY_MINCOLS");
    const long long r = e ? std::atoll(e) : 0;
    return r >= 1 ? r : (long long)SK_TNQ;
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
  return sizeof(float) * ((size_t)(SK_KB + 1) * (d + dv) + (size_t)SK_KB * 384 + d);
}
size_t query_lds_bytes(int d) {
  // Qs + max(At + Bt, Ys)
  const size_t ab = (size_t)SK_KB * (SK_TMQ + SK_PAD) + (size_t)SK_KB * (SK_TNQ + SK_PAD);
  const size_t ys = (size_t)64 * (SK_TNQ + 1);
  return sizeof(float) * ((size_t)d * (SK_TMQ + 1) + std::max(ab, ys));
}

size_t sym_update_lds_bytes(int d, int dv) {
  // Ks (+ ones and zeros rows) + Vs, prefix products
  return sizeof(float) * ((size_t)(d + 2 + dv) * SY_LDK + (size_t)SY_KB * SY_LDP + d);
}
size_t sym_query_lds_bytes(int d) {
  // Qs + At + Bt (widest column tile, 128 columns: row stride 144) + row codes
  return sizeof(float) * ((size_t)d * (SY_TQ + 4) + (size_t)SY_QKB * (SY_TQ + 16) +
                          (size_t)SY_QKB * 144) +
         sizeof(unsigned long long) * SY_QKB;
}
// row blocks of 16 per wave of the multiset update: 1, 2 or 4, tiles of 64 * rb
// rows (EXPSKETCH_SYM_RB overrides the default 4; tuning aid)
int sym_update_rb() {
  static const int v = [] {
    const char* e = std::getenv("EXPSKETCH_SYM_RB");
    const int r = e ? std::atoi(e) : 4;
    return (r == 1 || r == 2 || r == 4) ? r : 4;
  }();
  return v;
}
// state rows per range of the multiset query (EXPSKETCH_SYM_QUERY_ROWS overrides)
int sym_query_rows() {
  static const int v = [] {
    const char* e = std::getenv("EXPSKETCH_SYM_QUERY_ROWS");
    const int r = e ? std::atoi(e) : 0;
    return r >= SY_QKB ? r / SY_QKB * SY_QKB : 128;
  }();
  return v;
}

// The full-layout update kernel is instantiated per centring and per prefetch
// depth (float4 of K and of V per thread per 32-key stage: 1 up to d, dv = 32,
// 2 for 64, 4 for 128), so narrow keys do not hold registers for wide ones.
using UpdateKernel = void (*)(const float*, const float*, long long, long long, int, int, int,
                              const UpdTile*, int, long long, int, int, float*, long long,
                              long long, int, const float*, PendingReduce);
using UpdateKrKernel = void (*)(const float*, const float*, long long, long long, int,
                                const KrUnit*, KrSplits, int, float*, long long,
                                long long, int, const float*, PendingReduce);
UpdateKernel update_kernel_for(bool center, int d, int dv) {
  const int w = std::max(d, dv);
  if (w <= 32) return center ? sk_update_kernel<true, 1> : sk_update_kernel<false, 1>;
  if (w <= 64) return center ? sk_update_kernel<true, 2> : sk_update_kernel<false, 2>;
  return center ? sk_update_kernel<true, 4> : sk_update_kernel<false, 4>;
}

// The digit-organised update kernel (sk_update_kr.h) per key width d = 16 RT.
// It runs for d = 16, 32 and 64, where it is the faster of the two full-layout
// kernels; the other widths run the tile kernel.
UpdateKrKernel update_kr_kernel_for(bool center, int d) {
  if (d == 16) return center ? sk_update_kr_kernel<1, true> : sk_update_kr_kernel<1, false>;
  if (d == 32) return center ? sk_update_kr_kernel<2, true> : sk_update_kr_kernel<2, false>;
  return center ? sk_update_kr_kernel<4, true> : sk_update_kr_kernel<4, false>;
}
// key widths that run the digit kernel
bool kr_width(int d) { return d == 16 || d == 32 || d == 64; }
// EXPSKETCH_EXACT_MFMA16=0 keeps the 32x32 batched exact kernel at dv = 16.
bool use_exact_mfma16() {
  static const bool v = [] {
    const char* e = std::getenv("EXPSKETCH_EXACT_MFMA16");
    return e == nullptr || std::atoi(e) != 0;
  }();
  return v;
}
// EXPSKETCH_UPDATE_KR=0 keeps the tile kernels for every key width.
bool use_update_kr() {
  static const bool v = [] {
    const char* e = std::getenv("EXPSKETCH_UPDATE_KR");
    return e == nullptr || std::atoi(e) != 0;
  }();
  return v;
}

// The multiset update kernel is instantiated per tile shape (rb, cb).
using SymUpdateKernel = void (*)(const float*, const float*, long long, long long, int, int,
                                 const SymUpdTile*, int, SymTables, long long, int, int,
                                 float*, long long, long long, int, const float*,
                                 PendingReduce);
SymUpdateKernel sym_update_kernel_for(int rb, int cb, bool center) {
#define SY_PICK(RB_, CB_) \
  return center ? sk_sym_update_kernel<RB_, CB_, true> : sk_sym_update_kernel<RB_, CB_, false>
  switch (rb * 8 + cb) {
    case 4 * 8 + 1: SY_PICK(4, 1);
    case 4 * 8 + 2: SY_PICK(4, 2);
    case 4 * 8 + 4: SY_PICK(4, 4);
    case 2 * 8 + 1: SY_PICK(2, 1);
    case 2 * 8 + 2: SY_PICK(2, 2);
    case 2 * 8 + 4: SY_PICK(2, 4);
    case 1 * 8 + 4: SY_PICK(1, 4);
    default: return nullptr;
  }
#undef SY_PICK
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

// Query kernels by the last digit (sk_query_dg.h), per log2(d) and 32-column tiles.
using QueryDgKernel = QueryKernel;
// d <= 64: the register-query kernel; d = 128: the LDS-query kernel
QueryDgKernel query_dg_kernel_for(int logd) {
  switch (logd) {
    case 2: return sk_query_dgr_kernel<2>;
    case 3: return sk_query_dgr_kernel<3>;
    case 4: return sk_query_dgr_kernel<4>;
    case 5: return sk_query_dgr_kernel<5>;
    case 6: return sk_query_dgr_kernel<6>;
    default: return sk_query_dg_kernel<7>;
  }
}
QueryDgKernel query_dg16_kernel_for(int logd) {
  switch (logd) {
    case 2: return sk_query_dg16_kernel<2>;
    case 3: return sk_query_dg16_kernel<3>;
    default: return sk_query_dg16_kernel<4>;
  }
}
size_t query_dg_lds_bytes(int d) {
  const size_t ldb = 32 * SK_DGNT + 32;
  if (d <= 64) return sizeof(float) * 2 * (size_t)(d >= 8 ? 64 : SK_DGK) * ldb;
  return sizeof(float) * ((size_t)d * (SK_DGQ + 33) + 2 * (size_t)SK_DGK * ldb);
}
size_t query_dg16_lds_bytes(int d) {
  return sizeof(float) * ((size_t)d * (SK_DGQ + 1) + 2 * (size_t)SK_DGK * (16 + 4));
}
// EXPSKETCH_QUERY_DG16=1 puts levels of 8 < C <= 16 columns on the 16-column
// last-digit kernel (tuning aid).
bool use_query_dg16() {
  static const bool v = [] {
    const char* e = std::getenv("EXPSKETCH_QUERY_DG16");
    return e != nullptr && std::atoi(e) != 0;
  }();
  return v;
}
// EXPSKETCH_QUERY_DG=0 keeps every level on the feature-tile query kernel.
bool use_query_dg() {
  static const bool v = [] {
    const char* e = std::getenv("EXPSKETCH_QUERY_DG");
    return e == nullptr || std::atoi(e) != 0;
  }();
  return v;
}

// Per-call partials (query, exact path).  A hipMallocAsync that follows a
// hipFreeAsync on the same stream makes the host wait here until that stream has
// drained (measured: back-to-back calls then return only as each previous call's
// kernels finish), so the partials live in a buffer kept across calls.  Every
// use of a kept buffer is on one stream (the handle's stream, which waits for
// the previous one on a change; or the stream an exact-path buffer belongs to),
// so stream order alone serialises its users: no event is recorded or waited
// for per call (each would add a barrier packet between the kernels).  Requests
// above kKeepBytes take a stream-ordered allocation of their own (their kernels
// run longer than that wait).
constexpr size_t kKeepBytes = size_t(256) << 20;

struct Workspace {
  float* ptr = nullptr;
  size_t cap = 0;                          // bytes
};

// Points *out at `bytes` of device memory for one call on stream st, the stream
// of every earlier use of ws: the kept buffer (grown, once the stream has
// finished the work that used it, when too small) or, beyond kKeepBytes, its own
// stream-ordered allocation (*own = true).
int take_workspace(Workspace* ws, size_t bytes, hipStream_t st, float** out, bool* own) {
  *out = nullptr;
  *own = false;
  if (bytes > kKeepBytes) {
    if (hipMallocAsync((void**)out, bytes, st) != hipSuccess) {
      (void)hipGetLastError();
      return SK_ENOMEM;
    }
    *own = true;
    return SK_OK;
  }
  if (bytes > ws->cap) {
    SK_TRY(hipStreamSynchronize(st));
    (void)hipFree(ws->ptr);
    ws->ptr = nullptr;
    ws->cap = 0;
    const size_t cap = std::min(kKeepBytes, std::max(bytes, size_t(1) << 20));
    if (hipMalloc((void**)&ws->ptr, cap) != hipSuccess) {
      (void)hipGetLastError();
      return SK_ENOMEM;
    }
    ws->cap = cap;
  }
  *out = ws->ptr;
  return SK_OK;
}

// Ends the call's use of what take_workspace gave it (work already enqueued).
void release_workspace(float* p, bool own, hipStream_t st) {
  if (own) (void)hipFreeAsync(p, st);
}

// Frees the kept buffer; no work that uses it may be in flight.
void free_workspace(Workspace* ws) {
  (void)hipFree(ws->ptr);
  *ws = Workspace{};
}

// exact_attend's kept partials, per (device, stream): at most kMaxXws buffers;
// a new (device, stream) pair beyond that takes the place of the one used least
// recently, after the device has finished all its work.  (A stream's handle
// names one live stream object for as long as work queued on it runs: the
// runtime keeps a destroyed stream's object until that work is done, so a new
// stream cannot take the handle of one whose kernels still use the buffer.)
constexpr size_t kMaxXws = 8;
struct XwsEntry {
  Workspace ws;
  unsigned long long last_use = 0;
};
std::mutex g_xws_mutex;
std::map<std::pair<int, void*>, XwsEntry> g_xws;
unsigned long long g_xws_clock = 0;

// Kernel timing of the exact path (exact_timing): pairs of events around the
// slice kernel of each exact_attend call, up to kTimingPairsX; guarded by
// g_xws_mutex.
constexpr int kTimingPairsX = 256;
bool g_xtiming = false;
std::vector<hipEvent_t> g_xev[2];
int g_xrec = 0;

// The kept partials of (dev, stream); the caller holds g_xws_mutex.
int xws_for(int dev, hipStream_t stream, XwsEntry** out) {
  const auto key = std::make_pair(dev, reinterpret_cast<void*>(stream));
  auto it = g_xws.find(key);
  if (it == g_xws.end()) {
    if (g_xws.size() >= kMaxXws) {
      auto old = g_xws.begin();
      for (auto i = g_xws.begin(); i != g_xws.end(); ++i)
        if (i->second.last_use < old->second.last_use) old = i;
      int cur = 0;
      (void)hipGetDevice(&cur);
      if (old->first.first != cur) (void)hipSetDevice(old->first.first);
      (void)hipDeviceSynchronize();             // its stream may be gone: all work
      free_workspace(&old->second.ws);
      if (old->first.first != cur) (void)hipSetDevice(cur);
      g_xws.erase(old);
    }
    it = g_xws.emplace(key, XwsEntry{}).first;
  }
  it->second.last_use = ++g_xws_clock;
  *out = &it->second;
  return SK_OK;
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
  UpdTile* d_utiles = nullptr;
  std::vector<KrUnit> kunits;      // digit-organised update units (d >= 16)
  std::vector<int> kgroup0;        // their groups (first unit of each, then the count)
  std::vector<int> kweight;        // work per key of each group's units
  KrUnit* d_kunits = nullptr;
  // query plans: the full layout one per row length of its tiles (longest
  // first), the multiset layout one (its tiles are sqtiles; the plan holds the
  // finishing records)
  struct QGroup { int kind, nt, off, count; };
  struct QPlan {
    long long rows = 0;                    // a_hi rows per tile
    std::vector<QryTile> tiles;            // in level order
    std::vector<int> kind;                 // per tile: kind * 16
    // launches of the full layout: tiles grouped by kernel (0: feature tiles,
    // 1: by the last digit, 2: by the last digit, 16 columns); each group's
    // tiles are contiguous in run
    std::vector<QryTile> run;
    std::vector<QGroup> groups;
    long long pb = 0;                      // floats of partials per (head, query tile)
    QryTile* d_run = nullptr;
    FinTile* d_fin = nullptr;              // finishing records, one per tile
  };
  std::vector<QPlan> qplans;
  float* view = nullptr;    // canonical view buffer
  bool timing = false;      // kernel timing (sketch_timing)
  std::vector<hipEvent_t> tev[3][2];   // [kind][start, stop], created on first use
  int trec[3] = {0, 0, 0};  // pairs recorded per kind
  size_t view_bytes = 0;
  DeviceInfo dev;
  // multiset layout (SK_LAYOUT_SYM)
  int layout = SK_LAYOUT_FULL;
  long long Dsym = 0, Rlo = 0, Rtop = 0;   // canonical rows; lower and top block rows
  void* symbuf = nullptr;                  // device tables (one allocation)
  SymTables tb{};
  std::vector<SymUpdTile> sutiles;         // grouped by tile shape
  std::vector<int> sgroup;                 // first tile of each shape group, + end
  std::vector<SymQryTile> sqtiles;
  SymUpdTile* d_sutiles = nullptr;
  SymQryTile* d_sqtiles = nullptr;
  // multiset blocks queried by the last index (sk_sym_dg.h): tiles and runs
  std::vector<SymDgTile> sdtiles;
  std::vector<SymDgRun> sdruns;
  SymDgTile* d_sdtiles = nullptr;
  SymDgRun* d_sdruns = nullptr;
  // decode steps (sketch_step): row-range tiles of the whole state, partials
  std::vector<StepTile> stiles;
  StepTile* d_stiles = nullptr;
  float* sparts = nullptr;                 // [h][tiles][1 + dv]
  // fixed centre (sketch_set_center): moments are of k - c; null = no centre
  float* center = nullptr;                 // device [h][d]
  std::vector<float> center_host;          // the same values, for merge checks
  // split partials of update calls: two buffers used in turn; the last call's
  // partials are added into the state by the next update launch (or by a
  // reduce kernel before anything else reads or writes the state)
  float* pbuf[2] = {nullptr, nullptr};
  size_t pbuf_floats = 0;                  // capacity of each buffer
  int pcur = 0;                            // buffer the next call writes
  float* pend = nullptr;                   // partials not yet in the state
  int pend_ns = 0;
  hipEvent_t flush_ev = nullptr;           // orders the two streams around a merge
  hipEvent_t switch_ev = nullptr;          // orders a stream change (sketch_set_stream)
  // staging of small update calls: their keys and values are copied here and
  // contracted in one launch when the buffer fills or the state is needed
  float* stage_k = nullptr;                // [h][stage_cap][d]
  float* stage_v = nullptr;                // [h][stage_cap][dv]
  long long stage_cap = -1;                // keys per head; 0 = off, -1 = default
  long long stage_n = 0;                   // keys per head staged
  Workspace qws;                           // query partials, kept across calls
};

namespace {

constexpr int kTimingPairs = 256;

// The current timed pair of `kind` (both null when not timing or when the pairs
// are used up): its start event goes to the first kernel launch of the timed
// region and its stop event to the last (launch_ev); timing_done moves on to the
// next pair.
void timing_pair(sk_sketch* s, int kind, hipEvent_t* ev0, hipEvent_t* ev1) {
  *ev0 = *ev1 = nullptr;
  if (!s->timing || s->trec[kind] >= (int)s->tev[kind][0].size()) return;
  *ev0 = s->tev[kind][0][s->trec[kind]];
  *ev1 = s->tev[kind][1][s->trec[kind]];
}
void timing_done(sk_sketch* s, int kind) {
  if (s->timing && s->trec[kind] < (int)s->tev[kind][0].size()) ++s->trec[kind];
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

// Units of the digit-organised update (key widths d >= 16), see sk_update_kr.h:
// levels 0 and 1 per 16-column tile; level 2 per (16-chunk of c, 8 b1 digits,
// 64 columns); levels >= 3 per (leading digits F, 4 b2 digits and 8 b1 digits,
// 16-chunk of c) when the row width is at most 16, else per (F, 2 b2 digits, 8 b1
// digits, 16-chunk of c, 32 columns).  Returns false (no units: the tile kernels
// run instead) past KR_MAXF leading digits or when the count would not fit.
bool plan_kr_units(sk_sketch* s) {
  const int d = s->d, RT = d / 16;
  std::vector<KrUnit> u;
  auto add = [&](int j, int mode, long long F, int b2, int b1, int rc, int ct) {
    u.push_back(KrUnit{s->xoff[j], j, s->C[j], j == s->p ? 1 : 0, mode, (int)F, b2, b1, rc, ct, 0});
  };
  for (int j = 0; j <= s->p; ++j) {
    const int C = s->C[j];
    double count = 0.0;
    if (j <= 1) {
      count = (C + 15) / 16;
    } else if (j == 2) {
      count = (double)RT * (d / 8) * ((C + 63) / 64);
    } else {
      if (j - 3 > KR_MAXF) return false;
      const double nF = std::pow((double)d, j - 3);
      count = C <= 16 ? nF * (d / 4) * (d / 8) * RT : nF * (d / 2) * (d / 8) * RT * ((C + 31) / 32);
    }
    if (count + (double)u.size() > (double)(1 << 26)) return false;
    if (j <= 1) {
      for (int ct = 0; ct < (C + 15) / 16; ++ct) add(j, KR_SMALL, 0, 0, 0, 0, ct);
    } else if (j == 2) {
      for (int rc = 0; rc < RT; ++rc)
        for (int b1 = 0; b1 < d; b1 += 8)
          for (int cg = 0; cg < (C + 63) / 64; ++cg) add(j, KR_WIDE, 0, 0, b1, rc, cg);
    } else {
      const long long nF = (long long)std::llround(std::pow((double)d, j - 3));
      for (long long F = 0; F < nF; ++F) {
        if (C <= 16) {
          for (int b2 = 0; b2 < d; b2 += 4)
            for (int b1 = 0; b1 < d; b1 += 8)
              for (int rc = 0; rc < RT; ++rc) add(j, KR_PAIR, F, b2, b1, rc, 0);
        } else {
          for (int b2 = 0; b2 < d; b2 += 2)
            for (int b1 = 0; b1 < d; b1 += 8)
              for (int rc = 0; rc < RT; ++rc)
                for (int ct = 0; ct < (C + 31) / 32; ++ct) add(j, KR_SINGLE, F, b2, b1, rc, ct);
        }
      }
    }
  }
  // groups by work per key (matrix instructions per key, in 32x32x2 units): the
  // 8-block units 4, a 4-block level-2 unit 2, the level 0/1 units 1 (few matrix
  // instructions, but each 4-key step waits on its loads); groups sorted
  // heaviest first, so a unit's position no longer follows its level (the
  // kernel takes a head's items in the reverse order, lightest group first)
  auto weight = [&](const KrUnit& x) {
    if (x.mode == KR_SMALL) return 1;
    if (x.mode == KR_WIDE) return x.C - 64 * x.ct > 32 ? 4 : 2;
    return 4;
  };
  std::stable_sort(u.begin(), u.end(),
                   [&](const KrUnit& a, const KrUnit& b) { return weight(a) > weight(b); });
  s->kgroup0.clear();
  s->kweight.clear();
  for (size_t i = 0; i < u.size(); ++i)
    if (i == 0 || weight(u[i]) != weight(u[i - 1])) {
      s->kgroup0.push_back((int)i);
      s->kweight.push_back(weight(u[i]));
    }
  s->kgroup0.push_back((int)u.size());
  if (s->kweight.size() > KR_MAXG) return false;
  s->kunits.swap(u);
  return true;
}

// EXPSKETCH_QUERY_FOLD=0 keeps levels of 8 or 16 columns off the last-digit
// kernel (tuning aid).
bool use_query_fold() {
  static const bool v = [] {
    const char* e = std::getenv("EXPSKETCH_QUERY_FOLD");
    return e == nullptr || std::atoi(e) != 0;
  }();
  return v;
}
// Level j runs on the register-query kernel with its last digit on the column
// side: C of 8, 16 or 32 (dividing the 32 columns of an MFMA tile, so that a
// 64-column tile is full) and 16 <= d <= 64; for C = 32, which unfolded already
// fills one MFMA tile, only from j = 2 on (at least d rows left).  (At d = 8
// the feature-tile kernel measured faster: 0.50 against 0.48 of peak on the
// d = 8, p = 6 workload.)
bool query_level_fold(const sk_sketch* s, int j) {
  const int C = s->C[j];
  return use_query_fold() && (C == 8 || C == 16 || (C == 32 && j >= 2)) && s->d >= 16 &&
         s->d <= 64 && j >= 1;
}

// Query tiles of level j: t trailing digits in the columns (the fewest giving at
// least SK_TNQ columns), 128-column tiles, a_hi ranges of the plan's rows.
// Kernel of level j's query: by the last digit when its C columns fill MFMA
// columns (32x32x2 for C > 16, in 64-column tiles), or with the last digit on
// the column side for C = 8, 16 or 32 (query_level_fold); 16x16x4 for other
// 8 < C <= 16 at d <= 16 when asked for; else the feature-tile kernel.  Returns
// kind * 16.
int query_level_kind(const sk_sketch* s, int j) {
  const int C = s->C[j];
  if (!use_query_dg()) return 0;
  if (C > 16 || query_level_fold(s, j)) return 16;
  // (other 8 < C <= 16 stay on the feature-tile kernel: its folded 128-column
  // tiles measured faster than sk_query_dg16_kernel at d = 16 and d = 8)
  if (C > 8 && C <= 16 && s->d <= 16 && use_query_dg16()) return 32;
  return 0;
}

// MFMA work of a last-digit query tile, in row-steps of 32 columns: its rows
// times its 32-column GEMM tiles (one or two)
long long query_tile_work(const QryTile& T) {
  const long long gw = T.t ? (long long)T.nalo * T.C : T.fw;
  return (T.s == 0 ? 1 : T.a1 - T.a0) * ((gw + 31) / 32);
}

void plan_query_level(sk_sketch* s, int j, sk_sketch::QPlan* qp) {
  const int d = s->d, C = s->C[j];
  const int kind = query_level_kind(s, j);
  // t trailing digits go to the epilogue (folded with the weights q^(x)t): the
  // fewest whose d^t C columns fill a column tile.  A level whose own C columns
  // fill half a tile takes none: the half-empty tile, with its deeper rows and
  // half the partials, costs less than folding a digit (measured at C = 64 and
  // 128 against one folded digit; at C = 8 a half-filled tile cost more).
  int t = j;
  for (int tt = 0; tt <= j; ++tt) {
    const double cols = std::pow((double)d, tt) * C;
    if (cols >= query_min_cols() || (tt == 0 && 2 * C >= SK_TNQ)) { t = tt; break; }
  }
  // both sides of the split hold at most SK_MAXDIG digits: the kernel forms
  // q^(x)s from that many (p <= 16 keeps j - SK_MAXDIG <= t <= SK_MAXDIG feasible)
  while (t > SK_MAXDIG) --t;
  if (t < j - SK_MAXDIG) t = j - SK_MAXDIG;
  // by the last digit: every row on the row side, or one digit on the column side
  const bool fold = kind != 0 && query_level_fold(s, j);
  if (kind != 0) t = fold ? 1 : 0;
  const int sd = j - t;
  const long long N = (long long)std::llround(std::pow((double)d, t)) * C;
  const long long Kr = (long long)std::llround(std::pow((double)d, sd));
  double fj = 1.0;
  for (int i = 2; i <= j; ++i) fj *= i;
  // the last-digit kernel owns 64 columns a tile and writes a partial of those
  // columns only; the feature-tile kernel 128 GEMM columns folded into all C
  const long long tn = kind == 16 ? 32 * SK_DGNT : SK_TNQ;
  for (long long col0 = 0; col0 < N; col0 += tn) {
    const long long last = std::min(N, col0 + tn) - 1;
    for (long long a0 = 0; a0 < Kr; a0 += qp->rows) {
      QryTile q{};
      q.xoff = s->xoff[j];
      q.a0 = a0;
      q.a1 = std::min(Kr, a0 + qp->rows);
      q.pofs = qp->pb;
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
      q.fc0 = (kind == 16 && !fold) ? (int)col0 : 0;
      q.fw = (kind == 16 && !fold) ? (int)(last - col0 + 1) : C;
      qp->pb += (long long)SK_TMQ * q.fw;
      qp->tiles.push_back(q);
      qp->kind.push_back(kind);
    }
  }
}

// Multiset layout: canonical tables, update row tiles (with their prefix slots)
// and query row ranges.  Level j is generated from level j - 1 in order: for each
// multiset beta of size j - 1, beta + {e} for e from the largest index of beta
// (0 for the empty multiset) to d - 1.  That is lexicographic order of the sorted
// tuples, and it gives the prefix, the multiplicity of the largest index and
// 1/alpha! = (1/beta!) / (multiplicity of e in beta + 1) on the way.
struct SymHost {
  std::vector<unsigned long long> code;
  std::vector<int> prefix, last, lmul, rslot, slots;
  std::vector<float> winv;
};

void sym_tables(int d, int p, SymHost* t, long long* Rlo) {
  std::vector<double> wv;
  t->code.push_back(0ull);
  t->prefix.push_back(-1);
  t->last.push_back(d);
  t->lmul.push_back(0);
  wv.push_back(1.0);
  long long b0 = 0, b1 = 1;
  *Rlo = p > 0 ? 1 : 0;
  for (int j = 1; j <= p; ++j) {
    for (long long b = b0; b < b1; ++b) {
      const int lb = (j == 1) ? 0 : t->last[b];
      for (int e = lb; e < d; ++e) {
        const int mult = (j > 1 && e == t->last[b]) ? t->lmul[b] : 0;
        const unsigned long long base = t->code[b] & 0x00ffffffffffffffull;
        t->code.push_back(base | ((unsigned long long)e << (8 * (j - 1))) |
                          ((unsigned long long)j << 56));
        t->prefix.push_back((int)b);
        t->last.push_back(e);
        t->lmul.push_back(mult + 1);
        wv.push_back(wv[b] / (double)(mult + 1));
      }
    }
    b0 = b1;
    b1 = (long long)t->code.size();
    if (j < p) *Rlo = b1;
  }
  t->winv.assign(wv.begin(), wv.end());
  t->rslot.assign(t->code.size(), 0);
}

// Column blocks of 16 per wave of the multiset update.  One shape serves both
// blocks of a sketch (one launch per update call): the top block's width dv sets
// it, and the wider lower block (d + dv) takes more column tiles.
int sym_update_cb(int dv) { return dv <= 16 ? 1 : (dv <= 32 ? 2 : 4); }

// Update tiles of one block: row tiles of at most TM rows and SY_NS prefix slots
// (rows with one prefix are consecutive), each cut into column tiles.
void plan_sym_update_block(sk_sketch* s, SymHost* t, long long xoff, int rc0, int nrows,
                           int C, int top) {
  const int cb = sym_update_cb(s->dv);
  const int rb = sym_update_rb();
  const int TM = 64 * rb, TN = 16 * cb;   // TM <= SY_NS: a tile never runs out of slots
  int r = 0;
  while (r < nrows) {
    const int row0 = r, slot0 = (int)t->slots.size();
    int ns = 0, cnt = 0, lastpid = 0;
    while (r < nrows && cnt < TM) {
      const int cid = rc0 + r;
      const int pid = t->prefix[cid];
      if (ns == 0 || pid != lastpid) {
        if (ns == SY_NS) break;
        t->slots.push_back(pid);
        ++ns;
        lastpid = pid;
      }
      t->rslot[cid] = ns - 1;
      ++r;
      ++cnt;
    }
    for (int col0 = 0; col0 < C; col0 += TN) {
      SymUpdTile u{};
      u.xoff = xoff;
      u.rc0 = rc0;
      u.row0 = row0;
      u.nrows = cnt;
      u.col0 = col0;
      u.C = C;
      u.top = top;
      u.slot0 = slot0;
      u.nslots = ns;
      u.cb = cb;
      u.rb = (rb == 1 && cb != 4) ? 2 : rb;   // (1, 1) and (1, 2) are not instantiated
      s->sutiles.push_back(u);
    }
  }
}

// Query ranges of one block: one [SY_TQ][C] partial per range of sym_query_rows()
// rows, filled by the range's column tiles.
void plan_sym_query_block(sk_sketch* s, long long xoff, int rc0, int nrows, int C, int top) {
  sk_sketch::QPlan& qp = s->qplans[0];
  const int cb = C <= 16 ? 1 : (C <= 32 ? 2 : (C <= 64 ? 4 : 8));
  const int TN = 16 * cb;
  for (int r0 = 0; r0 < nrows; r0 += sym_query_rows()) {
    QryTile f{};
    f.pofs = qp.pb;
    f.C = C;
    f.top = top;
    f.fc0 = 0;
    f.fw = C;
    qp.tiles.push_back(f);
    for (int col0 = 0; col0 < C; col0 += TN) {
      SymQryTile q{};
      q.xoff = xoff;
      q.pofs = qp.pb;
      q.rc0 = rc0;
      q.row0 = r0;
      q.nrows = std::min(sym_query_rows(), nrows - r0);
      q.col0 = col0;
      q.C = C;
      q.top = top;
      q.cb = cb;
      s->sqtiles.push_back(q);
    }
    qp.pb += (long long)SY_TQ * C;
  }
}

// EXPSKETCH_SYM_DG=0 keeps every multiset block on the row-range query kernel
// (tuning aid).
bool use_sym_dg() {
  static const bool v = [] {
    const char* e = std::getenv("EXPSKETCH_SYM_DG");
    return e == nullptr || std::atoi(e) != 0;
  }();
  return v;
}

// The multiset block of width C whose largest multiset size is jhi runs on the
// last-index query kernel: C >= 64 columns (two full MFMA tiles per wave), d <= 64
// (the query components in registers) and sizes up to 2 (a prefix of at most one
// index; runs pair up into full slots).  Measured: the d = 64, p = 2 workload
// 0.157 (row ranges) -> 0.302 of the fp32 peak; with sizes up to 3 and one run
// per slot, the d = 32, p = 3 workload went 0.149 -> 0.100 with both its blocks
// on it (the top block's 32 columns and runs of about d / 3 rows give too few
// matrix instructions per stage), 0.105 with its lower block alone.
bool sym_dg_block(const sk_sketch* s, int C, int jhi) {
  return use_sym_dg() && C >= 64 && s->d <= 64 && jhi <= 2 && jhi <= sd_max_j(s->d);
}

using SymDgKernel = void (*)(const float*, long long, const float*, long long, const SymDgTile*,
                             int, const SymDgRun*, int, long long, float*);
SymDgKernel sym_dg_kernel_for(int logd) {
  switch (logd) {
    case 2: return sk_sym_dg_kernel<2>;
    case 3: return sk_sym_dg_kernel<3>;
    case 4: return sk_sym_dg_kernel<4>;
    case 5: return sk_sym_dg_kernel<5>;
    default: return sk_sym_dg_kernel<6>;
  }
}
size_t sym_dg_lds_bytes() { return sizeof(float) * 2 * SD_R * (32 * SK_DGNT + 32); }

// Last-index query tiles of the multiset sizes jlo .. jhi of one block (block row
// 0 = canonical row rc0, float offset xoff): per size, its runs (one per
// multiset of the size below) paired into slots, and tiles of up to 64 columns
// and about six full stages' work, each with a [128][fw] partial and a
// finishing record.
void plan_sym_dg_block(sk_sketch* s, const SymHost& t, long long xoff, long long rc0, int C,
                       int top, int jlo, int jhi) {
  sk_sketch::QPlan& qp = s->qplans[0];
  const int d = s->d;
  const int NF = SD_R / d;
  const SymDgRun none{0, d, 0, 0.f, 0ull};
  // canonical start of each size
  std::vector<long long> start(s->p + 2, (long long)t.code.size());
  for (long long r = (long long)t.code.size() - 1; r >= 0; --r)
    start[(int)(t.code[r] >> 56)] = r;
  for (int j = jlo; j <= jhi; ++j) {
    const long long cnt = start[j + 1] - start[j];
    const long long lxoff = xoff + (start[j] - rc0) * C;
    const int run0 = (int)s->sdruns.size() / 2;
    if (j == 0) {
      s->sdruns.push_back(SymDgRun{0, 0, 0, 1.f, 0ull});
      s->sdruns.push_back(none);
    } else {
      std::vector<SymDgRun> lv;
      long long lr = 0;      // level row of the run's first multiset
      for (long long b = start[j - 1]; b < start[j]; ++b) {
        const int lb = j == 1 ? 0 : t.last[b];
        SymDgRun R{};
        R.row0 = (int)(lr - lb);
        R.lb = lb;
        R.mlb = j == 1 ? 0 : t.lmul[b];
        R.winv = t.winv[b];
        R.code = t.code[b] & 0x00ffffffffffffffull;
        lv.push_back(R);
        lr += d - lb;
      }
      // slots: the longest run left with the shortest when the shorter one's
      // positions (pairwise reversed: up to its length - 1, or its length when
      // odd) stay below the longer one's first index rounded down to even, else alone
      auto fits = [&](const SymDgRun& a, const SymDgRun& b) {
        const int L = d - b.lb;
        return L - 1 + (L & 1) < (a.lb & ~1);
      };
      std::vector<int> ord(lv.size());
      std::iota(ord.begin(), ord.end(), 0);
      std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return lv[x].lb < lv[y].lb; });
      for (int lo = 0, hi = (int)ord.size() - 1; lo <= hi;) {
        s->sdruns.push_back(lv[ord[lo]]);
        if (lo < hi && fits(lv[ord[lo]], lv[ord[hi]])) {
          s->sdruns.push_back(lv[ord[hi]]);
          --hi;
        } else {
          s->sdruns.push_back(none);
        }
        ++lo;
      }
    }
    const int nrun = (int)s->sdruns.size() / 2 - run0;
    // tiles of about equal work: a stage costs the rows of its k-step groups
    // that hold rows of their slots (the kernel skips the others) plus 32 rows'
    // worth of fixed cost; a tile takes stages up to five full stages' cost.
    // Measured on the d = 64, p = 2 workload (fraction of the fp32 peak), with
    // paired runs: 5 stages and 32 rows 0.302, 5 and 64 0.300, 6 and 0/32/64
    // 0.28, 4 and 32 0.27, 7 and 32 0.26, 3 and 32 0.22, 2 and 32 0.22; with one
    // run per slot the best was 6 and 32 at 0.247 (of 8 and 64 0.218, 16 and 64
    // 0.139, equal counts of 8 runs 0.230).  EXPSKETCH_SYM_DG_STAGES and
    // EXPSKETCH_SYM_DG_OVH set the two numbers (tuning aids).
    auto live_rows = [&](int r) {
      // rows of the 8-row groups of slot r that hold a row of either run
      const int la = s->sdruns[2 * (run0 + r)].lb, lb2 = s->sdruns[2 * (run0 + r) + 1].lb;
      if (j == 0) return 8;
      if (d < 8) return (la < d || lb2 < d) ? 4 : 0;
      int rows = 0;
      for (int p0 = 0; p0 < d; p0 += 8)
        if (p0 + 7 >= la || p0 <= d - 1 - lb2) rows += 8;
      return rows;
    };
    std::vector<int> cut{0};
    {
      static const long long stages = [] {
        const char* e = std::getenv("EXPSKETCH_SYM_DG_STAGES");
        return e && std::atoll(e) > 0 ? std::atoll(e) : 5LL;
      }();
      static const long long ovh = [] {
        const char* e = std::getenv("EXPSKETCH_SYM_DG_OVH");
        return e && std::atoll(e) >= 0 ? std::atoll(e) : 32LL;
      }();
      const long long target = stages * (SD_R + ovh);
      long long cost = 0;
      for (int r = 0; r < nrun; r += NF) {
        long long sc = ovh;
        for (int f = 0; f < NF && r + f < nrun; ++f) sc += live_rows(r + f);
        if (cost > 0 && cost + sc > target) {
          cut.push_back(r);
          cost = 0;
        }
        cost += sc;
      }
      cut.push_back(nrun);
    }
    for (int col0 = 0; col0 < C; col0 += 64) {
      for (size_t ci = 0; ci + 1 < cut.size(); ++ci) {
        const int r0 = cut[ci];
        SymDgTile T{};
        T.xoff = lxoff;
        T.pofs = qp.pb;
        T.nrows = (int)cnt;
        T.C = C;
        T.top = top;
        T.j = j;
        T.col0 = col0;
        T.fw = std::min(64, C - col0);
        T.run0 = run0 + r0;
        T.nrun = cut[ci + 1] - r0;
        s->sdtiles.push_back(T);
        QryTile f{};
        f.pofs = qp.pb;
        f.C = C;
        f.top = top;
        f.fc0 = col0;
        f.fw = T.fw;
        qp.tiles.push_back(f);
        qp.pb += (long long)SK_DGQ * T.fw;
      }
    }
  }
}

// Builds the multiset layout's plans and device tables of a new handle.
int build_sym(sk_sketch* s) {
  SymHost t;
  sym_tables(s->d, s->p, &t, &s->Rlo);
  s->Dsym = (long long)t.code.size();
  s->Rtop = s->Dsym - s->Rlo;
  const int Cl = s->d + s->dv;
  s->XS = s->Rlo * Cl + s->Rtop * s->dv;
  if (s->Rlo > 0) plan_sym_update_block(s, &t, 0, 0, (int)s->Rlo, Cl, 0);
  plan_sym_update_block(s, &t, s->Rlo * Cl, (int)s->Rlo, (int)s->Rtop, s->dv, 1);
  // group the update tiles by shape (one launch per shape), order kept inside
  std::stable_sort(s->sutiles.begin(), s->sutiles.end(),
                   [](const SymUpdTile& a, const SymUpdTile& b) {
                     return a.rb * 8 + a.cb < b.rb * 8 + b.cb;
                   });
  for (size_t i = 0; i < s->sutiles.size(); ++i)
    if (i == 0 || s->sutiles[i].rb * 8 + s->sutiles[i].cb !=
                      s->sutiles[i - 1].rb * 8 + s->sutiles[i - 1].cb)
      s->sgroup.push_back((int)i);
  s->sgroup.push_back((int)s->sutiles.size());
  s->qplans.resize(1);
  // both blocks by the last index, or both by row ranges (one launch either way;
  // the two kernels side by side measured slower than the row-range kernel alone)
  const bool dg = (s->Rlo == 0 || sym_dg_block(s, Cl, s->p - 1)) && sym_dg_block(s, s->dv, s->p);
  if (dg) {
    if (s->Rlo > 0) plan_sym_dg_block(s, t, 0, 0, Cl, 0, 0, s->p - 1);
    plan_sym_dg_block(s, t, s->Rlo * Cl, s->Rlo, s->dv, 1, s->p, s->p);
  } else {
    if (s->Rlo > 0) plan_sym_query_block(s, 0, 0, (int)s->Rlo, Cl, 0);
    plan_sym_query_block(s, s->Rlo * Cl, (int)s->Rlo, (int)s->Rtop, s->dv, 1);
  }
  // one device allocation: code | prefix | last | lmul | rslot | winv | slots
  const size_t n = (size_t)s->Dsym, ns = t.slots.size();
  const size_t bytes = 8 * n + 4 * (5 * n + ns) + 64;
  if (hipMalloc(&s->symbuf, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return SK_ENOMEM;
  }
  char* base = static_cast<char*>(s->symbuf);
  size_t off = 0;
  auto put = [&](const void* src, size_t sz) -> void* {
    void* dst = base + off;
    off += (sz + 7) / 8 * 8;
    if (sz > 0 && hipMemcpy(dst, src, sz, hipMemcpyHostToDevice) != hipSuccess) return nullptr;
    return dst;
  };
  s->tb.code = static_cast<const unsigned long long*>(put(t.code.data(), 8 * n));
  s->tb.prefix = static_cast<const int*>(put(t.prefix.data(), 4 * n));
  s->tb.last = static_cast<const int*>(put(t.last.data(), 4 * n));
  s->tb.lmul = static_cast<const int*>(put(t.lmul.data(), 4 * n));
  s->tb.rslot = static_cast<const int*>(put(t.rslot.data(), 4 * n));
  s->tb.winv = static_cast<const float*>(put(t.winv.data(), 4 * n));
  s->tb.slots = static_cast<const int*>(put(t.slots.data(), 4 * ns));
  if (!s->tb.code || !s->tb.prefix || !s->tb.last || !s->tb.lmul || !s->tb.rslot ||
      !s->tb.winv || !s->tb.slots)
    return SK_EHIP;
  return SK_OK;
}

// Decode-step tiles: every block of the state cut into row ranges of at most
// fpt floats (and ST_ROWS rows).
void plan_step_block(sk_sketch* s, long long xoff, long long rows, int C, int top, int level,
                     int rc0, int j, long long fpt) {
  const long long rpt = std::max(1LL, std::min<long long>(ST_ROWS, fpt / C));
  double fj = 1.0;
  for (int i = 2; i <= j; ++i) fj *= i;
  for (long long r0 = 0; r0 < rows; r0 += rpt) {
    StepTile t{};
    t.xoff = xoff;
    t.row0 = r0;
    t.nrows = (int)std::min(rpt, rows - r0);
    t.C = C;
    t.top = top;
    t.level = level;
    t.rc0 = rc0;
    t.wn = (float)(1.0 / fj);
    t.wz = (float)(1.0 / (j + 1));
    s->stiles.push_back(t);
  }
}

void plan_step(sk_sketch* s) {
  // floats per tile: ST_FLOATS, halved (down to 2048) while the launch (tiles
  // times heads) would have fewer than two workgroups per CU
  // (EXPSKETCH_STEP_FLOATS lowers the largest tile, tuning aid)
  static const long long cap = [] {
    const char* e = std::getenv("EXPSKETCH_STEP_FLOATS");
    const long long v = e ? std::atoll(e) : 0;
    return (v >= 256 && v <= ST_FLOATS) ? v : (long long)ST_FLOATS;
  }();
  const long long total = (long long)s->XS * s->h;
  long long fpt = cap;
  while (fpt > 2048 && total / fpt < 2LL * std::max(1, s->dev.num_cu)) fpt /= 2;
  if (s->layout == SK_LAYOUT_SYM) {
    const int Cl = s->d + s->dv;
    if (s->Rlo > 0) plan_step_block(s, 0, s->Rlo, Cl, 0, -1, 0, 0, fpt);
    plan_step_block(s, s->Rlo * Cl, s->Rtop, s->dv, 1, -1, (int)s->Rlo, 0, fpt);
  } else {
    for (int j = 0; j <= s->p; ++j)
      plan_step_block(s, s->xoff[j], s->rows[j], s->C[j], j == s->p, j, 0, j, fpt);
  }
}

int update_tile_count(const sk_sketch* s) {
  return (int)(s->layout == SK_LAYOUT_SYM ? s->sutiles.size() : s->utiles.size());
}

// Keys per launch of the digit-organised update: byte offsets from a split's
// first key or value row stay below 2^31 (EXPSKETCH_UPDATE_MAXKEYS lowers it, to
// test the cut).
long long kr_max_keys(const sk_sketch* s) {
  static const long long forced = [] {
    const char* v = std::getenv("EXPSKETCH_UPDATE_MAXKEYS");
    return v ? std::max(0LL, std::atoll(v)) : 0LL;
  }();
  const long long row = 4LL * std::max(s->d, s->dv);
  const long long lim = ((1LL << 31) - (1LL << 20)) / row / 1024 * 1024;
  return forced > 0 ? std::min(forced, lim) : lim;
}

// Key splits of the digit-organised update for n keys, given the split count of
// the heaviest group: a lighter group takes proportionally fewer, longer splits.
// Bytes of each of the two split-partials buffers above which an update call
// takes per-call partials and reduces them at once instead.
constexpr size_t kDeferBytes = size_t(1) << 30;

KrSplits kr_splits_for(const sk_sketch* s, long long n, long long ns0) {
  KrSplits P{};
  P.ngroup = (int)s->kweight.size();
  P.nsplit = 1;
  long long items = 0;
  for (int g = 0; g < P.ngroup; ++g) {
    const long long want =
        std::max(1LL, (ns0 * s->kweight[g] + s->kweight[0] - 1) / s->kweight[0]);
    const long long kps = std::max(1LL, (n + want - 1) / want);
    const long long ns = std::max(1LL, (n + kps - 1) / kps);
    P.unit0[g] = s->kgroup0[g];
    P.ns[g] = (int)ns;
    P.kps[g] = kps;
    P.item0[g] = items;
    items += (long long)(s->kgroup0[g + 1] - s->kgroup0[g]) * ns;
    P.nsplit = std::max(P.nsplit, (int)ns);
  }
  P.unit0[P.ngroup] = s->kgroup0[P.ngroup];
  P.item0[P.ngroup] = items;
  return P;
}

// Splits of the heaviest group: the fewest key-steps on the busiest SIMD (waves
// per SIMD times the heaviest group's split length), plus a small charge per
// partial buffer (written, then read by the reduce), plus a tail when a SIMD
// takes its waves in more than one round; at least 256 keys a split.
KrSplits choose_kr_splits(const sk_sketch* s, long long n) {
  static const int forced = [] {
    const char* v = std::getenv("EXPSKETCH_UPDATE_SPLITS");
    return v ? std::max(0, std::atoi(v)) : 0;
  }();
  // A head's items are taken lightest group first (EXPSKETCH_KR_REVERSE=0 takes
  // the heaviest first, tuning aid): a light unit's split runs over the most
  // keys, so its waves are the longest; started last they set the launch's tail
  // (measured on MI355X: 32-head workload 23.6 -> 20.5 ms per launch on one box,
  // 20.5-20.9 -> 20.5 on others; d = 32, p = 3 workload 0.76 -> 0.79 of the fp32
  // peak; d = 16, p = 4 unchanged).
  static const int rev = [] {
    const char* v = std::getenv("EXPSKETCH_KR_REVERSE");
    return v ? (std::atoi(v) != 0 ? 1 : 0) : 1;
  }();
  if (forced > 0) {
    KrSplits P = kr_splits_for(s, n, std::min<long long>(forced, std::max(1LL, n)));
    P.rev = rev;
    return P;
  }
  const long long simds = (long long)std::max(1, s->dev.num_cu) * 4;
  const long long max_ns = std::max(1LL, std::min(64LL, n / 256));
  // split partials that fit the kept buffers (the deferred reduce) are preferred
  // to more splits that would need per-call buffers
  const size_t state_bytes = sizeof(float) * (size_t)s->XS * (size_t)s->h;
  KrSplits best = kr_splits_for(s, n, 1);
  double best_cost = -1.0;
  for (long long ns = 1; ns <= max_ns; ++ns) {
    const KrSplits P = kr_splits_for(s, n, ns);
    if (P.nsplit > 1 && 2 * state_bytes <= kDeferBytes &&
        (size_t)P.nsplit * state_bytes > kDeferBytes)
      continue;
    const long long waves = P.item0[P.ngroup] * s->h;
    const long long per_simd = (waves + simds - 1) / simds;   // they share its matrix core
    // measured on MI355X (a SIMD holds three of this kernel's waves): with one
    // wave per SIMD a launch runs about 20% slower than with three (no other wave
    // covers its waits), with two about 5% slower
    const double shape = per_simd == 1 ? 1.2 : per_simd == 2 ? 1.05 : 1.0;
    // with more waves than a SIMD holds at once (three), they start as earlier
    // ones end and finish unevenly: the launch's tail, measured on MI355X as
    // about 2.2 wave lengths (32-head d = 64 workload: 8 splits 20.0 ms per
    // launch, 12 19.5, 16 19.0, 24 18.1-18.4, 32 18.2; one-round launches, where
    // all waves start together, have no such tail)
    const double tail = per_simd > 3 ? 2.2 : 0.0;
    const double cost =
        (double)P.kps[0] * ((double)per_simd * (1.0 + 0.003 * P.nsplit) * shape + tail);
    if (best_cost < 0.0 || cost < best_cost - 1e-9) {
      best_cost = cost;
      best = P;
    }
  }
  best.rev = rev;
  return best;
}

int choose_update_splits(const sk_sketch* s, long long n) {
  // EXPSKETCH_UPDATE_SPLITS=<k> fixes the number of key splits (tuning aid).
  static const int forced = [] {
    const char* v = std::getenv("EXPSKETCH_UPDATE_SPLITS");
    return v ? std::max(0, std::atoi(v)) : 0;
  }();
  if (forced > 0) return (int)std::max(1LL, std::min<long long>(forced, (n + SK_KB - 1) / SK_KB));
  const long long base = (long long)update_tile_count(s) * s->h;
  const bool sym = s->layout == SK_LAYOUT_SYM;
  // workgroups resident per CU: two for the full layout's kernel; for the
  // multiset kernel its wave bound (four, two for the 16-block shape) and LDS
  long long per_cu = 2;
  if (sym) {
    const int cb = sym_update_cb(s->dv);
    per_cu = (sym_update_rb() * cb >= 16) ? 2 : 4;
    const long long fit = (long long)s->dev.max_lds / (long long)sym_update_lds_bytes(s->d, s->dv);
    per_cu = std::max(1LL, std::min(per_cu, fit));
  }
  const long long slots = per_cu * std::max(1, s->dev.num_cu);
  // at least 256 keys (multiset layout: 128) per split
  const long long minkeys = sym ? 128 : 256;
  const long long max_ns = std::max(1LL, std::min(sym ? 128LL : 64LL, n / minkeys));
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


// Adds the last update call's pending partials into the state (fixed split order).
int flush_pending(sk_sketch* s) {
  if (s->pend == nullptr) return SK_OK;
  const long long c4 = s->XS * s->h / 4;
  const int grid = (int)std::min<long long>((c4 + 255) / 256, 16384);
  hipLaunchKernelGGL(sk_split_reduce_kernel, dim3(grid), dim3(256), 0, s->stream,
                     reinterpret_cast<float4*>(s->state),
                     reinterpret_cast<const float4*>(s->pend), c4, s->pend_ns, c4);
  s->pend = nullptr;
  s->pend_ns = 0;
  SK_TRY(hipGetLastError());
  return SK_OK;
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

int sk_version(void) { return 101; }

const char* sk_strerror(int code) {
  switch (code) {
    case SK_OK: return "ok";
    case SK_EINVAL: return "invalid argument";
    case SK_ENOMEM: return "out of device memory";
    case SK_EMISMATCH: return "sketch shapes differ";
    case SK_EHIP: return "HIP runtime error";
    case SK_ESCRATCH: return "request exceeds the fixed scratch buffer";
    default: return "unknown status";
  }
}

int sketch_create_ex(int d, int dv, int p, int h, int layout, void* hip_stream,
                     sk_handle* out) {
  if (out == nullptr) return SK_EINVAL;
  *out = nullptr;
  if (!is_pow2_in(d, 4, 128) || !is_pow2_in(dv, 4, 128) || p < 0 || p > kMaxP || h < 1)
    return SK_EINVAL;
  if (layout != SK_LAYOUT_FULL && layout != SK_LAYOUT_SYM) return SK_EINVAL;
  if (layout == SK_LAYOUT_SYM && p > SY_MAXP) return SK_EINVAL;
  // sizes, with overflow checks in floating point first
  double XSd = 0.0, rowsd = 0.0;
  for (int j = 0; j <= p; ++j) {
    double r = std::pow((double)d, j);
    if (layout == SK_LAYOUT_SYM) {            // C(d + j - 1, j)
      r = 1.0;
      for (int i = 1; i <= j; ++i) r = r * (double)(d + i - 1) / (double)i;
    }
    XSd += r * (double)(j < p ? d + dv : dv);
    rowsd += r;
  }
  if (XSd * (double)h * 4.0 > 1.0e15) return SK_ENOMEM;
  if (layout == SK_LAYOUT_SYM && rowsd > 2.0e8) return SK_ENOMEM;   // int row ids, tables

  sk_sketch* s = new (std::nothrow) sk_sketch();
  if (s == nullptr) return SK_ENOMEM;
  s->d = d; s->dv = dv; s->p = p; s->h = h; s->logd = ilog2(d);
  s->layout = layout;
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
  const bool sym = layout == SK_LAYOUT_SYM;
  const size_t ul = sym ? sym_update_lds_bytes(d, dv) : update_lds_bytes(d, dv);
  const size_t ql = sym ? sym_query_lds_bytes(d) : query_lds_bytes(d);
  if (ul > (size_t)s->dev.max_lds || ql > (size_t)s->dev.max_lds) {
    delete s;
    return SK_EINVAL;
  }
  if (sym) {
    rc = build_sym(s);   // sets XS, the sym tiles, the finishing records and tables
    if (rc != SK_OK) {
      (void)hipFree(s->symbuf);
      delete s;
      return rc;
    }
  } else {
    for (int j = 0; j <= p; ++j) plan_update_level(s, j, &s->utiles);
    if (query_rows_fixed() > 0) {
      s->qplans.resize(1);
      s->qplans[0].rows = query_rows_fixed();
    } else {
      s->qplans.resize(3);
      for (int i = 0; i < 3; ++i) s->qplans[i].rows = 512 >> i;
    }
    for (sk_sketch::QPlan& qp : s->qplans) {
      for (int j = 0; j <= p; ++j) plan_query_level(s, j, &qp);
      // group the query tiles by kernel (tile order kept inside a group)
      for (int key : {0, 16, 32}) {
        const int off = (int)qp.run.size();
        for (size_t i = 0; i < qp.tiles.size(); ++i)
          if (qp.kind[i] == key) qp.run.push_back(qp.tiles[i]);
        const int cnt = (int)qp.run.size() - off;
        // the last-digit kernels dispatch their tiles in this order: longest first,
        // so the short ones fill the slots the long ones leave at the end
        if (key == 16)
          std::stable_sort(qp.run.begin() + off, qp.run.end(),
                           [](const QryTile& x, const QryTile& y) {
                             return query_tile_work(x) > query_tile_work(y);
                           });
        if (cnt > 0) qp.groups.push_back(sk_sketch::QGroup{key / 16, key % 16, off, cnt});
      }
    }
    if (kr_width(d) && use_update_kr()) plan_kr_units(s);
  }

  plan_step(s);
  const size_t state_bytes = sizeof(float) * (size_t)s->XS * (size_t)h;
  if (hipMalloc(&s->state, state_bytes) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(s->symbuf);
    delete s;
    return SK_ENOMEM;
  }
  auto upload = [](void** dst, const void* src, size_t bytes) {
    if (bytes == 0) return true;
    return hipMalloc(dst, bytes) == hipSuccess &&
           hipMemcpy(*dst, src, bytes, hipMemcpyHostToDevice) == hipSuccess;
  };
  bool ok = true;
  for (sk_sketch::QPlan& qp : s->qplans) {
    // finishing records: tile record offset, width, entry column of its column 0
    std::vector<FinTile> fin;
    for (const QryTile& T : qp.tiles) fin.push_back(FinTile{T.pofs, T.fw, (T.top ? d : 0) + T.fc0});
    ok = ok && upload((void**)&qp.d_fin, fin.data(), sizeof(FinTile) * fin.size()) &&
         upload((void**)&qp.d_run, qp.run.data(), sizeof(QryTile) * qp.run.size());
  }
  ok = ok &&
            upload((void**)&s->d_stiles, s->stiles.data(),
                   sizeof(StepTile) * s->stiles.size()) &&
            hipMalloc(&s->sparts, sizeof(float) * (size_t)h * s->stiles.size() * (1 + dv)) ==
                hipSuccess;
  if (ok && sym)
    ok = upload((void**)&s->d_sutiles, s->sutiles.data(),
                sizeof(SymUpdTile) * s->sutiles.size()) &&
         upload((void**)&s->d_sqtiles, s->sqtiles.data(),
                sizeof(SymQryTile) * s->sqtiles.size()) &&
         upload((void**)&s->d_sdtiles, s->sdtiles.data(),
                sizeof(SymDgTile) * s->sdtiles.size()) &&
         upload((void**)&s->d_sdruns, s->sdruns.data(), sizeof(SymDgRun) * s->sdruns.size()) &&
         hipFuncSetAttribute((const void*)sym_dg_kernel_for(s->logd),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)sym_dg_lds_bytes()) == hipSuccess &&
         hipFuncSetAttribute((const void*)sk_sym_query_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ql) == hipSuccess;
  for (size_t g = 0; ok && sym && g + 1 < s->sgroup.size(); ++g) {
    const SymUpdTile& t0 = s->sutiles[s->sgroup[g]];
    for (int cen = 0; cen < 2 && ok; ++cen)
      ok = hipFuncSetAttribute((const void*)sym_update_kernel_for(t0.rb, t0.cb, cen != 0),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)ul) == hipSuccess;
  }
  for (size_t g = 0; ok && !sym && g < s->qplans[0].groups.size(); ++g) {
    const sk_sketch::QGroup& G = s->qplans[0].groups[g];
    if (G.kind == 1)
      ok = hipFuncSetAttribute((const void*)query_dg_kernel_for(s->logd),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)query_dg_lds_bytes(d)) == hipSuccess;
    else if (G.kind == 2)
      ok = hipFuncSetAttribute((const void*)query_dg16_kernel_for(s->logd),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)query_dg16_lds_bytes(d)) == hipSuccess;
  }
  if (ok && !sym)
    ok = upload((void**)&s->d_utiles, s->utiles.data(), sizeof(UpdTile) * s->utiles.size()) &&
         upload((void**)&s->d_kunits, s->kunits.data(), sizeof(KrUnit) * s->kunits.size()) &&
         hipFuncSetAttribute((const void*)update_kernel_for(false, d, dv),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ul) == hipSuccess &&
         hipFuncSetAttribute((const void*)update_kernel_for(true, d, dv),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ul) == hipSuccess &&
         hipFuncSetAttribute((const void*)query_kernel_for(s->logd),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ql) == hipSuccess;
  if (ok) ok = launch_fill_zero(s->state, s->XS * h, s->stream) == SK_OK;
  if (!ok) {
    (void)hipGetLastError();
    (void)hipFree(s->state); (void)hipFree(s->d_utiles);
    for (sk_sketch::QPlan& qp : s->qplans) { (void)hipFree(qp.d_fin); (void)hipFree(qp.d_run); }
    (void)hipFree(s->d_kunits);
    (void)hipFree(s->d_sutiles); (void)hipFree(s->d_sqtiles); (void)hipFree(s->symbuf);
    (void)hipFree(s->d_sdtiles); (void)hipFree(s->d_sdruns);
    (void)hipFree(s->d_stiles); (void)hipFree(s->sparts);
    delete s;
    return SK_EHIP;
  }
  *out = s;
  return SK_OK;
}

int sketch_create(int d, int dv, int p, int h, void* hip_stream, sk_handle* out) {
  return sketch_create_ex(d, dv, p, h, SK_LAYOUT_FULL, hip_stream, out);
}

int sketch_layout(sk_handle s, int* layout, int64_t* rows) {
  if (s == nullptr) return SK_EINVAL;
  if (layout) *layout = s->layout;
  if (rows) *rows = s->layout == SK_LAYOUT_SYM ? s->Dsym : s->D;
  return SK_OK;
}

int sketch_update_path(sk_handle s, int* kind) {
  if (s == nullptr || kind == nullptr) return SK_EINVAL;
  *kind = s->layout == SK_LAYOUT_SYM ? SK_UPDATE_MULTISET
          : s->kunits.empty()        ? SK_UPDATE_TILES
                                     : SK_UPDATE_DIGITS;
  return SK_OK;
}

int sketch_destroy(sk_handle s) {
  if (s == nullptr) return SK_OK;
  int rc = SK_OK;
  if (hipStreamSynchronize(s->stream) != hipSuccess) rc = SK_EHIP;
  (void)hipFree(s->state);
  (void)hipFree(s->d_utiles);
  (void)hipFree(s->d_kunits);
  for (sk_sketch::QPlan& qp : s->qplans) {
    (void)hipFree(qp.d_fin);
    (void)hipFree(qp.d_run);
  }
  (void)hipFree(s->d_sutiles);
  (void)hipFree(s->d_sqtiles);
  (void)hipFree(s->d_sdtiles);
  (void)hipFree(s->d_sdruns);
  (void)hipFree(s->symbuf);
  (void)hipFree(s->d_stiles);
  (void)hipFree(s->sparts);
  (void)hipFree(s->center);
  (void)hipFree(s->pbuf[0]);
  (void)hipFree(s->pbuf[1]);
  (void)hipFree(s->stage_k);
  (void)hipFree(s->stage_v);
  if (s->flush_ev != nullptr) (void)hipEventDestroy(s->flush_ev);
  if (s->switch_ev != nullptr) (void)hipEventDestroy(s->switch_ev);
  free_workspace(&s->qws);
  (void)hipFree(s->view);
  for (int k = 0; k < 3; ++k)
    for (int w = 0; w < 2; ++w)
      for (hipEvent_t e : s->tev[k][w]) (void)hipEventDestroy(e);
  delete s;
  return rc;
}

int sketch_set_stream(sk_handle s, void* hip_stream) {
  if (s == nullptr) return SK_EINVAL;
  const hipStream_t ns = reinterpret_cast<hipStream_t>(hip_stream);
  if (ns == s->stream) return SK_OK;
  // the handle's buffers (state, staged keys, pending partials, query partials)
  // are ordered by its stream alone: the new stream first waits for everything
  // issued so far on the old one
  if (s->switch_ev == nullptr)
    SK_TRY(hipEventCreateWithFlags(&s->switch_ev, hipEventDisableTiming));
  SK_TRY(hipEventRecord(s->switch_ev, s->stream));
  SK_TRY(hipStreamWaitEvent(ns, s->switch_ev, 0));
  s->stream = ns;
  return SK_OK;
}

int sketch_reset(sk_handle s) {
  if (s == nullptr) return SK_EINVAL;
  s->count = 0;
  s->pend = nullptr;            // pending partials and staged keys belong to the
  s->stage_n = 0;               // old contents
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

}  // extern "C"

namespace {

// The moment update of n keys per head, K [h][hkeys][d] (keys of head h start at
// K + h * hkeys * d), V likewise: one launch (plus the deferred reduce).
int run_update(sk_sketch* s, const float* K, const float* V, int64_t n, long long hkeys) {
  const bool kr = s->layout == SK_LAYOUT_FULL && !s->kunits.empty();
  if (kr) {
    // the digit kernel addresses a split's rows with 32-bit byte offsets: longer
    // calls run as several launches
    const long long maxkeys = kr_max_keys(s);
    if (n > maxkeys) {
      for (long long off = 0; off < n; off += maxkeys) {
        const int rc = run_update(s, K + off * s->d, V + off * s->dv,
                                  std::min<long long>(maxkeys, n - off), hkeys);
        if (rc != SK_OK) return rc;
      }
      return SK_OK;
    }
  }
  KrSplits ksp{};
  long long kps = 0;
  int nsplit = 1;
  if (kr) {
    ksp = choose_kr_splits(s, n);
    nsplit = ksp.nsplit;
  } else {
    const int ns = choose_update_splits(s, n);
    kps = (n + ns - 1) / ns;
    kps = (kps + SK_KB - 1) / SK_KB * SK_KB;
    nsplit = (int)((n + kps - 1) / kps);
  }
  const bool sym = s->layout == SK_LAYOUT_SYM;
  const int ntiles = update_tile_count(s);
  const long long total = s->XS * s->h;
  const long long rmax = (total / 4 + SK_RED4 - 1) / SK_RED4;     // reduce workgroups
  const long long kr_wgs = kr ? (ksp.item0[ksp.ngroup] * s->h + KR_WAVES - 1) / KR_WAVES : 0;
  if ((long long)ntiles * nsplit * s->h + rmax > 0x7fffffffLL || kr_wgs + rmax > 0x7fffffffLL)
    return SK_EINVAL;
  const size_t lds = sym ? sym_update_lds_bytes(s->d, s->dv) : update_lds_bytes(s->d, s->dv);
  int rc = SK_OK;
  float* dst = s->state;
  float* tmp = nullptr;         // per-call partials (states too large to defer)
  bool deferred = false;
  PendingReduce red{};
  red.state = reinterpret_cast<float4*>(s->state);
  red.count4 = total / 4;
  if (nsplit == 1) {
    rc = flush_pending(s);      // this call adds into the state itself
    if (rc != SK_OK) return rc;
  } else {
    const size_t need = (size_t)total * nsplit;
    if (need * sizeof(float) <= kDeferBytes) {
      if (s->pbuf_floats < need) {
        rc = flush_pending(s);
        if (rc != SK_OK) return rc;
        SK_TRY(hipStreamSynchronize(s->stream));
        (void)hipFree(s->pbuf[0]);
        (void)hipFree(s->pbuf[1]);
        s->pbuf[0] = s->pbuf[1] = nullptr;
        s->pbuf_floats = 0;
        if (hipMalloc(&s->pbuf[0], need * sizeof(float)) == hipSuccess &&
            hipMalloc(&s->pbuf[1], need * sizeof(float)) == hipSuccess) {
          s->pbuf_floats = need;
        } else {
          (void)hipGetLastError();
          (void)hipFree(s->pbuf[0]);
          (void)hipFree(s->pbuf[1]);
          s->pbuf[0] = s->pbuf[1] = nullptr;
        }
      }
      deferred = s->pbuf_floats >= need;
    }
    if (deferred) {
      dst = s->pbuf[s->pcur];
      if (s->pend != nullptr) {
        red.parts = reinterpret_cast<const float4*>(s->pend);
        red.nsplit = s->pend_ns;
      }
    } else {
      rc = flush_pending(s);
      if (rc != SK_OK) return rc;
      if (hipMallocAsync((void**)&tmp, sizeof(float) * need, s->stream) != hipSuccess) {
        (void)hipGetLastError();
        return SK_ENOMEM;
      }
      dst = tmp;
    }
  }
  const long long sstride = nsplit > 1 ? total : 0;
  const int acc = nsplit > 1 ? 0 : 1;
  const long long rwgs = red.parts != nullptr ? rmax : 0;
  hipError_t err = hipSuccess;
  hipEvent_t ev0, ev1;
  timing_pair(s, 0, &ev0, &ev1);
  if (sym) {
    const size_t ng = s->sgroup.size() - 1;
    for (size_t g = 0; g < ng; ++g) {
      const int t0 = s->sgroup[g], nt = s->sgroup[g + 1] - t0;
      const SymUpdTile& sh = s->sutiles[t0];
      PendingReduce rg = red;                  // the reduce rides on the first launch
      if (g > 0) rg.parts = nullptr;
      const long long extra = g == 0 ? rwgs : 0;
      launch_ev(sym_update_kernel_for(sh.rb, sh.cb, s->center != nullptr),
                dim3((unsigned)((long long)nt * nsplit * s->h + extra)), dim3(SK_WG), lds,
                s->stream, g == 0 ? ev0 : nullptr, g + 1 == ng ? ev1 : nullptr, K, V,
                (long long)n, hkeys, s->d, s->dv, s->d_sutiles + t0, nt, s->tb, kps, nsplit,
                s->h, dst, s->XS, sstride, acc, s->center, rg);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) err = e;
    }
  } else if (kr) {
    launch_ev(update_kr_kernel_for(s->center != nullptr, s->d), dim3((unsigned)(kr_wgs + rwgs)),
              dim3(64 * KR_WAVES), 0, s->stream, ev0, ev1, K, V, (long long)n, hkeys, s->dv,
              s->d_kunits, ksp, s->h, dst, s->XS, sstride, acc, s->center, red);
    err = hipGetLastError();
  } else {
    launch_ev(update_kernel_for(s->center != nullptr, s->d, s->dv),
              dim3((unsigned)((long long)ntiles * nsplit * s->h + rwgs)), dim3(SK_WG), lds,
              s->stream, ev0, ev1, K, V, (long long)n, hkeys, s->d, s->dv, s->logd, s->d_utiles,
              ntiles, kps, nsplit, s->h, dst, s->XS, sstride, acc, s->center, red);
    err = hipGetLastError();
  }
  timing_done(s, 0);
  if (deferred) {
    s->pend = dst;
    s->pend_ns = nsplit;
    s->pcur ^= 1;
  } else if (tmp != nullptr) {
    const long long c4 = total / 4;
    const int grid = (int)std::min<long long>((c4 + 255) / 256, 16384);
    hipLaunchKernelGGL(sk_split_reduce_kernel, dim3(grid), dim3(256), 0, s->stream,
                       reinterpret_cast<float4*>(s->state),
                       reinterpret_cast<const float4*>(tmp), c4, nsplit, c4);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) err = e;
    (void)hipFreeAsync(tmp, s->stream);
  }
  if (err != hipSuccess) return SK_EHIP;
  return SK_OK;
}

// Contracts the staged keys (if any) into the state.
int flush_stage(sk_sketch* s) {
  if (s->stage_n == 0) return SK_OK;
  const long long n = s->stage_n;
  s->stage_n = 0;
  return run_update(s, s->stage_k, s->stage_v, n, s->stage_cap);
}

// Everything a reader of the state needs done first: staged keys, then pending
// split partials.
int settle(sk_sketch* s) {
  int rc = flush_stage(s);
  if (rc == SK_OK) rc = flush_pending(s);
  return rc;
}

// Default staging size: up to 32768 keys per head in at most 32 MB, off below
// 1024 keys.
long long default_stage_cap(const sk_sketch* s) {
  const long long per_key = (long long)sizeof(float) * (s->d + s->dv) * s->h;
  static const long long keys = [] {   // EXPSKETCH_STAGE_KEYS overrides 32768 (tuning aid)
    const char* e = std::getenv("EXPSKETCH_STAGE_KEYS");
    const long long v = e ? std::atoll(e) : 0;
    return v > 0 ? v : 32768LL;
  }();
  long long cap = std::min<long long>(keys, (32LL << 20) / per_key);
  cap = cap / SK_KB * SK_KB;
  return cap >= 1024 ? cap : 0;
}

}  // namespace

extern "C" {

int sketch_update(sk_handle s, const float* K, const float* V, int64_t n) {
  if (s == nullptr || n < 0) return SK_EINVAL;
  if (n == 0) return SK_OK;
  if (K == nullptr || V == nullptr || !aligned16(K) || !aligned16(V)) return SK_EINVAL;
  if (s->stage_cap < 0) s->stage_cap = default_stage_cap(s);
  // calls of fewer than half the staging size are staged; larger ones run at once
  if (s->stage_cap > 0 && 2 * n <= s->stage_cap) {
    int rc = SK_OK;
    if (s->stage_n + n > s->stage_cap) rc = flush_stage(s);
    if (rc != SK_OK) return rc;
    if (s->stage_k == nullptr) {
      const size_t kb = sizeof(float) * (size_t)s->h * s->stage_cap * s->d;
      const size_t vb = sizeof(float) * (size_t)s->h * s->stage_cap * s->dv;
      if (hipMalloc(&s->stage_k, kb) != hipSuccess || hipMalloc(&s->stage_v, vb) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(s->stage_k);
        (void)hipFree(s->stage_v);
        s->stage_k = s->stage_v = nullptr;
        s->stage_cap = 0;          // no staging from now on
      }
    }
    if (s->stage_cap > 0) {
      // one launch appends K and V of every head (n <= stage_cap / 2 keys)
      const long long w4 = std::max(s->d, s->dv) / 4;
      const int nb = (int)std::min<long long>(64, (n * w4 + 255) / 256);
      if ((long long)nb * 2 * s->h > 0x7fffffffLL) return SK_EINVAL;
      hipLaunchKernelGGL(sk_stage_copy_kernel, dim3((unsigned)(nb * 2 * s->h)), dim3(256), 0,
                         s->stream, reinterpret_cast<const float4*>(K),
                         reinterpret_cast<const float4*>(V), (long long)n, s->d / 4, s->dv / 4,
                         nb, reinterpret_cast<float4*>(s->stage_k),
                         reinterpret_cast<float4*>(s->stage_v), s->stage_cap, s->stage_n);
      SK_TRY(hipGetLastError());
      s->stage_n += n;
      s->count += n;
      return s->stage_n == s->stage_cap ? flush_stage(s) : SK_OK;
    }
  }
  int rc = flush_stage(s);           // staged keys go first (the order is fixed)
  if (rc == SK_OK) rc = run_update(s, K, V, n, n);
  if (rc != SK_OK) return rc;
  s->count += n;
  return SK_OK;
}

int sketch_set_staging(sk_handle s, int64_t keys) {
  if (s == nullptr || keys < 0) return SK_EINVAL;
  int rc = flush_stage(s);
  if (rc != SK_OK) return rc;
  SK_TRY(hipStreamSynchronize(s->stream));
  (void)hipFree(s->stage_k);
  (void)hipFree(s->stage_v);
  s->stage_k = s->stage_v = nullptr;
  s->stage_cap = keys / SK_KB * SK_KB;
  return SK_OK;
}

int sketch_merge(sk_handle dst, sk_handle src) {
  if (dst == nullptr || src == nullptr || dst == src) return SK_EINVAL;
  if (dst->d != src->d || dst->dv != src->dv || dst->p != src->p || dst->h != src->h ||
      dst->layout != src->layout || dst->center_host != src->center_host)
    return SK_EMISMATCH;
  // src's pending partials go into its state on src's stream; dst's stream then
  // waits for everything issued on src's stream before reading its state
  int rc = settle(src);
  if (rc == SK_OK && src->stream != dst->stream) {
    if (src->flush_ev == nullptr)
      SK_TRY(hipEventCreateWithFlags(&src->flush_ev, hipEventDisableTiming));
    SK_TRY(hipEventRecord(src->flush_ev, src->stream));
    SK_TRY(hipStreamWaitEvent(dst->stream, src->flush_ev, 0));
  }
  if (rc == SK_OK) rc = settle(dst);
  if (rc != SK_OK) return rc;
  const long long c4 = dst->XS * dst->h / 4;
  const int grid = (int)std::min<long long>((c4 + 255) / 256, 16384);
  hipLaunchKernelGGL(sk_add_kernel, dim3(grid), dim3(256), 0, dst->stream,
                     reinterpret_cast<float4*>(dst->state),
                     reinterpret_cast<const float4*>(src->state), c4);
  SK_TRY(hipGetLastError());
  if (src->stream != dst->stream) {
    // src's later writes wait until the add has read its state
    SK_TRY(hipEventRecord(src->flush_ev, dst->stream));
    SK_TRY(hipStreamWaitEvent(src->stream, src->flush_ev, 0));
  }
  dst->count += src->count;
  return SK_OK;
}

int sketch_query(sk_handle s, const float* Q, int64_t m, float* out, float* Z) {
  if (s == nullptr || m < 0) return SK_EINVAL;
  if (m == 0) return SK_OK;
  if (Q == nullptr || out == nullptr || Z == nullptr || !aligned16(Q)) return SK_EINVAL;
  {
    const int rc = settle(s);
    if (rc != SK_OK) return rc;
  }
  const long long nqt = (m + SK_TMQ - 1) / SK_TMQ;
  // the plan with the longest row ranges whose launch still gives every CU two
  // workgroups (shorter ranges: more partials to add, so only where needed)
  size_t pi = 0;
  while (pi + 1 < s->qplans.size() &&
         (long long)s->qplans[pi].tiles.size() * nqt * s->h < 2LL * s->dev.num_cu)
    ++pi;
  const sk_sketch::QPlan& qp = s->qplans[pi];
  const int ntiles = (int)qp.tiles.size();
  const long long nlaunch = std::max<long long>(
      ntiles, std::max<long long>((long long)s->sqtiles.size(), (long long)s->sdtiles.size()));
  if (nqt * nlaunch * s->h > 0x7fffffffLL || m * s->h > 0x7fffffffLL) return SK_EINVAL;
  const size_t pbytes = sizeof(float) * (size_t)s->h * nqt * qp.pb;
  float* parts = nullptr;
  bool own = false;
  {
    const int rc = take_workspace(&s->qws, pbytes, s->stream, &parts, &own);
    if (rc != SK_OK) return rc;
  }
  hipError_t e1 = hipSuccess;
  {
    // the timed region's kernels: the start event on the first, the stop event on
    // the last
    hipEvent_t ev0, ev1;
    timing_pair(s, 1, &ev0, &ev1);
    const bool sq = s->layout == SK_LAYOUT_SYM && !s->sqtiles.empty();
    const bool sd = s->layout == SK_LAYOUT_SYM && !s->sdtiles.empty();
    const int nl = s->layout == SK_LAYOUT_SYM ? (sq ? 1 : 0) + (sd ? 1 : 0)
                                              : (int)qp.groups.size();
    int li = 0;
    auto evs = [&](hipEvent_t* a, hipEvent_t* b) {
      *a = li == 0 ? ev0 : nullptr;
      *b = li + 1 == nl ? ev1 : nullptr;
      ++li;
    };
    hipEvent_t a, b;
    if (sq) {
      const long long nst = (long long)s->sqtiles.size();
      evs(&a, &b);
      launch_ev(sk_sym_query_kernel, dim3((unsigned)(nst * nqt * s->h)), dim3(SK_WG),
                sym_query_lds_bytes(s->d), s->stream, a, b, Q, (long long)m, s->d,
                (const float*)s->state, s->XS, (const SymQryTile*)s->d_sqtiles, (int)nst,
                (int)nqt, s->tb, qp.pb, parts);
      e1 = hipGetLastError();
    }
    if (sd) {
      const long long nsd = (long long)s->sdtiles.size();
      evs(&a, &b);
      launch_ev(sym_dg_kernel_for(s->logd), dim3((unsigned)(nsd * nqt * s->h)), dim3(SK_WG),
                sym_dg_lds_bytes(), s->stream, a, b, Q, (long long)m, (const float*)s->state,
                s->XS, (const SymDgTile*)s->d_sdtiles, (int)nsd, (const SymDgRun*)s->d_sdruns,
                (int)nqt, qp.pb, parts);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) e1 = e;
    }
    for (size_t g = 0; s->layout != SK_LAYOUT_SYM && g < qp.groups.size(); ++g) {
      const sk_sketch::QGroup& G = qp.groups[g];
      QueryKernel kern = G.kind == 0   ? query_kernel_for(s->logd)
                         : G.kind == 1 ? query_dg_kernel_for(s->logd)
                                       : query_dg16_kernel_for(s->logd);
      const size_t lds = G.kind == 0   ? query_lds_bytes(s->d)
                         : G.kind == 1 ? query_dg_lds_bytes(s->d)
                                       : query_dg16_lds_bytes(s->d);
      evs(&a, &b);
      launch_ev(kern, dim3((unsigned)((long long)G.count * nqt * s->h)), dim3(SK_WG), lds,
                s->stream, a, b, Q, (long long)m, (const float*)s->state, s->XS,
                (const QryTile*)(qp.d_run + G.off), G.count, (int)nqt, qp.pb, parts);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) e1 = e;
    }
    timing_done(s, 1);
  }
  // one finishing workgroup per (head, query)
  hipLaunchKernelGGL(sk_query_finish, dim3((unsigned)(m * s->h)), dim3(256), 0, s->stream,
                     parts, qp.d_fin, ntiles, (int)nqt, qp.pb, (long long)m, s->d, s->dv,
                     (float)s->count, Q, s->center, out, Z);
  hipError_t e2 = hipGetLastError();
  release_workspace(parts, own, s->stream);
  if (e1 != hipSuccess || e2 != hipSuccess) return SK_EHIP;
  return SK_OK;
}

int sketch_set_center(sk_handle s, const float* c) {
  if (s == nullptr) return SK_EINVAL;
  if (s->count != 0) return SK_EINVAL;            // only on an empty sketch
  if (c == nullptr) {
    SK_TRY(hipStreamSynchronize(s->stream));
    (void)hipFree(s->center);
    s->center = nullptr;
    s->center_host.clear();
    return SK_OK;
  }
  if (!aligned16(c)) return SK_EINVAL;
  const size_t bytes = sizeof(float) * (size_t)s->h * s->d;
  SK_TRY(hipStreamSynchronize(s->stream));
  if (s->center == nullptr && hipMalloc(&s->center, bytes) != hipSuccess) {
    (void)hipGetLastError();
    s->center = nullptr;
    return SK_ENOMEM;
  }
  s->center_host.assign((size_t)s->h * s->d, 0.f);
  SK_TRY(hipMemcpy(s->center, c, bytes, hipMemcpyDeviceToDevice));
  SK_TRY(hipMemcpy(s->center_host.data(), s->center, bytes, hipMemcpyDeviceToHost));
  return SK_OK;
}

int sketch_step(sk_handle s, const float* k, const float* v, const float* q, float* out,
                float* Z) {
  if (s == nullptr || k == nullptr || v == nullptr || q == nullptr || out == nullptr ||
      Z == nullptr)
    return SK_EINVAL;
  const int nt = (int)s->stiles.size();
  if ((long long)nt * s->h > 0x7fffffffLL) return SK_EINVAL;
  {
    const int rc = settle(s);
    if (rc != SK_OK) return rc;
  }
  hipEvent_t ev0, ev1;
  timing_pair(s, 2, &ev0, &ev1);
  launch_ev(sk_step_kernel, dim3((unsigned)((long long)nt * s->h)), dim3(256), 0, s->stream, ev0,
            ev1, s->state, s->XS, (const StepTile*)s->d_stiles, nt, s->d, s->dv, s->logd, k, v,
            q, s->tb, s->sparts, (const float*)s->center);
  hipError_t e1 = hipGetLastError();
  timing_done(s, 2);
  hipLaunchKernelGGL(sk_step_finish, dim3((unsigned)s->h), dim3(256), 0, s->stream, s->sparts,
                     nt, s->d, s->dv, (float)(s->count + 1), q, s->center, out, Z);
  hipError_t e2 = hipGetLastError();
  if (e1 != hipSuccess || e2 != hipSuccess) return SK_EHIP;
  s->count += 1;
  return SK_OK;
}

int sketch_timing(sk_handle s, int enable) {
  if (s == nullptr) return SK_EINVAL;
  if (enable && s->tev[0][0].empty()) {
    for (int k = 0; k < 3; ++k)
      for (int w = 0; w < 2; ++w) {
        s->tev[k][w].resize(kTimingPairs);
        for (int i = 0; i < kTimingPairs; ++i) SK_TRY(hipEventCreate(&s->tev[k][w][i]));
      }
  }
  s->timing = enable != 0;
  s->trec[0] = s->trec[1] = s->trec[2] = 0;
  return SK_OK;
}

int sketch_kernel_times(sk_handle s, int kind, float* ms, int cap, int* count) {
  if (s == nullptr || kind < 0 || kind > 2 || cap < 0 || (ms == nullptr && cap > 0))
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
  {
    const int rc = settle(s);
    if (rc != SK_OK) return rc;
  }
  if (s->layout == SK_LAYOUT_SYM) {
    const long long total = s->Dsym * (1 + s->dv) * s->h;
    const int grid = (int)std::min<long long>((total + 255) / 256, 16384);
    hipLaunchKernelGGL(sk_sym_export_kernel, dim3(grid), dim3(256), 0, s->stream, s->state,
                       s->XS, s->tb, s->Dsym, s->Rlo, s->d, s->dv, (float)s->count, dst, total);
    SK_TRY(hipGetLastError());
    return SK_OK;
  }
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
  const long long vrows = s->layout == SK_LAYOUT_SYM ? s->Dsym : s->D;
  const size_t bytes = sizeof(float) * (size_t)(vrows * (1 + s->dv) * s->h);
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
  if (rows_D) *rows_D = vrows;
  if (cols) *cols = 1 + s->dv;
  if (count) *count = s->count;
  return SK_OK;
}

}  // extern "C"

namespace {

// The exact path.  fixed == nullptr: the partials live in the kept per-(device,
// stream) buffer (or a stream-ordered allocation); otherwise in `fixed`, which
// holds fixed_floats floats, and the slice count is lowered until they fit.
int exact_run(const float* K, const float* V, int64_t n, int d, int dv, int h,
              const float* Q, int64_t m, float* out, float* Z, void* hip_stream,
              float* fixed, long long fixed_floats) {
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
  // many queries: fp32 MFMA when the rows are wide enough to fill its operands,
  // one thread per query on the VALU for d, dv <= 8 (there the value columns
  // would be padded 4x and the exponentials dominate)
  const bool use_mfma = !decode && bmax >= 16;
  // 16 value columns: the 16x16x4 kernel (no padding of the value columns), 64
  // queries per wave up to d = 32 (32 at d = 64, for registers); its buffer loads
  // address a slice with 32-bit byte offsets, so the whole KV of a head must fit
  const bool mfma16 = use_mfma && dv == 16 && d >= 16 && d <= 64 && use_exact_mfma16() &&
                      (long long)n * 4LL * bmax < (1LL << 31) - (1LL << 16);
  const bool qb4 = mfma16 && d <= 32;
  const long long per_wg = !use_mfma ? 256 : (qb4 ? 256 : SK_XQ);   // queries per workgroup
  const long long nqt = decode ? 1 : (m + per_wg - 1) / per_wg;
  // EXPSKETCH_EXACT_MINKEYS=<k> sets the fewest keys per slice, and
  // EXPSKETCH_EXACT_WGCU=<w> the long decode slices per CU (tuning aids).
  static const long long min_keys_env = [] {
    const char* v = std::getenv("EXPSKETCH_EXACT_MINKEYS");
    return v ? std::max(0LL, std::atoll(v)) : 0LL;
  }();
  static const long long wg_per_cu = [] {
    const char* v = std::getenv("EXPSKETCH_EXACT_WGCU");
    const long long x = v ? std::atoll(v) : 0LL;
    return x >= 1 ? x : 2LL;
  }();
  // Decode streams K/V once: about two long (>= 2048-key) slices per CU keep HBM
  // busiest, but never fewer slices than one per CU while slices stay >= 512
  // keys.  The batched kernel is compute-bound: more, shorter slices.
  const long long hq = h * nqt;
  long long ns;
  if (decode) {
    const long long lk = min_keys_env > 0 ? min_keys_env : 2048;
    const long long nn = n;
    const long long ns_long = std::min((wg_per_cu * di.num_cu + hq - 1) / hq, (nn + lk - 1) / lk);
    const long long ns_fill = std::min(((long long)di.num_cu + hq - 1) / hq, (nn + 511) / 512);
    ns = std::max(ns_long, ns_fill);
  } else {
    // (measured: 1024-key slices for the 16x16x4 kernel with 32 queries per wave,
    // 512 otherwise)
    const long long lk = min_keys_env > 0 ? min_keys_env : (mfma16 && !qb4 ? 1024 : 512);
    ns = std::min((8LL * di.num_cu + hq - 1) / hq, ((long long)n + lk - 1) / lk);
  }
  ns = std::max(1LL, ns);
  if (fixed != nullptr) {
    const long long per_slice = (long long)h * m * (2 + dv);
    if (per_slice > fixed_floats) return SK_ESCRATCH;
    ns = std::min(ns, fixed_floats / per_slice);
  }
  long long kps = n > 0 ? (n + ns - 1) / ns : 0;
  kps = (kps + 31) / 32 * 32;
  const int nsplit = kps > 0 ? (int)((n + kps - 1) / kps) : 1;
  const size_t pbytes = sizeof(float) * (size_t)h * m * nsplit * (2 + dv);
  // one kept partials buffer per (device, stream), held until released; the
  // lock covers the whole call, so calls from several threads on one stream do
  // not interleave their kernels on it
  std::unique_lock<std::mutex> ws_lock(g_xws_mutex, std::defer_lock);
  XwsEntry* xe = nullptr;
  float* parts = fixed;
  bool own = false;
  if (fixed == nullptr) {
    ws_lock.lock();
    rc = xws_for(dev, st, &xe);
    if (rc == SK_OK) rc = take_workspace(&xe->ws, pbytes, st, &parts, &own);
    if (rc != SK_OK) return rc;
  }
  const long long nn = n;
  const long long mm = m;
  const bool timed = fixed == nullptr && g_xtiming && g_xrec < (int)g_xev[0].size();
  hipEvent_t xev0 = timed ? g_xev[0][g_xrec] : nullptr;
  hipEvent_t xev1 = timed ? g_xev[1][g_xrec] : nullptr;
  if (decode) {
    const int mq = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8;
    dim3 grid(nsplit, h), blk(256);
#define SK_DEC(BB, MQ)                                                                \
  launch_ev(sk_exact_decode<BB, MQ>, grid, blk, 0, st, xev0, xev1, K, V, nn, d, dv, Q, mm, kps, \
            nsplit, parts)
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
  } else if (!use_mfma) {
    dim3 grid((unsigned)(nsplit * nqt), h), blk(256);
    if (bmax <= 4)
      launch_ev(sk_exact_tiled<4, 32>, grid, blk, 0, st, xev0, xev1, K, V, nn, d, dv, Q, mm, kps,
                nsplit, parts);
    else
      launch_ev(sk_exact_tiled<8, 32>, grid, blk, 0, st, xev0, xev1, K, V, nn, d, dv, Q, mm, kps,
                nsplit, parts);
  } else {
    // fp32 MFMA: queries x keys, then values x keys; value columns in blocks of 32
    dim3 grid((unsigned)(nsplit * nqt), h), blk(256);
    const int ncb = dv <= 32 ? 1 : (dv <= 64 ? 2 : 4);
#define SK_XM(DD, NC)                                                                     \
  launch_ev(sk_exact_mfma<DD, NC>, grid, blk, 0, st, xev0, xev1, K, V, nn, dv, Q, mm, kps, nsplit, \
            parts)
#define SK_XM_D(DD)                   \
  switch (ncb) {                      \
    case 1: SK_XM(DD, 1); break;      \
    case 2: SK_XM(DD, 2); break;      \
    default: SK_XM(DD, 4); break;     \
  }
#define SK_XM16(DD, QB)                                                                  \
  launch_ev(sk_exact_mfma16<DD, 16, QB>, grid, blk, 0, st, xev0, xev1, K, V, nn, Q, mm, kps, \
            nsplit, parts)
    if (mfma16) {
      switch (d) {
        case 16: SK_XM16(16, 4); break;
        case 32: SK_XM16(32, 4); break;
        default: SK_XM16(64, 2); break;
      }
    } else {
      switch (d) {
        case 4: SK_XM_D(4); break;
        case 8: SK_XM_D(8); break;
        case 16: SK_XM_D(16); break;
        case 32: SK_XM_D(32); break;
        case 64: SK_XM_D(64); break;
        default: SK_XM_D(128); break;
      }
    }
#undef SK_XM16
#undef SK_XM_D
#undef SK_XM
  }
  hipError_t e1 = hipGetLastError();
  if (timed) ++g_xrec;
  hipLaunchKernelGGL(sk_exact_combine, dim3((unsigned)(h * m)), dim3(256), 0, st, parts,
                     nsplit, mm, dv, h, out, Z);
  hipError_t e2 = hipGetLastError();
  if (xe != nullptr) release_workspace(parts, own, st);
  if (e1 != hipSuccess || e2 != hipSuccess) return SK_EHIP;
  return SK_OK;
}

std::mutex g_scratch_mutex;
std::vector<float*> g_scratch;

// The scratch array's device address on the current device (looked up on the
// first call on that device).
int scratch_on_device(float** out) {
  *out = nullptr;
  int dev = 0;
  SK_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return SK_EHIP;
    }
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return SK_OK;
}

}  // namespace

extern "C" {

int exact_attend(const float* K, const float* V, int64_t n, int d, int dv, int h,
                 const float* Q, int64_t m, float* out, float* Z, void* hip_stream) {
  return exact_run(K, V, n, d, dv, h, Q, m, out, Z, hip_stream, nullptr, 0);
}

int exact_attend_noalloc(const float* K, const float* V, int64_t n, int d, int dv, int h,
                         const float* Q, int64_t m, float* out, float* Z,
                         void* hip_stream) {
  if (!is_pow2_in(d, 4, 128) || !is_pow2_in(dv, 4, 128) || h < 1 || n < 0 || m < 0)
    return SK_EINVAL;
  if (m == 0) return SK_OK;
  if (Q == nullptr || out == nullptr || Z == nullptr || !aligned16(Q)) return SK_EINVAL;
  if (n > 0 && (K == nullptr || V == nullptr || !aligned16(K) || !aligned16(V)))
    return SK_EINVAL;
  if ((long long)h * m * (2 + dv) > kScratchFloats) return SK_ESCRATCH;
  float* buf = nullptr;
  const int rc = scratch_on_device(&buf);
  if (rc != SK_OK) return rc;
  return exact_run(K, V, n, d, dv, h, Q, m, out, Z, hip_stream, buf, kScratchFloats);
}


int exact_timing(int enable) {
  std::lock_guard<std::mutex> lock(g_xws_mutex);
  if (enable && g_xev[0].empty()) {
    for (int w = 0; w < 2; ++w) {
      g_xev[w].resize(kTimingPairsX);
      for (int i = 0; i < kTimingPairsX; ++i) SK_TRY(hipEventCreate(&g_xev[w][i]));
    }
  }
  g_xtiming = enable != 0;
  g_xrec = 0;
  return SK_OK;
}

int exact_kernel_times(float* ms, int cap, int* count) {
  if (cap < 0 || (ms == nullptr && cap > 0)) return SK_EINVAL;
  std::lock_guard<std::mutex> lock(g_xws_mutex);
  const int nrec = g_xrec;
  if (count) *count = nrec;
  if (nrec > 0) {
    SK_TRY(hipEventSynchronize(g_xev[1][nrec - 1]));
    for (int i = 0; i < nrec && i < cap; ++i)
      SK_TRY(hipEventElapsedTime(&ms[i], g_xev[0][i], g_xev[1][i]));
  }
  g_xrec = 0;
  return SK_OK;
}

int exact_release_workspaces(void) {
  std::lock_guard<std::mutex> ws_lock(g_xws_mutex);
  int cur = 0;
  SK_TRY(hipGetDevice(&cur));
  for (auto& kv : g_xws) {
    if (kv.first.first != cur) (void)hipSetDevice(kv.first.first);
    SK_TRY(hipDeviceSynchronize());             // the buffers' last uses
    free_workspace(&kv.second.ws);
  }
  g_xws.clear();
  SK_TRY(hipSetDevice(cur));
  return SK_OK;
}

}  // extern "C"
