// Host side of the tail coreset (sk_coreset.h): the Merge-and-Reduce schedule,
// block buffers and the calls declared in expsketch.h (coreset_*).
//
// Source: "Rumo a Limites Estritos para Atenção em Streaming", "Metodologia" >
// "1. Limites Superiores Algorítmicos", pillar "Construções de Coreset Baseadas
// em Discrepância" and the closing Merge-and-Reduce paragraph.
//
// The structure is a binary counter of blocks of B points per head: level l
// holds at most one block (weight 2^l); a full partial buffer enters at level 0;
// two blocks of one level (the older first) are halved into one block of the next
// level.  The host simulates the counter to list the reduces of a call in the
// order they happen (which fixes their serial numbers, hence their uniforms),
// then runs them level of dependence by level of dependence: the reduces of one
// level share launches, up to CS_MAXOPS and a Gram workspace budget at a time.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "expsketch.h"
#include "sk_coreset.h"

namespace {

#define CS_TRY(expr)                          \
  do {                                        \
    if ((expr) != hipSuccess) return SK_EHIP; \
  } while (0)

bool cs_pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }
bool cs_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Gram workspace budget of one launch of reduces (at least one reduce always fits)
constexpr size_t kGramBytes = size_t(256) << 20;
// raw blocks of one update call handled per round (bounds the live buffers)
constexpr long long kRoundBlocks = 64;
// full blocks of small calls wait, copied, until this many (or this many bytes)
// have gathered or a reader needs the coreset: the reduces of several calls then
// share launches (a call of 4096 keys alone gives four reduces, one per depth)
constexpr size_t kPendBytes = size_t(64) << 20;

}  // namespace

struct sk_coreset {
  int d = 0, dv = 0, p = 0, h = 0, B = 0;
  double c0 = 0.0;
  unsigned long long seed = 0;
  hipStream_t stream = nullptr;
  int device = 0;
  int num_cu = 256;           // compute units of the device (tail-query slicing)
  int64_t count = 0;          // points ingested per head
  int nfill = 0;              // points in the partial buffer
  long long serial = 0;       // reduces done
  // block buffers: library-owned [h][B][d] and [h][B][dv]
  std::vector<float*> bufK, bufV;
  std::vector<int> freebuf;
  int fill = -1;              // buffer of the partial block
  std::vector<int> level;     // buffer per level, -1 = empty
  std::vector<int> pending;   // full blocks not yet entered at level 0, in order
  double* inv = nullptr;      // 1/j, j < CS_NINV; then (p+1)!/(p+1+k)!
  double* gram = nullptr;     // Gram workspace
  size_t gram_bytes = 0;
  float* parts = nullptr;     // tail-query partials
  size_t parts_bytes = 0;
  hipEvent_t switch_ev = nullptr;
};

namespace {

int take_buffer(sk_coreset* c, int* out) {
  if (!c->freebuf.empty()) {
    *out = c->freebuf.back();
    c->freebuf.pop_back();
    return SK_OK;
  }
  float *k = nullptr, *v = nullptr;
  if (hipMalloc(&k, sizeof(float) * (size_t)c->h * c->B * c->d) != hipSuccess ||
      hipMalloc(&v, sizeof(float) * (size_t)c->h * c->B * c->dv) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(k);
    return SK_ENOMEM;
  }
  c->bufK.push_back(k);
  c->bufV.push_back(v);
  *out = (int)c->bufK.size() - 1;
  return SK_OK;
}

CsRef lib_ref(const sk_coreset* c, int b) {
  return CsRef{c->bufK[b], c->bufV[b], (long long)c->B * c->d, (long long)c->B * c->dv};
}

// A block in the schedule: a library buffer or a block of the caller's input.
struct Blk {
  int buf = -1;               // library buffer, or -1
  CsRef ref{};                // the rows (either kind)
  int depth = 0;              // reduces it waits for
};

struct PlannedOp {
  Blk a, b;
  int out = -1;               // library buffer of the result
  long long serial = 0;
  int depth = 0;
};

// Simulates one block entering at level l (the binary counter of the oracle's
// Merge-and-Reduce); appends the reduces it causes.  slots: the level states.
int plan_carry(sk_coreset* c, std::vector<Blk>* slots, Blk blk, int l,
               std::vector<PlannedOp>* ops) {
  for (;;) {
    if ((int)slots->size() <= l) slots->resize(l + 1);
    Blk& s = (*slots)[l];
    if (s.ref.K == nullptr) {
      s = blk;
      return SK_OK;
    }
    PlannedOp op;
    op.a = s;
    op.b = blk;
    op.serial = c->serial++;
    op.depth = 1 + std::max(s.depth, blk.depth);
    const int rc = take_buffer(c, &op.out);
    if (rc != SK_OK) return rc;
    ops->push_back(op);
    blk = Blk{op.out, lib_ref(c, op.out), op.depth};
    s = Blk{};
    ++l;
  }
}

// Runs planned reduces, depth by depth; a library input buffer returns to the
// free list once the launch that reads it is issued (the stream orders its reuse).
int run_ops(sk_coreset* c, std::vector<PlannedOp>& ops) {
  if (ops.empty()) return SK_OK;
  int maxd = 0;
  for (const PlannedOp& o : ops) maxd = std::max(maxd, o.depth);
  const size_t per_op = sizeof(double) * (size_t)c->h * c->B * c->B;
  const int cap = (int)std::max<size_t>(1, std::min<size_t>(CS_MAXOPS, kGramBytes / per_op));
  const size_t need = per_op * (size_t)std::min<size_t>(cap, ops.size());
  if (c->gram_bytes < need) {
    CS_TRY(hipStreamSynchronize(c->stream));
    (void)hipFree(c->gram);
    c->gram = nullptr;
    c->gram_bytes = 0;
    if (hipMalloc(&c->gram, need) != hipSuccess) {
      (void)hipGetLastError();
      return SK_ENOMEM;
    }
    c->gram_bytes = need;
  }
  const int nt = c->B / CS_TP;
  const long long ntiles = (long long)nt * (nt + 1) / 2;
  for (int dep = 1; dep <= maxd; ++dep) {
    std::vector<const PlannedOp*> lvl;
    for (const PlannedOp& o : ops)
      if (o.depth == dep) lvl.push_back(&o);
    for (size_t i0 = 0; i0 < lvl.size(); i0 += cap) {
      CsOps batch{};
      batch.n = (int)std::min<size_t>(cap, lvl.size() - i0);
      for (int k = 0; k < batch.n; ++k) {
        const PlannedOp& o = *lvl[i0 + k];
        batch.op[k] = CsOp{o.a.ref, o.b.ref, c->bufK[o.out], c->bufV[o.out], o.serial};
      }
      hipLaunchKernelGGL(cs_gram_kernel, dim3((unsigned)(batch.n * c->h * ntiles)), dim3(256), 0,
                         c->stream, batch, c->B, c->d, c->dv, c->p, c->h, c->inv, c->gram);
      CS_TRY(hipGetLastError());
      hipLaunchKernelGGL(cs_walk_kernel, dim3((unsigned)(batch.n * c->h)), dim3(256), 0,
                         c->stream, batch, c->B, c->d, c->dv, c->h, c->gram, c->c0, c->seed);
      CS_TRY(hipGetLastError());
      for (int k = 0; k < batch.n; ++k) {
        const PlannedOp& o = *lvl[i0 + k];
        if (o.a.buf >= 0) c->freebuf.push_back(o.a.buf);
        if (o.b.buf >= 0) c->freebuf.push_back(o.b.buf);
      }
    }
  }
  return SK_OK;
}

int copy_rows(sk_coreset* c, const CsRef& src, long long r0, int rows, int dst, int w0) {
  if (rows <= 0) return SK_OK;
  const long long total = (long long)rows * (c->d / 4 + c->dv / 4) * c->h;
  const int grid = (int)std::min<long long>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(cs_copy_rows_kernel, dim3(grid), dim3(256), 0, c->stream, src.K, src.V,
                     src.hsK, src.hsV, r0, rows, c->d, c->dv, c->bufK[dst], c->bufV[dst], c->B,
                     w0, c->h);
  CS_TRY(hipGetLastError());
  return SK_OK;
}

// Level slots of the handle as schedule blocks (library buffers, depth 0).
std::vector<Blk> slots_of(const sk_coreset* c) {
  std::vector<Blk> s(c->level.size());
  for (size_t l = 0; l < c->level.size(); ++l)
    if (c->level[l] >= 0) s[l] = Blk{c->level[l], lib_ref(c, c->level[l]), 0};
  return s;
}

// Stores the simulated slots back; a caller block left in a slot is copied into
// a library buffer first.
int store_slots(sk_coreset* c, std::vector<Blk>& slots) {
  c->level.assign(slots.size(), -1);
  for (size_t l = 0; l < slots.size(); ++l) {
    if (slots[l].ref.K == nullptr) continue;
    if (slots[l].buf < 0) {
      int b = -1;
      int rc = take_buffer(c, &b);
      if (rc == SK_OK) rc = copy_rows(c, slots[l].ref, 0, c->B, b, 0);
      if (rc != SK_OK) return rc;
      slots[l].buf = b;
    }
    c->level[l] = slots[l].buf;
  }
  return SK_OK;
}

// The pending blocks enter level 0 in order (one schedule, reduces batched by
// depth).
int flush(sk_coreset* c) {
  if (c->pending.empty()) return SK_OK;
  std::vector<Blk> slots = slots_of(c);
  std::vector<PlannedOp> ops;
  for (int b : c->pending) {
    const int rc = plan_carry(c, &slots, Blk{b, lib_ref(c, b), 0}, 0, &ops);
    if (rc != SK_OK) return rc;
  }
  c->pending.clear();
  int rc = run_ops(c, ops);
  if (rc == SK_OK) rc = store_slots(c, slots);
  return rc;
}

int pend(sk_coreset* c, int b) {
  c->pending.push_back(b);
  const size_t bytes = sizeof(float) * (size_t)c->h * c->B * (c->d + c->dv);
  if ((long long)c->pending.size() >= kRoundBlocks || c->pending.size() * bytes >= kPendBytes)
    return flush(c);
  return SK_OK;
}

// Appends n rows per head of src to the partial buffer; every full buffer joins
// the pending blocks.  With no blocks pending, rounds of kRoundBlocks whole
// blocks of the input enter level 0 in place (read from the caller's memory by
// the reduces); fewer whole blocks are copied and join the pending ones.  Blocks
// enter the binary counter in stream order either way, so every reduce gets the
// same inputs and serial number as when each block enters at once.
int append_rows(sk_coreset* c, const CsRef& src, long long n) {
  long long i = 0;
  while (i < n) {
    if (c->nfill == 0 && n - i >= c->B) {
      const long long nb = (n - i) / c->B;
      if (c->pending.empty() && nb >= kRoundBlocks) {
        std::vector<Blk> slots = slots_of(c);
        std::vector<PlannedOp> ops;
        for (long long k = 0; k < kRoundBlocks; ++k, i += c->B) {
          Blk blk{-1, CsRef{src.K + i * c->d, src.V + i * c->dv, src.hsK, src.hsV}, 0};
          const int rc = plan_carry(c, &slots, blk, 0, &ops);
          if (rc != SK_OK) return rc;
        }
        int rc = run_ops(c, ops);
        if (rc == SK_OK) rc = store_slots(c, slots);
        if (rc != SK_OK) return rc;
        continue;
      }
      int b = -1;
      int rc = take_buffer(c, &b);
      if (rc == SK_OK) rc = copy_rows(c, src, i, c->B, b, 0);
      if (rc == SK_OK) rc = pend(c, b);
      if (rc != SK_OK) return rc;
      i += c->B;
      continue;
    }
    if (c->fill < 0) {
      const int rc = take_buffer(c, &c->fill);
      if (rc != SK_OK) return rc;
    }
    const int take = (int)std::min<long long>(c->B - c->nfill, n - i);
    int rc = copy_rows(c, src, i, take, c->fill, c->nfill);
    if (rc != SK_OK) return rc;
    c->nfill += take;
    i += take;
    if (c->nfill == c->B) {
      const int b = c->fill;
      c->fill = -1;
      c->nfill = 0;
      rc = pend(c, b);
      if (rc != SK_OK) return rc;
    }
  }
  return SK_OK;
}

// Segments of the points: the partial buffer, then the levels (increasing), cut
// into slices of `slice` points for the tail query.
CsSegs segments(const sk_coreset* c, long long* npts, int slice_pts = CS_SLICE) {
  CsSegs sg{};
  long long tot = 0;
  int slice = 0;
  auto add = [&](int b, int count, float w) {
    if (count <= 0 || sg.n >= CS_MAXSEG) return;
    CsSeg& s = sg.s[sg.n++];
    s.K = c->bufK[b];
    s.V = c->bufV[b];
    s.hsK = (long long)c->B * c->d;
    s.hsV = (long long)c->B * c->dv;
    s.count = count;
    s.slice0 = slice;
    s.w = w;
    slice += (count + slice_pts - 1) / slice_pts;
    tot += count;
  };
  if (c->fill >= 0) add(c->fill, c->nfill, 1.f);
  for (size_t l = 0; l < c->level.size(); ++l)
    if (c->level[l] >= 0) add(c->level[l], c->B, std::ldexp(1.f, (int)l));
  sg.nslices = slice;
  *npts = tot;
  return sg;
}

using TailKernel = void (*)(const float*, long long, int, CsSegs, int, float*);
template <int D>
TailKernel tail_for_dv(int dv) {
  switch (dv) {
    case 4: return cs_tail_kernel<D, 4>;
    case 8: return cs_tail_kernel<D, 8>;
    case 16: return cs_tail_kernel<D, 16>;
    case 32: return cs_tail_kernel<D, 32>;
    case 64: return cs_tail_kernel<D, 64>;
    default: return cs_tail_kernel<D, 128>;
  }
}
TailKernel tail_kernel_for(int d, int dv) {
  switch (d) {
    case 4: return tail_for_dv<4>(dv);
    case 8: return tail_for_dv<8>(dv);
    case 16: return tail_for_dv<16>(dv);
    case 32: return tail_for_dv<32>(dv);
    case 64: return tail_for_dv<64>(dv);
    default: return tail_for_dv<128>(dv);
  }
}

}  // namespace

extern "C" {

int coreset_create(int d, int dv, int p, int h, int block, double c0, uint64_t seed,
                   void* hip_stream, sk_coreset_handle* out) {
  if (out == nullptr) return SK_EINVAL;
  *out = nullptr;
  if (!cs_pow2_in(d, 4, 128) || !cs_pow2_in(dv, 4, 128) || p < 0 || p > 16 || h < 1 ||
      block < 64 || block > CS_MAXB || block % 64 != 0 || !(c0 > 0.0) || !std::isfinite(c0))
    return SK_EINVAL;
  sk_coreset* c = new (std::nothrow) sk_coreset();
  if (c == nullptr) return SK_ENOMEM;
  c->d = d; c->dv = dv; c->p = p; c->h = h; c->B = block; c->c0 = c0; c->seed = seed;
  c->stream = reinterpret_cast<hipStream_t>(hip_stream);
  // 1/j for j < CS_NINV, then the tail series' coefficients (p+1)!/(p+1+k)!
  // (zero once p + 1 + k reaches CS_NINV)
  std::vector<double> inv(2 * CS_NINV, 0.0);
  inv[0] = 1.0;
  for (int j = 1; j < CS_NINV; ++j) inv[j] = 1.0 / (double)j;
  inv[CS_NINV] = 1.0;
  for (int k = 1; k < CS_NINV && p + 1 + k < CS_NINV; ++k)
    inv[CS_NINV + k] = inv[CS_NINV + k - 1] * inv[p + 1 + k];
  if (hipGetDevice(&c->device) != hipSuccess ||
      hipDeviceGetAttribute(&c->num_cu, hipDeviceAttributeMultiprocessorCount, c->device) !=
          hipSuccess ||
      hipMalloc(&c->inv, sizeof(double) * 2 * CS_NINV) != hipSuccess ||
      hipMemcpy(c->inv, inv.data(), sizeof(double) * 2 * CS_NINV, hipMemcpyHostToDevice) !=
          hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(c->inv);
    delete c;
    return SK_EHIP;
  }
  *out = c;
  return SK_OK;
}

int coreset_destroy(sk_coreset_handle c) {
  if (c == nullptr) return SK_OK;
  int rc = SK_OK;
  if (hipStreamSynchronize(c->stream) != hipSuccess) rc = SK_EHIP;
  for (float* p : c->bufK) (void)hipFree(p);
  for (float* p : c->bufV) (void)hipFree(p);
  (void)hipFree(c->inv);
  (void)hipFree(c->gram);
  (void)hipFree(c->parts);
  if (c->switch_ev != nullptr) (void)hipEventDestroy(c->switch_ev);
  delete c;
  return rc;
}

int coreset_set_stream(sk_coreset_handle c, void* hip_stream) {
  if (c == nullptr) return SK_EINVAL;
  const hipStream_t ns = reinterpret_cast<hipStream_t>(hip_stream);
  if (ns == c->stream) return SK_OK;
  if (c->switch_ev == nullptr)
    CS_TRY(hipEventCreateWithFlags(&c->switch_ev, hipEventDisableTiming));
  CS_TRY(hipEventRecord(c->switch_ev, c->stream));
  CS_TRY(hipStreamWaitEvent(ns, c->switch_ev, 0));
  c->stream = ns;
  return SK_OK;
}

int coreset_reset(sk_coreset_handle c) {
  if (c == nullptr) return SK_EINVAL;
  for (int b : c->level)
    if (b >= 0) c->freebuf.push_back(b);
  for (int b : c->pending) c->freebuf.push_back(b);
  c->pending.clear();
  c->level.clear();
  c->nfill = 0;
  c->count = 0;
  c->serial = 0;
  return SK_OK;
}

int coreset_update(sk_coreset_handle c, const float* K, const float* V, int64_t n) {
  if (c == nullptr || n < 0) return SK_EINVAL;
  if (n == 0) return SK_OK;
  if (K == nullptr || V == nullptr || !cs_aligned16(K) || !cs_aligned16(V)) return SK_EINVAL;
  const int rc = append_rows(c, CsRef{K, V, (long long)n * c->d, (long long)n * c->dv}, n);
  if (rc != SK_OK) return rc;
  c->count += n;
  return SK_OK;
}

int coreset_merge(sk_coreset_handle dst, sk_coreset_handle src) {
  if (dst == nullptr || src == nullptr || dst == src) return SK_EINVAL;
  if (dst->d != src->d || dst->dv != src->dv || dst->p != src->p || dst->h != src->h ||
      dst->B != src->B)
    return SK_EMISMATCH;
  if (src->stream != dst->stream) {
    if (src->switch_ev == nullptr)
      CS_TRY(hipEventCreateWithFlags(&src->switch_ev, hipEventDisableTiming));
    CS_TRY(hipEventRecord(src->switch_ev, src->stream));
    CS_TRY(hipStreamWaitEvent(dst->stream, src->switch_ev, 0));
  }
  // src's buffered points enter dst's buffer in order, then src's blocks carry in
  // at their own levels, lowest first; src's buffers are read, never kept.  Both
  // first take in their pending blocks.
  int rc = flush(src);
  if (rc == SK_OK) rc = flush(dst);
  if (rc != SK_OK) return rc;
  if (src->fill >= 0 && src->nfill > 0)
    rc = append_rows(dst, lib_ref(src, src->fill), src->nfill);
  if (rc == SK_OK) rc = flush(dst);
  if (rc != SK_OK) return rc;
  std::vector<Blk> slots = slots_of(dst);
  std::vector<PlannedOp> ops;
  for (size_t l = 0; l < src->level.size() && rc == SK_OK; ++l)
    if (src->level[l] >= 0)
      rc = plan_carry(dst, &slots, Blk{-1, lib_ref(src, src->level[l]), 0}, (int)l, &ops);
  if (rc == SK_OK) rc = run_ops(dst, ops);
  if (rc == SK_OK) rc = store_slots(dst, slots);
  if (rc != SK_OK) return rc;
  if (src->stream != dst->stream) {
    CS_TRY(hipEventRecord(src->switch_ev, dst->stream));
    CS_TRY(hipStreamWaitEvent(src->stream, src->switch_ev, 0));
  }
  dst->count += src->count;
  return SK_OK;
}

int coreset_info(sk_coreset_handle c, int64_t* points, int64_t* count, int64_t* reduces) {
  if (c == nullptr) return SK_EINVAL;
  const int rc = flush(c);
  if (rc != SK_OK) return rc;
  long long np = 0;
  (void)segments(c, &np);
  if (points) *points = np;
  if (count) *count = c->count;
  if (reduces) *reduces = c->serial;
  return SK_OK;
}

int coreset_export(sk_coreset_handle c, float* K, float* V, float* w) {
  if (c == nullptr || K == nullptr || V == nullptr || w == nullptr) return SK_EINVAL;
  const int rc = flush(c);
  if (rc != SK_OK) return rc;
  long long np = 0;
  const CsSegs sg = segments(c, &np);
  if (np == 0) return SK_OK;
  const long long total = (long long)c->h * np * (c->d + c->dv + 1);
  const int grid = (int)std::min<long long>((total + 255) / 256, 16384);
  hipLaunchKernelGGL(cs_export_kernel, dim3(grid), dim3(256), 0, c->stream, sg, c->d, c->dv,
                     c->h, np, K, V, w);
  CS_TRY(hipGetLastError());
  return SK_OK;
}

int coreset_query(sk_coreset_handle c, const float* Q, int64_t m, float* out, float* Z) {
  if (c == nullptr || m < 0) return SK_EINVAL;
  if (m == 0) return SK_OK;
  if (Q == nullptr || out == nullptr || Z == nullptr || !cs_aligned16(Q)) return SK_EINVAL;
  const int rc = flush(c);
  if (rc != SK_OK) return rc;
  long long np = 0;
  const long long nqt = (m + CS_QT - 1) / CS_QT;
  // slices of 512 points, shorter (down to 64) until the launch has about four
  // workgroups per CU: a decode-sized query (a few hundred queries per head) has
  // few query tiles, and one workgroup per (query tile, slice, head)
  int slice_pts = CS_SLICE;
  CsSegs sg = segments(c, &np, slice_pts);
  while (slice_pts > 64 && nqt * sg.nslices * c->h < 4LL * c->num_cu) {
    slice_pts /= 2;
    sg = segments(c, &np, slice_pts);
  }
  if (np == 0) return SK_OK;                  // no tail: the head answer stands
  if (nqt > 0x7fffffffLL || sg.nslices > 65535 || c->h > 65535) return SK_EINVAL;
  const size_t need = sizeof(float) * (size_t)c->h * m * sg.nslices * (1 + c->dv);
  if (c->parts_bytes < need) {
    CS_TRY(hipStreamSynchronize(c->stream));
    (void)hipFree(c->parts);
    c->parts = nullptr;
    c->parts_bytes = 0;
    if (hipMalloc(&c->parts, need) != hipSuccess) {
      (void)hipGetLastError();
      return SK_ENOMEM;
    }
    c->parts_bytes = need;
  }
  hipLaunchKernelGGL(tail_kernel_for(c->d, c->dv), dim3((unsigned)nqt, sg.nslices, c->h),
                     dim3(CS_QT * CS_TPQ), 0, c->stream, Q, (long long)m, c->p, sg, slice_pts,
                     c->parts);
  CS_TRY(hipGetLastError());
  hipLaunchKernelGGL(cs_tail_combine, dim3((unsigned)(c->h * m)), dim3(256), 0, c->stream,
                     c->parts, sg.nslices, (long long)m, c->dv, out, Z);
  CS_TRY(hipGetLastError());
  return SK_OK;
}

}  // extern "C"
