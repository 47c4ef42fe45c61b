// Host side of libmok: argument validation, buffer layouts and the launch
// sequences behind the C ABI declared in include/mok.h. Nothing here reads
// device memory or synchronises: every count the device computes stays there.
#include <string.h>

#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mok.h"
#include "mok_device.h"
#include "mok_launch.h"

namespace {

constexpr int32_t kVersion = 100;   // 0.1.0
constexpr int kMaxE = kMaxExperts;
constexpr size_t kAlign = 256;
constexpr uint64_t kPersistWaitSeconds = 2;   // a persistent-driver wait gives up after this long

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Resolved {
  int64_t T, H, I, R;
  int E, k;
  bool mx;
  int driver;
  int M, n_slots, n_mb;
  int max_fwd_tiles, max_bwd_tiles;
};

mok_status resolve(const mok_problem* p, const mok_config* c, Resolved* r) {
  if (!p) return MOK_ERR_INVALID_ARG;
  if (p->T < 0 || p->H <= 0 || p->I <= 0 || p->E <= 0 || p->topk <= 0) return MOK_ERR_INVALID_ARG;
  if (p->topk > p->E) return MOK_ERR_INVALID_ARG;
  if (p->dtype != MOK_BF16 && p->dtype != MOK_MXFP8) return MOK_ERR_INVALID_ARG;
  if (p->E > kMaxE) return MOK_ERR_UNSUPPORTED;
  if (p->H % 128 != 0 || p->I % 128 != 0) return MOK_ERR_UNSUPPORTED;
  if (p->H > (1 << 20) || p->I > (1 << 20)) return MOK_ERR_UNSUPPORTED;
  const int64_t R = p->T * (int64_t)p->topk;
  if (R >= (int64_t)1 << 31 || R * p->H >= (int64_t)1 << 46) return MOK_ERR_UNSUPPORTED;
  mok_config d;
  memset(&d, 0, sizeof d);
  if (c) d = *c;
  if (d.minibatch_rows < 0 || d.ring_slots < 0 || d.num_cus < 0) return MOK_ERR_INVALID_ARG;
  if (!(d.capacity_multiplier == 0.0f || d.capacity_multiplier >= 1.0f)) return MOK_ERR_INVALID_ARG;
  if (d.driver < 0 || d.driver > 2) return MOK_ERR_INVALID_ARG;
  r->T = p->T; r->H = p->H; r->I = p->I; r->R = R;
  r->E = p->E; r->k = p->topk; r->mx = p->dtype == MOK_MXFP8;
  r->driver = d.driver;
  // [MoK clip] How-to item 3: size the minibatch so that each expert grouped
  // GEMM fills at least two waves of the machine, written there as
  // M >= 4*S*H/I for the pages' tiles. For this library's gate/up tiles
  // (256 rows x 256 columns of the 2I-wide gate|up output, one workgroup per
  // CU) two waves of S workgroups need M*2I/(256*256) >= 2*S, i.e.
  // M >= S*65536/I. The default takes the larger of the two bounds, rounded up
  // to a multiple of 256 rows.
  int64_t M = d.minibatch_rows;
  if (M == 0) {
    const int64_t S = d.num_cus ? d.num_cus : 256;
    const int64_t m_pages = cdiv(4 * S * p->H, p->I);
    const int64_t m_tiles = cdiv(S * 65536, p->I);
    M = cdiv(std::max(m_pages, m_tiles), 256) * 256;
  }
  if (M < 1) return MOK_ERR_INVALID_ARG;
  M = std::min<int64_t>(M, std::max<int64_t>(R, 1));
  r->M = (int)M;
  r->n_mb = (int)cdiv(R, M);
  int ns = d.ring_slots ? d.ring_slots : 4;
  ns = std::max(1, std::min(ns, std::max(r->n_mb, 1)));
  r->n_slots = ns;
  r->max_fwd_tiles = (int)(cdiv(R, kTileRowsFwd) + r->E + r->n_mb + 1);
  r->max_bwd_tiles = (int)(cdiv(R, kTileRowsBwd) + r->E + 1);
  return MOK_OK;
}

struct SchedLayout {
  size_t status, counts, offsets, perm, dest, n_fwd, fwd_tiles, mb_start, n_bwd, bwd_tiles, tok, eorder,
      chunk_counts, total;
};

SchedLayout sched_layout(const Resolved& r) {
  SchedLayout L;
  size_t o = 0;
  L.status = o;    o = align_up(o + 4);
  L.counts = o;    o = align_up(o + 4 * (size_t)r.E);
  L.offsets = o;   o = align_up(o + 4 * (size_t)(r.E + 1));
  L.perm = o;      o = align_up(o + 4 * (size_t)r.R);
  L.dest = o;      o = align_up(o + 4 * (size_t)r.R);
  L.n_fwd = o;     o = align_up(o + 4);
  L.fwd_tiles = o; o = align_up(o + sizeof(mok_tile) * (size_t)r.max_fwd_tiles);
  L.mb_start = o;  o = align_up(o + 4 * (size_t)(r.n_mb + 1));
  L.n_bwd = o;     o = align_up(o + 4);
  L.bwd_tiles = o; o = align_up(o + sizeof(mok_tile) * (size_t)r.max_bwd_tiles);
  // token of each permuted row (perm[p] / k), read by the GEMMs' row loaders
  L.tok = o;       o = align_up(o + 4 * ((size_t)r.R + kTokPad));
  // experts by descending count (ties to the lower id)
  L.eorder = o;    o = align_up(o + 4 * (size_t)r.E);
  // scratch of the build: per-chunk counts per bucket
  const int64_t chunk = mok_schedule_chunk_rows(r.R);
  L.chunk_counts = o; o = align_up(o + 4 * (size_t)((r.R + chunk - 1) / chunk) * (r.E + 1));
  L.total = o;
  return L;
}

mok_sched_ptrs sched_ptrs(const Resolved& r, void* base) {
  const SchedLayout L = sched_layout(r);
  uint8_t* b = static_cast<uint8_t*>(base);
  mok_sched_ptrs s;
  s.status = reinterpret_cast<int32_t*>(b + L.status);
  s.counts = reinterpret_cast<int32_t*>(b + L.counts);
  s.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  s.perm = reinterpret_cast<int32_t*>(b + L.perm);
  s.dest = reinterpret_cast<int32_t*>(b + L.dest);
  s.tok = reinterpret_cast<int32_t*>(b + L.tok);
  s.n_fwd_tiles = reinterpret_cast<int32_t*>(b + L.n_fwd);
  s.fwd_tiles = reinterpret_cast<mok_tile*>(b + L.fwd_tiles);
  s.mb_tile_start = reinterpret_cast<int32_t*>(b + L.mb_start);
  s.n_bwd_tiles = reinterpret_cast<int32_t*>(b + L.n_bwd);
  s.bwd_tiles = reinterpret_cast<mok_tile*>(b + L.bwd_tiles);
  s.eorder = reinterpret_cast<int32_t*>(b + L.eorder);
  return s;
}

// Workspace carve-up. Forward and backward never run inside one call, so
// they share the same bytes.
struct FwdWs {
  size_t ring_h, ring_hs, obuf, xq, xqs, ctr, total;
};
struct BwdWs {
  size_t dab, wperm, hb, dxrows;
  // MXFP8 only
  size_t dOq, dOs, dabq, dabs, dOT, dOTs, hT, hTs, dabT, dabTs, xT, xTs, koff;
  size_t total;
};

FwdWs fwd_ws(const Resolved& r) {
  FwdWs w;
  const size_t slots = (size_t)r.n_slots * r.M;
  size_t o = 0;
  w.ring_h = o;  o = align_up(o + slots * (r.mx ? r.I : 2 * r.I));
  w.ring_hs = o; o = align_up(o + (r.mx ? slots * (r.I / 32) : 0));
  w.obuf = o;    o = align_up(o + (size_t)r.R * 2 * r.H);
  w.xq = o;      o = align_up(o + (r.mx ? (size_t)r.T * r.H : 0));
  w.xqs = o;     o = align_up(o + (r.mx ? (size_t)r.T * (r.H / 32) : 0));
  // completion counters of the persistent driver (driver 2)
  w.ctr = o;     o = align_up(o + 4 * (size_t)mok_persist_counters(r.max_fwd_tiles));
  w.total = o;
  return w;
}

BwdWs bwd_ws(const Resolved& r) {
  BwdWs w;
  size_t o = 0;
  w.dab = o;    o = align_up(o + (r.mx ? 0 : (size_t)r.R * 4 * r.I));   // bf16 dA|dB (bf16 path only)
  w.wperm = o;  o = align_up(o + (r.mx ? 0 : (size_t)r.R * 4));         // w per permuted row (bf16 path only)
  w.hb = o;     o = align_up(o + (size_t)r.R * 2 * r.I);
  w.dxrows = o; o = align_up(o + (size_t)r.R * 2 * r.H);
  w.dOq = w.dOs = w.dabq = w.dabs = w.dOT = w.dOTs = w.hT = w.hTs = w.dabT = w.dabTs = w.xT = w.xTs = w.koff = 0;
  if (r.mx) {
    // token-blocked operands: KT bounds the padded token axis (each expert's
    // rows rounded up to 128)
    const size_t R = (size_t)r.R, H = (size_t)r.H, I = (size_t)r.I;
    const size_t KT = R + 128 * (size_t)r.E;
    w.dOq = o;   o = align_up(o + R * H);
    w.dOs = o;   o = align_up(o + R * (H / 32));
    w.dabq = o;  o = align_up(o + R * 2 * I);
    w.dabs = o;  o = align_up(o + R * (2 * I / 32));
    w.dOT = o;   o = align_up(o + H * KT);
    w.dOTs = o;  o = align_up(o + H * (KT / 32));
    w.hT = o;    o = align_up(o + I * KT);
    w.hTs = o;   o = align_up(o + I * (KT / 32));
    w.dabT = o;  o = align_up(o + 2 * I * KT);
    w.dabTs = o; o = align_up(o + 2 * I * (KT / 32));
    w.xT = o;    o = align_up(o + H * KT);
    w.xTs = o;   o = align_up(o + H * (KT / 32));
    w.koff = o;  o = align_up(o + 4 * ((size_t)r.E + 1 + (size_t)mok_token_blocks(r.R, r.E)));
  }
  w.total = o;
  return w;
}

size_t ws_bytes(const Resolved& r) { return std::max(fwd_ws(r).total, bwd_ws(r).total); }

// fwd_ctx: the down outputs in flat row order [R][H] and the gate/up
// pre-activations a | b [R][2I] (permuted order). The backward reads x rows
// in place, so no gathered copy of x is kept.
struct CtxLayout {
  size_t obuf, ab, total;
};
CtxLayout ctx_layout(const Resolved& r) {
  CtxLayout c;
  c.obuf = 0;
  c.ab = align_up((size_t)r.R * 2 * r.H);
  c.total = c.ab + align_up((size_t)r.R * 4 * r.I);
  return c;
}

size_t ctx_bytes(const Resolved& r) { return ctx_layout(r).total; }

// gfx950 check and compute-unit count, once per device (device properties
// only; no device memory is touched).
int g_cus[64] = {0};
int g_wclk_khz[64] = {0};   // rate of the device's 64-bit real-time counter

mok_status check_device(int* cus = nullptr, int* wclk_khz = nullptr) {
  static std::mutex mu;
  static int state[64] = {0};   // 0 unknown, 1 ok, 2 bad
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOK_ERR_DEVICE;
  std::lock_guard<std::mutex> g(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOK_ERR_DEVICE;
    state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_cus[dev] = prop.multiProcessorCount;
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
      khz = 100000;
    g_wclk_khz[dev] = khz;
  }
  if (cus) *cus = g_cus[dev];
  if (wclk_khz) *wclk_khz = g_wclk_khz[dev];
  return state[dev] == 1 ? MOK_OK : MOK_ERR_DEVICE;
}

mok_status launched(hipError_t e) { return e == hipSuccess ? MOK_OK : MOK_ERR_DEVICE; }

// Launch tracing: when on, each launch is bracketed by two events recorded on
// its stream; within one API call, consecutive launches on one stream share
// the event between them (the end of one is the start of the next), since
// nothing else is enqueued there in between. Events come from a pool that is
// reused across collections.
struct Tracer {
  std::mutex mu;
  bool on = false;
  struct Rec {
    const char* name;
    hipEvent_t a, b;
    bool shared_a;         // a is the previous record's b
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t chain = nullptr;   // end event of the last launch of the current API call
  hipStream_t chain_st = nullptr;
  hipEvent_t get() {
    hipEvent_t e = nullptr;
    if (!pool.empty()) {
      e = pool.back();
      pool.pop_back();
    } else if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      // timing-only events: no system-scope cache writeback and invalidation
      // between the traced kernels (mok_trace_collect synchronises the device)
      e = nullptr;
    }
    return e;
  }
};
Tracer g_tr;

// One per API call that launches work: no event chain crosses its boundary
// (the caller may enqueue its own work between calls).
struct TraceCall {
  TraceCall() { reset(); }
  ~TraceCall() { reset(); }
  static void reset() {
    if (!g_tr.on && !g_tr.chain) return;
    std::lock_guard<std::mutex> g(g_tr.mu);
    g_tr.chain = nullptr;
    g_tr.chain_st = nullptr;
  }
};

struct TraceScope {
  const char* name;
  hipStream_t st;
  hipEvent_t a = nullptr;
  bool shared = false;
  TraceScope(const char* n, hipStream_t s) : name(n), st(s) {
    if (!g_tr.on) return;
    std::lock_guard<std::mutex> g(g_tr.mu);
    if (g_tr.chain && g_tr.chain_st == st) {
      a = g_tr.chain;
      shared = true;
    } else {
      a = g_tr.get();
      if (a) (void)hipEventRecord(a, st);
    }
  }
  ~TraceScope() {
    if (!a) return;
    std::lock_guard<std::mutex> g(g_tr.mu);
    hipEvent_t b = g_tr.get();
    if (!b) {
      if (!shared) g_tr.pool.push_back(a);
      g_tr.chain = nullptr;
      return;
    }
    (void)hipEventRecord(b, st);
    g_tr.recs.push_back({name, a, b, shared});
    g_tr.chain = b;
    g_tr.chain_st = st;
  }
};

#define MOK_TRY(expr)                               \
  do {                                              \
    const mok_status _s = launched(expr);           \
    if (_s != MOK_OK) return _s;                    \
  } while (0)

// Launch `expr` (which enqueues one kernel on `st`) under the tracer.
#define MOK_RUN(name, expr)                         \
  do {                                              \
    TraceScope _ts(name, st);                       \
    MOK_TRY(expr);                                  \
  } while (0)

}  // namespace

// ---------------------------------------------------------------- schedule build without a caller scratch
// The per-chunk count table of the schedule build (hist -> scan -> scatter),
// for mok_build_schedule_noalloc: a static device array, one copy on every GPU
// the library runs on, held until the process ends. Its size covers every
// supported problem (at most 2048 chunks x (512 + 1) buckets of 4 bytes).
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, once per device, and kernels get that pointer.
constexpr size_t kNoAllocScratchBytes = (size_t)2048 * (kMaxE + 1) * 4;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static mok_status noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOK_ERR_DEVICE;
  std::lock_guard<std::mutex> g(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOK_ERR_DEVICE;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return MOK_OK;
}

extern "C" {

int32_t mok_version(void) { return kVersion; }

const char* mok_status_string(int32_t s) {
  switch (s) {
    case MOK_OK: return "ok";
    case MOK_ERR_INVALID_ARG: return "invalid argument";
    case MOK_ERR_UNSUPPORTED: return "unsupported problem or configuration";
    case MOK_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case MOK_ERR_DEVICE: return "device error (no gfx950 device or launch failure)";
    default: return "unknown status";
  }
}

mok_status mok_buffer_sizes(const mok_problem* problem, const mok_config* config,
                            size_t* workspace_bytes, size_t* schedule_bytes,
                            size_t* fwd_ctx_bytes) {
  Resolved r;
  const mok_status s = resolve(problem, config, &r);
  if (s != MOK_OK) return s;
  if (workspace_bytes) *workspace_bytes = ws_bytes(r);
  if (schedule_bytes) *schedule_bytes = sched_layout(r).total;
  if (fwd_ctx_bytes) *fwd_ctx_bytes = ctx_bytes(r);
  return MOK_OK;
}

mok_status mok_build_schedule_noalloc(const mok_problem* problem, const mok_config* config,
                                      const int32_t* topk_ids, void* schedule, size_t schedule_bytes,
                                      void* stream) {
  TraceCall tc;
  Resolved r;
  mok_status s = resolve(problem, config, &r);
  if (s != MOK_OK) return s;
  if (!schedule || (r.R > 0 && !topk_ids)) return MOK_ERR_INVALID_ARG;
  const SchedLayout L = sched_layout(r);
  if (schedule_bytes < L.chunk_counts) return MOK_ERR_BUFFER_TOO_SMALL;
  const int64_t chunk = mok_schedule_chunk_rows(r.R);
  const size_t need = 4 * (size_t)((r.R + chunk - 1) / chunk) * (size_t)(r.E + 1);
  if (need > kNoAllocScratchBytes) return MOK_ERR_UNSUPPORTED;
  if ((s = check_device()) != MOK_OK) return s;
  void* ptr = nullptr;
  if ((s = noalloc_scratch(&ptr)) != MOK_OK) return s;
  const mok_sched_ptrs p = sched_ptrs(r, schedule);
  hipStream_t st = (hipStream_t)stream;
  // the count table is written in full by the first launch (no clearing needed)
  MOK_RUN("schedule", mok_launch_schedule(topk_ids, p, (int)r.R, r.E, r.k, r.M, kTileRowsFwd,
                                          kTileRowsBwd, r.n_mb, r.max_fwd_tiles,
                                          r.max_bwd_tiles, static_cast<int32_t*>(ptr), st));
  return MOK_OK;
}

mok_status mok_get_schedule_layout(const mok_problem* problem, const mok_config* config,
                                   mok_schedule_layout* out) {
  if (!out) return MOK_ERR_INVALID_ARG;
  Resolved r;
  const mok_status s = resolve(problem, config, &r);
  if (s != MOK_OK) return s;
  const SchedLayout L = sched_layout(r);
  out->status = L.status; out->counts = L.counts; out->offsets = L.offsets;
  out->perm = L.perm; out->dest = L.dest; out->n_fwd_tiles = L.n_fwd;
  out->fwd_tiles = L.fwd_tiles; out->mb_tile_start = L.mb_start; out->n_bwd_tiles = L.n_bwd;
  out->bwd_tiles = L.bwd_tiles; out->total = L.total; out->arrays = L.chunk_counts;
  out->expert_order = L.eorder;
  out->minibatch_rows = r.M; out->ring_slots = r.n_slots; out->n_minibatches = r.n_mb;
  out->max_fwd_tiles = r.max_fwd_tiles; out->max_bwd_tiles = r.max_bwd_tiles;
  out->fwd_tile_rows = kTileRowsFwd; out->bwd_tile_rows = kTileRowsBwd;
  return MOK_OK;
}

mok_status mok_build_schedule(const mok_problem* problem, const mok_config* config,
                              const int32_t* topk_ids, void* schedule, size_t schedule_bytes,
                              void* stream) {
  TraceCall tc;
  Resolved r;
  mok_status s = resolve(problem, config, &r);
  if (s != MOK_OK) return s;
  if (!schedule || (r.R > 0 && !topk_ids)) return MOK_ERR_INVALID_ARG;
  if (schedule_bytes < sched_layout(r).total) return MOK_ERR_BUFFER_TOO_SMALL;
  if ((s = check_device()) != MOK_OK) return s;
  const mok_sched_ptrs p = sched_ptrs(r, schedule);
  hipStream_t st = (hipStream_t)stream;
  int32_t* chunk_counts =
      reinterpret_cast<int32_t*>(static_cast<uint8_t*>(schedule) + sched_layout(r).chunk_counts);
  MOK_RUN("schedule", mok_launch_schedule(topk_ids, p, (int)r.R, r.E, r.k, r.M, kTileRowsFwd,
                                          kTileRowsBwd, r.n_mb, r.max_fwd_tiles,
                                          r.max_bwd_tiles, chunk_counts, st));
  return MOK_OK;
}

namespace {

// The forward's kernel arguments (the schedule at sp, buffers carved from the
// workspace and fwd_ctx); x is the bf16 input (for MXFP8 the caller points
// a.x / a.xs at the quantized copy).
mok_fwd_args fwd_args(const Resolved& r, const mok_sched_ptrs& sp, uint8_t* ws, const FwdWs& W, void* fwd_ctx,
                      const mok_weights* weights, const void* x) {
  mok_fwd_args a;
  memset(&a, 0, sizeof a);
  a.T = r.T; a.H = r.H; a.I = r.I; a.E = r.E; a.topk = r.k;
  a.M = r.M; a.n_slots = r.n_slots; a.n_mb = r.n_mb;
  a.perm = sp.perm; a.tiles = sp.fwd_tiles; a.n_tiles = sp.n_fwd_tiles;
  a.mb_tile_start = sp.mb_tile_start;
  a.wg = weights->w_gate; a.wu = weights->w_up; a.wd = weights->w_down;
  a.sg = weights->s_gate; a.su = weights->s_up; a.sd = weights->s_down;
  a.tok = sp.tok;
  a.ring_h = ws + W.ring_h; a.ring_hs = ws + W.ring_hs;
  uint8_t* ctx = static_cast<uint8_t*>(fwd_ctx);
  const CtxLayout C = ctx_layout(r);
  a.obuf = reinterpret_cast<bf16_t*>(ctx ? ctx + C.obuf : ws + W.obuf);
  a.ab = ctx ? reinterpret_cast<bf16_t*>(ctx + C.ab) : nullptr;
  a.x = static_cast<const uint8_t*>(x);
  a.xs = nullptr;
  return a;
}

// Persistent-driver checks: tickets (int32) per queue stay below 2^31.
bool persist_fits(const Resolved& r, int cus, int* max_mb_tiles) {
  const int64_t ntu = cdiv(r.I, 128), ntd = cdiv(r.H, 256);
  *max_mb_tiles = (int)std::min<int64_t>(cdiv(r.M, kTileRowsFwd) + r.E + 1, r.max_fwd_tiles);
  return (int64_t)r.max_fwd_tiles * (ntu + ntd) + cus < ((int64_t)1 << 31) &&
         (int64_t)*max_mb_tiles * ntd < ((int64_t)1 << 31);
}

mok_persist_args persist_args(const Resolved& r, const mok_sched_ptrs& sp, uint8_t* ws, const FwdWs& W,
                              int max_mb_tiles, int wclk_khz) {
  mok_persist_args ps;
  ps.ctr = reinterpret_cast<int*>(ws + W.ctr);
  ps.status = sp.status;
  ps.give_up_bit = MOK_STATUS_WATCHDOG;
  ps.max_tiles = r.max_fwd_tiles;
  ps.max_mb_tiles = max_mb_tiles;
  ps.spin_limit = (uint64_t)wclk_khz * 1000ull * kPersistWaitSeconds;
  // MOK_PERSIST_SPIN_TICKS=n replaces the limit by n ticks of the real-time
  // counter (0: a wait not met at once gives up), to test the give-up path
  const char* ticks = getenv("MOK_PERSIST_SPIN_TICKS");
  if (ticks && ticks[0]) ps.spin_limit = strtoull(ticks, nullptr, 10);
  // MOK_PERSIST_AGENT_SYNC=1 selects the agent-scope synchronisation of a
  // misplaced grid on any placement (to test that path)
  const char* env = getenv("MOK_PERSIST_AGENT_SYNC");
  ps.force_agent = (env && env[0] == '1') ? 1 : 0;
  return ps;
}

}  // namespace

mok_status mok_forward(const mok_problem* problem, const mok_config* config, const void* schedule,
                       const void* x, const float* topk_w, const mok_weights* weights, void* y,
                       void* fwd_ctx, void* workspace, size_t workspace_bytes, void* stream) {
  TraceCall tc;
  Resolved r;
  mok_status s = resolve(problem, config, &r);
  if (s != MOK_OK) return s;
  if (!schedule || !weights || (r.T > 0 && (!x || !topk_w || !y))) return MOK_ERR_INVALID_ARG;
  if (!weights->w_gate || !weights->w_up || !weights->w_down) return MOK_ERR_INVALID_ARG;
  if (r.mx && (!weights->s_gate || !weights->s_up || !weights->s_down)) return MOK_ERR_INVALID_ARG;
  const FwdWs W = fwd_ws(r);
  if (!workspace || workspace_bytes < ws_bytes(r)) return MOK_ERR_BUFFER_TOO_SMALL;
  int cus = 0, wclk_khz = 0;
  if ((s = check_device(&cus, &wclk_khz)) != MOK_OK) return s;
  int max_mb_tiles = 0;
  if (r.driver == 2 && !persist_fits(r, cus, &max_mb_tiles)) return MOK_ERR_UNSUPPORTED;
  if (r.T == 0) return MOK_OK;
  hipStream_t st = (hipStream_t)stream;
  const mok_sched_ptrs sp = sched_ptrs(r, const_cast<void*>(schedule));
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  mok_fwd_args a = fwd_args(r, sp, ws, W, fwd_ctx, weights, x);

  // Dispatch: the gate/up GEMM reads each routed row's x row in place through
  // the token table. MXFP8: x is quantized once per token (blocks lie inside a
  // row, so this is bitwise the same as quantizing each gathered row) and the
  // GEMM reads the fp8 rows and their scale rows the same way.
  if (r.mx) {
    MOK_RUN("mxfp8_quantize_x", mok_launch_mxfp8_quantize(static_cast<const bf16_t*>(x), r.T, r.H,
                                                          ws + W.xq, ws + W.xqs, st));
    a.x = ws + W.xq;
    a.xs = ws + W.xqs;
  }
  if (r.driver == 2) {
    // [MoK clip] Key points bullets 3-5: one resident grid consumes the
    // minibatches in order through the ring, the stages waking each other
    // through counters (fwd_persistent_kernel; the plan in persist_plan.h).
    // The counters are cleared by a fill kernel on the same stream.
    const mok_persist_args ps = persist_args(r, sp, ws, W, max_mb_tiles, wclk_khz);
    const int grid = std::max(1, cus / 8) * 8;
    MOK_RUN("persist_clear", mok_launch_zero(ps.ctr, 4 * mok_persist_counters(r.max_fwd_tiles), st));
    MOK_RUN("persistent_fwd", mok_launch_fwd_persistent(a, ps, grid, r.mx, st));
    MOK_RUN("combine", mok_launch_combine(a.obuf, topk_w, sp.dest, sp.offsets + r.E, r.T, r.k, r.H,
                               static_cast<bf16_t*>(y), st));
    return MOK_OK;
  }
  // Minibatches go through the ring N_s at a time: the group [m0, m1) with
  // m0 a multiple of N_s occupies slots 0 .. m1-m0-1, i.e. one contiguous
  // window of the ring, so each stage is one launch per group (one launch
  // per minibatch would add a partly filled last wave per minibatch).
  for (int m0 = 0; m0 < r.n_mb; m0 += r.n_slots) {
    const int m1 = std::min(r.n_mb, m0 + r.n_slots);
    const int64_t p0 = (int64_t)m0 * r.M;
    const int64_t rows = std::min<int64_t>((int64_t)m1 * r.M, r.R) - p0;
    const int max_tiles = (int)std::min<int64_t>(cdiv(rows, kTileRowsFwd) + r.E + (m1 - m0),
                                                 r.max_fwd_tiles);
    MOK_RUN("gateup_gemm", mok_launch_gateup(a, m0, m1, max_tiles, r.mx, st));
    MOK_RUN("down_gemm", mok_launch_down(a, m0, m1, max_tiles, r.mx, st));
  }
  MOK_RUN("combine", mok_launch_combine(a.obuf, topk_w, sp.dest, sp.offsets + r.E, r.T, r.k, r.H,
                             static_cast<bf16_t*>(y), st));
  return MOK_OK;
}

mok_status mok_forward_fused(const mok_problem* problem, const mok_config* config, const int32_t* topk_ids,
                             void* schedule, size_t schedule_bytes, const void* x, const float* topk_w,
                             const mok_weights* weights, void* y, void* fwd_ctx, void* workspace,
                             size_t workspace_bytes, void* stream) {
  TraceCall tc;
  Resolved r;
  mok_status s = resolve(problem, config, &r);
  if (s != MOK_OK) return s;
  if (!schedule || !weights || (r.R > 0 && !topk_ids) || (r.T > 0 && (!x || !topk_w || !y)))
    return MOK_ERR_INVALID_ARG;
  if (!weights->w_gate || !weights->w_up || !weights->w_down) return MOK_ERR_INVALID_ARG;
  if (r.mx && (!weights->s_gate || !weights->s_up || !weights->s_down)) return MOK_ERR_INVALID_ARG;
  const SchedLayout SL = sched_layout(r);
  if (schedule_bytes < SL.total) return MOK_ERR_BUFFER_TOO_SMALL;
  const FwdWs W = fwd_ws(r);
  if (!workspace || workspace_bytes < ws_bytes(r)) return MOK_ERR_BUFFER_TOO_SMALL;
  int cus = 0, wclk_khz = 0;
  if ((s = check_device(&cus, &wclk_khz)) != MOK_OK) return s;
  int max_mb_tiles = 0;
  if (!persist_fits(r, cus, &max_mb_tiles)) return MOK_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  const mok_sched_ptrs sp = sched_ptrs(r, schedule);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(schedule) + SL.chunk_counts);
  if (r.T == 0) {
    // nothing to run but the (empty) schedule
    MOK_RUN("schedule", mok_launch_schedule(topk_ids, sp, 0, r.E, r.k, r.M, kTileRowsFwd, kTileRowsBwd,
                                            r.n_mb, r.max_fwd_tiles, r.max_bwd_tiles, chunk_counts, st));
    return MOK_OK;
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  mok_fwd_args a = fwd_args(r, sp, ws, W, fwd_ctx, weights, x);
  if (r.mx) {
    a.x = ws + W.xq;
    a.xs = ws + W.xqs;
  }
  const mok_persist_args ps = persist_args(r, sp, ws, W, max_mb_tiles, wclk_khz);
  mok_layer_args L;
  L.ids = topk_ids;
  L.s = sp;
  L.R = (int)r.R;
  L.chunk = mok_schedule_chunk_rows(r.R);
  L.nchunks = (int)cdiv(r.R, L.chunk);
  L.bh = chunk_counts;
  L.bm_f = kTileRowsFwd; L.bm_b = kTileRowsBwd;
  L.max_f = r.max_fwd_tiles; L.max_b = r.max_bwd_tiles;
  L.x = static_cast<const bf16_t*>(x);
  L.topk_w = topk_w;
  L.y = static_cast<bf16_t*>(y);
  const int grid = std::max(1, cus / 8) * 8;
  // [MoK card] "What it is", [MoK clip] Key points 4-5: schedule, dispatch,
  // expert FFN and combine in one persistent launch (layer_fwd_kernel); its
  // counters are cleared by a fill kernel on the same stream first.
  MOK_RUN("layer_clear", mok_launch_zero(ps.ctr, 4 * mok_persist_counters(r.max_fwd_tiles), st));
  MOK_RUN("layer_clear", mok_launch_zero(sp.status, 4, st));     // the scan keeps a give-up set before it
  MOK_RUN("layer_fwd", mok_launch_layer_fwd(a, ps, L, grid, r.mx, st));
  return MOK_OK;
}

mok_status mok_backward(const mok_problem* problem, const mok_config* config,
                        const void* schedule, const void* fwd_ctx, const void* x,
                        const float* topk_w, const mok_weights* weights, const void* dy, void* dx,
                        void* dw_gate, void* dw_up, void* dw_down, float* d_topk_w,
                        void* workspace, size_t workspace_bytes, void* stream) {
  TraceCall tc;
  Resolved r;
  mok_status s = resolve(problem, config, &r);
  if (s != MOK_OK) return s;
  if (!schedule || !weights || !dw_gate || !dw_up || !dw_down) return MOK_ERR_INVALID_ARG;
  if (r.T > 0 && !fwd_ctx) return MOK_ERR_INVALID_ARG;
  if (r.mx && (!weights->w_down_t || !weights->w_gu_t || !weights->s_down_t || !weights->s_gu_t))
    return MOK_ERR_INVALID_ARG;
  if (r.T > 0 && (!x || !topk_w || !dy || !dx || !d_topk_w)) return MOK_ERR_INVALID_ARG;
  if (!weights->w_gate || !weights->w_up || !weights->w_down) return MOK_ERR_INVALID_ARG;
  const BwdWs W = bwd_ws(r);
  if (!workspace || workspace_bytes < ws_bytes(r)) return MOK_ERR_BUFFER_TOO_SMALL;
  if ((s = check_device()) != MOK_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const mok_sched_ptrs sp = sched_ptrs(r, const_cast<void*>(schedule));
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const uint8_t* ctx = static_cast<const uint8_t*>(fwd_ctx);

  mok_bwd_args a;
  memset(&a, 0, sizeof a);
  a.T = r.T; a.H = r.H; a.I = r.I; a.E = r.E; a.topk = r.k;
  a.perm = sp.perm; a.offsets = sp.offsets; a.eorder = sp.eorder;
  a.tiles = sp.bwd_tiles; a.n_tiles = sp.n_bwd_tiles;
  a.max_tiles = r.max_bwd_tiles;
  a.wg = static_cast<const bf16_t*>(weights->w_gate);
  a.wu = static_cast<const bf16_t*>(weights->w_up);
  a.wd = static_cast<const bf16_t*>(weights->w_down);
  const CtxLayout C = ctx_layout(r);
  const bf16_t* obuf = reinterpret_cast<const bf16_t*>(ctx + C.obuf);
  a.ab = reinterpret_cast<const bf16_t*>(ctx + C.ab);
  a.tok = sp.tok;
  a.topk_w = topk_w;
  a.dy = static_cast<const bf16_t*>(dy);
  a.x = static_cast<const bf16_t*>(x);
  a.dab = r.mx ? nullptr : reinterpret_cast<bf16_t*>(ws + W.dab);   // bf16 path only
  float* wperm = r.mx ? nullptr : reinterpret_cast<float*>(ws + W.wperm);
  a.wperm = wperm;
  a.hb = reinterpret_cast<bf16_t*>(ws + W.hb);
  a.dxrows = reinterpret_cast<bf16_t*>(ws + W.dxrows);
  a.dwg = static_cast<bf16_t*>(dw_gate);
  a.dwu = static_cast<bf16_t*>(dw_up);
  a.dwd = static_cast<bf16_t*>(dw_down);

  if (r.mx) {
    a.wdt = static_cast<const uint8_t*>(weights->w_down_t);
    a.wdt_s = weights->s_down_t;
    a.wgut = static_cast<const uint8_t*>(weights->w_gu_t);
    a.wgut_s = weights->s_gu_t;
    a.dOq = ws + W.dOq;   a.dOs = ws + W.dOs;
    a.dabq = ws + W.dabq; a.dabs = ws + W.dabs;
    a.dOT = ws + W.dOT;   a.dOTs = ws + W.dOTs;
    a.hT = ws + W.hT;     a.hTs = ws + W.hTs;
    a.dabT = ws + W.dabT; a.dabTs = ws + W.dabTs;
    a.xT = ws + W.xT;     a.xTs = ws + W.xTs;
    a.koff = reinterpret_cast<int32_t*>(ws + W.koff);
    MOK_RUN("token_offsets", mok_launch_token_offsets(sp.offsets, r.E, r.R, a.koff, st));
    if (r.T > 0) {
      // also quantizes the dO rows along H for dh
      MOK_RUN("reverse_combine", mok_launch_reverse_combine(static_cast<const bf16_t*>(dy), obuf, topk_w, sp.dest,
                                         sp.offsets + r.E, r.T, r.k, r.H, d_topk_w, nullptr, a.dOq, a.dOs, st));
      MOK_RUN("bwd_dh_gemm", mok_launch_bwd_dh8(a, st));
      // dO rows w * dy formed from the dy rows in place (bitwise the stored rows' values)
      MOK_RUN("token_quantize_dO", mok_launch_token_quantize(static_cast<const bf16_t*>(dy), r.H, sp.perm, r.k,
                                                          topk_w, sp.offsets, a.koff, r.E, r.R, r.H,
                                                          a.dOT, a.dOTs, st));
      MOK_RUN("token_quantize_h", mok_launch_token_quantize(a.hb, r.I, nullptr, r.k, nullptr, sp.offsets, a.koff, r.E, r.R, r.I,
                                                          a.hT, a.hTs, st));
      // (dA|dB token-blocked by the dh GEMM's epilogue)
      MOK_RUN("token_quantize_x", mok_launch_token_quantize(static_cast<const bf16_t*>(x), r.H, sp.perm, r.k,
                                                          nullptr, sp.offsets, a.koff, r.E, r.R, r.H, a.xT, a.xTs, st));
    }
    MOK_RUN("bwd_dwd_gemm", mok_launch_bwd_dwd8(a, st));
    MOK_RUN("bwd_dwgu_gemm", mok_launch_bwd_dwgu8(a, st));
    if (r.T > 0) {
      MOK_RUN("bwd_dx_gemm", mok_launch_bwd_dx8(a, st));
      MOK_RUN("reverse_dispatch", mok_launch_reverse_dispatch(a.dxrows, sp.dest, sp.offsets + r.E, r.T, r.k, r.H,
                                          static_cast<bf16_t*>(dx), st));
    }
    return MOK_OK;
  }
  if (r.T > 0) {
    MOK_RUN("reverse_combine", mok_launch_reverse_combine(static_cast<const bf16_t*>(dy), obuf, topk_w, sp.dest,
                                       sp.offsets + r.E, r.T, r.k, r.H, d_topk_w, wperm, nullptr, nullptr, st));
    MOK_RUN("bwd_dh_gemm", mok_launch_bwd_dh(a, st));
  }
  MOK_RUN("bwd_dwd_gemm", mok_launch_bwd_dwd(a, st));
  MOK_RUN("bwd_dwgu_gemm", mok_launch_bwd_dwgu(a, st));
  if (r.T > 0) {
    MOK_RUN("bwd_dx_gemm", mok_launch_bwd_dx(a, st));
    MOK_RUN("reverse_dispatch", mok_launch_reverse_dispatch(a.dxrows, sp.dest, sp.offsets + r.E, r.T, r.k, r.H,
                                        static_cast<bf16_t*>(dx), st));
  }
  return MOK_OK;
}

mok_status mok_mxfp8_quantize(const void* src, int64_t rows, int64_t K, uint8_t* q,
                              uint8_t* scales, void* stream) {
  TraceCall tc;
  if (rows < 0 || K <= 0 || K % 32 != 0) return MOK_ERR_INVALID_ARG;
  if (rows > 0 && (!src || !q || !scales)) return MOK_ERR_INVALID_ARG;
  mok_status s = check_device();
  if (s != MOK_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  MOK_RUN("mxfp8_quantize", mok_launch_mxfp8_quantize(static_cast<const bf16_t*>(src), rows, K, q,
                                                      scales, st));
  return MOK_OK;
}

mok_status mok_mxfp8_quantize_transposed(const void* src, int64_t batch, int64_t rows, int64_t cols,
                                         uint8_t* q, uint8_t* scales, int64_t ld, int64_t col0,
                                         void* stream) {
  TraceCall tc;
  if (batch < 0 || rows < 0 || cols < 0 || ld < 0 || col0 < 0) return MOK_ERR_INVALID_ARG;
  if (rows % 32 != 0 || cols % 8 != 0 || ld % 32 != 0 || col0 % 32 != 0 || col0 + rows > ld)
    return MOK_ERR_INVALID_ARG;
  if (batch == 0 || rows == 0 || cols == 0) return MOK_OK;
  if (!src || !q || !scales) return MOK_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(q) % 16 != 0)
    return MOK_ERR_INVALID_ARG;
  if (batch > 65535 || (rows + 63) / 64 > 65535) return MOK_ERR_UNSUPPORTED;
  mok_status s = check_device();
  if (s != MOK_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  MOK_RUN("mxfp8_quantize_t", mok_launch_mxfp8_quantize_t(static_cast<const bf16_t*>(src), batch, rows, cols,
                                                          q, scales, ld, col0, st));
  return MOK_OK;
}

mok_status mok_probe_mfma(int32_t kind, int32_t workgroups, int32_t iters, float* sink, void* stream) {
  TraceCall tc;
  if ((kind != 0 && kind != 1) || workgroups < 0 || iters < 0) return MOK_ERR_INVALID_ARG;
  if (workgroups > 0 && iters > 0 && !sink) return MOK_ERR_INVALID_ARG;
  mok_status s = check_device();
  if (s != MOK_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  MOK_RUN(kind == 0 ? "probe_mfma_bf16" : "probe_mfma_fp8",
          mok_launch_probe_mfma(kind, workgroups, iters, sink, st));
  return MOK_OK;
}

// [MoK clip] key chart "Router picks top-k" (reading stated in include/mok.h)
mok_status mok_router_forward(const mok_problem* problem, const void* x, const float* w_router,
                              const float* bias, int32_t* topk_ids, float* topk_w, void* stream) {
  TraceCall tc;
  Resolved r;
  mok_status s = resolve(problem, nullptr, &r);
  if (s != MOK_OK) return s;
  if (r.T > 0 && (!x || !w_router || !topk_ids || !topk_w)) return MOK_ERR_INVALID_ARG;
  if (r.k > 64) return MOK_ERR_UNSUPPORTED;
  if ((s = check_device()) != MOK_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  MOK_RUN("router_forward", mok_launch_router_forward(static_cast<const bf16_t*>(x), w_router, bias, r.T,
                                                      (int)r.H, r.E, r.k, topk_ids, topk_w, st));
  return MOK_OK;
}

mok_status mok_router_backward(const mok_problem* problem, const mok_config* config, const void* schedule,
                               const void* x, const float* w_router, const int32_t* topk_ids,
                               const float* topk_w, const float* d_topk_w, float* d_sel, void* dx,
                               float* d_w_router, void* stream) {
  TraceCall tc;
  Resolved r;
  mok_status s = resolve(problem, config, &r);
  if (s != MOK_OK) return s;
  if (!schedule || !d_w_router) return MOK_ERR_INVALID_ARG;
  if (r.T > 0 && (!x || !w_router || !topk_ids || !topk_w || !d_topk_w || !d_sel || !dx))
    return MOK_ERR_INVALID_ARG;
  if ((s = check_device()) != MOK_OK) return s;
  const mok_sched_ptrs sp = sched_ptrs(r, const_cast<void*>(schedule));
  hipStream_t st = (hipStream_t)stream;
  MOK_RUN("router_backward", mok_launch_router_backward(static_cast<const bf16_t*>(x), w_router, topk_ids,
                                                        topk_w, d_topk_w, r.T, (int)r.H, r.E, r.k, sp.offsets,
                                                        sp.perm, sp.tok, d_sel, static_cast<bf16_t*>(dx),
                                                        d_w_router, st));
  return MOK_OK;
}

mok_status mok_trace_enable(int32_t on) {
  std::lock_guard<std::mutex> g(g_tr.mu);
  g_tr.on = on != 0;
  return MOK_OK;
}

mok_status mok_trace_collect(mok_trace_stat* out, int32_t capacity, int32_t* n_out) {
  if (capacity < 0 || (capacity > 0 && !out) || !n_out) return MOK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_tr.mu);
  std::vector<std::string> names;
  std::vector<mok_trace_stat> stats;
  mok_status st = MOK_OK;
  if (!g_tr.recs.empty() && hipDeviceSynchronize() != hipSuccess) st = MOK_ERR_DEVICE;
  for (const auto& rec : g_tr.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(rec.b) != hipSuccess || hipEventElapsedTime(&ms, rec.a, rec.b) != hipSuccess)
      st = MOK_ERR_DEVICE;
    size_t k = 0;
    while (k < names.size() && names[k] != rec.name) ++k;
    if (k == names.size()) {
      names.emplace_back(rec.name);
      mok_trace_stat z;
      memset(&z, 0, sizeof z);
      strncpy(z.name, rec.name, sizeof z.name - 1);
      stats.push_back(z);
    }
    stats[k].launches += 1;
    stats[k].total_ms += ms;
    stats[k].max_ms = std::max(stats[k].max_ms, (double)ms);
    if (!rec.shared_a) g_tr.pool.push_back(rec.a);
    g_tr.pool.push_back(rec.b);
  }
  g_tr.recs.clear();
  g_tr.chain = nullptr;
  g_tr.chain_st = nullptr;
  *n_out = (int32_t)stats.size();
  for (int32_t i = 0; i < capacity && i < (int32_t)stats.size(); ++i) out[i] = stats[i];
  return st;
}

}  // extern "C"
