// Host side of the C ABI declared in include/sla.h: argument validation,
// block counts, workspace / saved-state layout and launch sequencing.
// Nothing here allocates device memory or synchronises the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "sla_device.h"
#include "sla_internal.h"

namespace sla {
namespace {

thread_local char g_last_error[512] = "";

sla_status fail(sla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Counts per row: critical rounds up, negligible rounds down (1e-6 slack for
// float noise), both in double from the float fractions.
sla_status counts(int T, float fc, float fn, int* kc, int* kn) {
  if (!(fc >= 0.f && fc <= 1.f) || !(fn >= 0.f && fn <= 1.f))
    return fail(SLA_ERR_INVALID_ARGUMENT, "fractions must lie in [0, 1] (got %g, %g)", fc, fn);
  long long c = static_cast<long long>(ceil(static_cast<double>(fc) * T - 1e-6));
  long long n = static_cast<long long>(floor(static_cast<double>(fn) * T + 1e-6));
  c = std::max(0LL, std::min<long long>(c, T));
  n = std::max(0LL, std::min<long long>(n, T));
  if (c + n > T)
    return fail(SLA_ERR_INVALID_ARGUMENT, "critical (%lld) + negligible (%lld) blocks exceed %d", c,
                n, T);
  *kc = static_cast<int>(c);
  *kn = static_cast<int>(n);
  return SLA_OK;
}

sla_status make_dims(const sla_config* cfg, Dims* d) {
  if (cfg == nullptr) return fail(SLA_ERR_INVALID_ARGUMENT, "config is NULL");
  if (cfg->batch < 1 || cfg->heads < 1)
    return fail(SLA_ERR_INVALID_ARGUMENT, "batch and heads must be >= 1");
  if (cfg->block != kBlock) return fail(SLA_ERR_UNSUPPORTED, "block must be 64 (got %d)", cfg->block);
  if (cfg->seq_len < kBlock || cfg->seq_len % kBlock != 0)
    return fail(SLA_ERR_INVALID_ARGUMENT, "seq_len must be a positive multiple of 64 (got %d)",
                cfg->seq_len);
  if (cfg->head_dim != 64 && cfg->head_dim != 128)
    return fail(SLA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", cfg->head_dim);
  const int N = cfg->seq_len;
  const int L = cfg->valid_len == 0 ? N : cfg->valid_len;
  if (L <= N - kBlock || L > N)
    return fail(SLA_ERR_INVALID_ARGUMENT, "valid_len must satisfy seq_len-64 < valid_len <= seq_len");
  const int T = N / kBlock;
  if (T > 2048) return fail(SLA_ERR_UNSUPPORTED, "seq_len above 131072 is not supported");
  if (cfg->mask_mode != SLA_MASK_COMPUTE && cfg->mask_mode != SLA_MASK_GIVEN)
    return fail(SLA_ERR_INVALID_ARGUMENT, "unknown mask_mode %d", cfg->mask_mode);
  if (!isfinite(cfg->softmax_scale))
    return fail(SLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (cfg->linear_mode != SLA_LINEAR_MARGINAL && cfg->linear_mode != SLA_LINEAR_GLOBAL)
    return fail(SLA_ERR_INVALID_ARGUMENT, "unknown linear_mode %d", cfg->linear_mode);
  const bool global = cfg->linear_mode == SLA_LINEAR_GLOBAL;
  if (global && !(cfg->linear_gate >= 0.f && cfg->linear_gate <= 1.f))
    return fail(SLA_ERR_INVALID_ARGUMENT, "linear_gate must lie in [0, 1] (got %g)", cfg->linear_gate);
  const long long elems = static_cast<long long>(cfg->batch) * cfg->heads * N;
  if (elems > (1LL << 40)) return fail(SLA_ERR_UNSUPPORTED, "problem too large");
  int kc = 0, kn = 0;
  sla_status st = counts(T, cfg->frac_critical, cfg->frac_negligible, &kc, &kn);
  if (st != SLA_OK) return st;
  d->B = cfg->batch;
  d->H = cfg->heads;
  d->N = N;
  d->D = cfg->head_dim;
  d->L = L;
  d->T = T;
  d->Tp = (T + 31) / 32 * 32;
  d->NB = d->D * d->D + 2 * d->D;
  d->kc = kc;
  d->kn = kn;
  d->km = T - kc - kn;
  d->scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / sqrtf(static_cast<float>(d->D));
  d->mask_mode = cfg->mask_mode;
  d->global = global;
  d->gate = global ? cfg->linear_gate : 1.0f;
  // two-level selection: groups of G key blocks, `keep` kept per row, the last
  // floor(k_n / G) negligible; the kept groups must hold k_c blocks even when
  // the short last group is one of them
  d->G = d->Tg = d->keep = d->ng = 0;
  if (cfg->select_group != 0) {
    const int G = cfg->select_group;
    if (G < 1 || G > T)
      return fail(SLA_ERR_INVALID_ARGUMENT, "select_group must lie in [1, T] (got %d)", G);
    const int Tg = (T + G - 1) / G;
    const int last = T - (Tg - 1) * G;
    if (cfg->select_keep < 1 || cfg->select_keep > Tg)
      return fail(SLA_ERR_INVALID_ARGUMENT, "select_keep must lie in [1, %d] (got %d)", Tg,
                  cfg->select_keep);
    if (kc > (cfg->select_keep - 1) * G + last)
      return fail(SLA_ERR_INVALID_ARGUMENT,
                  "the kept groups hold fewer than k_c = %d blocks (select_keep %d, group %d)", kc,
                  cfg->select_keep, G);
    d->G = G;
    d->Tg = Tg;
    d->keep = cfg->select_keep;
    d->ng = kn / G;
  }
  return SLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sla_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(SLA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(SLA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return SLA_OK;
}

#define SLA_CHECK(expr)              \
  do {                               \
    sla_status st_ = (expr);         \
    if (st_ != SLA_OK) return st_;   \
  } while (0)

sla_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SLA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return SLA_OK;
}

// Optional per-stage event recording.
struct Stages {
  hipEvent_t* ev;
  hipStream_t s;
  sla_status begin(int stage) {
    if (ev && hipEventRecord(ev[2 * stage], s) != hipSuccess)
      return fail(SLA_ERR_DEVICE, "hipEventRecord failed");
    return SLA_OK;
  }
  sla_status end(int stage) {
    if (ev && hipEventRecord(ev[2 * stage + 1], s) != hipSuccess)
      return fail(SLA_ERR_DEVICE, "hipEventRecord failed");
    return SLA_OK;
  }
};

}  // namespace

WorkspaceLayout workspace_layout(const Dims& d) {
  WorkspaceLayout w{};
  const size_t BH = static_cast<size_t>(d.BH());
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  w.qbar = take(BH * d.T * d.D * 4);
  w.kbar = take(BH * d.T * d.D * 4);
  w.kgbar = take(BH * (d.G > 0 ? d.Tg : 1) * d.D * 4);
  w.scores = take(BH * d.T * d.T * 4);
  w.lut = take(BH * d.T * d.T * 4);
  w.lut_cnt = take(BH * d.T * 4);
  w.col = take(BH * d.T * d.T * 4);
  w.col_cnt = take(BH * d.T * 4);
  w.rbits = take(BH * d.Tp * (d.Tp / 32) * 4);
  w.cbits = take(BH * d.Tp * (d.Tp / 32) * 4);
  w.states = take(BH * d.Tp * d.NB * 2);
  w.dstate = take(BH * d.T * d.D * d.D * 2);
  w.dstate_z = take(BH * d.T * 2 * d.D * 4);
  w.dsum = take(BH * d.N * 4);
  w.ddel = take(BH * d.N * 4);
  w.dn = take(BH * d.N * d.D * 2);
  w.wT = take(static_cast<size_t>(d.D) * d.D * 2);
  w.dw_part = take(static_cast<size_t>(kDwParts) * d.D * d.D * 4);
  w.total = off;
  return w;
}

SavedLayout saved_layout(const Dims& d) {
  SavedLayout s{};
  const size_t BH = static_cast<size_t>(d.BH());
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  s.lse = take(BH * d.N * 4);
  s.den = take(BH * d.N * 4);
  s.y = take(BH * d.N * d.D * 2);
  s.hst = take(BH * d.T * d.D * d.D * 2);
  s.zst = take(BH * d.T * 2 * d.D * 4);
  s.total = off;
  return s;
}

namespace {

sla_status check_forward_ptrs(const void* q, const void* k, const void* v, const void* w,
                              const void* o, const void* mask, const void* saved) {
  SLA_CHECK(check_ptr(q, "q"));
  SLA_CHECK(check_ptr(k, "k"));
  SLA_CHECK(check_ptr(v, "v"));
  SLA_CHECK(check_ptr(w, "w"));
  SLA_CHECK(check_ptr(o, "o"));
  SLA_CHECK(check_ptr(mask, "mask"));
  SLA_CHECK(check_ptr(saved, "saved"));
  return SLA_OK;
}

// The forward's scratch regions (a subset of the workspace).
struct FwdScratch {
  float* qbar;
  float* kbar;
  float* kgbar;
  float* scores;
  int32_t* lut;
  int32_t* lut_cnt;
  uint32_t* rbits;
  uint16_t* states;
};

// The forward's outputs: O, the mask and the regions of the saved state.
struct FwdOut {
  uint16_t* o;
  int8_t* mask;
  float* lse;
  float* den;
  uint16_t* y;
  uint16_t* hst;
  float* zst;
};

// Enqueue the whole forward for the B*H problems of d on s.
sla_status forward_run(const Dims& d, const uint16_t* q16, const uint16_t* k16,
                       const uint16_t* v16, const uint16_t* w16, const FwdOut& out,
                       const FwdScratch& fs, Stages stg, hipStream_t s) {
  int8_t* mask = out.mask;
  const bool given = d.mask_mode == SLA_MASK_GIVEN;
  // all blocks critical: plain dense attention, no classification, no linear branch
  const bool dense = !given && d.kc == d.T && !d.global;
  // (the two-level split can leave marginal blocks even when the flat one has none)
  const bool linear = d.global || given || ((d.km > 0 || d.G > 0) && d.kc < d.T);
  uint32_t* bits = d.global ? nullptr : fs.rbits;   // the global branch needs no marginal bits

  if (dense) {
    SLA_CHECK(launched(launch_fill_mask(d, mask, 1, s), "fill_mask"));
  } else {
    if (linear || !given) {
      SLA_CHECK(stg.begin(SLA_STAGE_KV_STATE));
      SLA_CHECK(launched(launch_kv_state(d, k16, v16, fs.kbar, fs.states, s), "kv_state"));
      SLA_CHECK(stg.end(SLA_STAGE_KV_STATE));
    }
    if (!given) {
      SLA_CHECK(stg.begin(SLA_STAGE_POOL_Q));
      SLA_CHECK(launched(launch_pool(d, q16, fs.qbar, s), "pool_q"));
      SLA_CHECK(stg.end(SLA_STAGE_POOL_Q));
      SLA_CHECK(stg.begin(SLA_STAGE_CLASSIFY));
      if (d.G > 0) {
        // two-level: group means of K, then coarse and candidate scores inside the classifier
        SLA_CHECK(launched(launch_group_means(d, fs.kbar, fs.kgbar, s), "group_means"));
        SLA_CHECK(launched(launch_classify_hier(d, fs.qbar, fs.kgbar, fs.kbar, nullptr, nullptr,
                                                mask, fs.lut, fs.lut_cnt, bits, s),
                           "classify_hier"));
      } else {
        SLA_CHECK(launched(launch_scores(d, fs.qbar, fs.kbar, fs.scores, s), "scores"));
        SLA_CHECK(launched(launch_classify(d, fs.scores, mask, fs.lut, fs.lut_cnt, bits, s),
                           "classify"));
      }
      SLA_CHECK(stg.end(SLA_STAGE_CLASSIFY));
    } else {
      SLA_CHECK(stg.begin(SLA_STAGE_CLASSIFY));
      SLA_CHECK(launched(launch_mask_lists(d, mask, fs.lut, fs.lut_cnt, bits, nullptr, nullptr,
                                           nullptr, s),
                         "mask_lists"));
      SLA_CHECK(stg.end(SLA_STAGE_CLASSIFY));
    }
    if (linear) {
      SLA_CHECK(stg.begin(SLA_STAGE_AGGREGATE));
      if (d.global)
        SLA_CHECK(launched(launch_state_total(d, fs.states, out.hst, out.zst, s), "state_total"));
      else
        SLA_CHECK(launched(launch_aggregate(d, fs.rbits, fs.states, out.hst, out.zst, s), "aggregate"));
      SLA_CHECK(stg.end(SLA_STAGE_AGGREGATE));
    }
  }
  SLA_CHECK(stg.begin(SLA_STAGE_ATTENTION));
  SLA_CHECK(launched(launch_attn_fwd(d, q16, k16, v16, w16, fs.lut, fs.lut_cnt, dense, linear,
                                     out.hst, out.zst, out.o, out.lse, out.den, out.y, s),
                     "attention"));
  SLA_CHECK(stg.end(SLA_STAGE_ATTENTION));
  return SLA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Allocation-free forward.  The forward's scratch lives in one fixed device
// array per GPU instead of a caller workspace; the B*H problems run in passes
// of as many (batch, head) problems as the array holds.  In host code the
// array's name only stands in for the symbol: kernels and copies get the
// device address that hipGetSymbolAddress returns for the current device,
// looked up once per device and kept in g_scratch.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[SLA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's copy of ``scratch``.
sla_status static_scratch(char** base) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SLA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SLA_ERR_UNSUPPORTED, "device %d is beyond the %d the library supports", dev,
                kMaxDevices);
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot]() {
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
  });
  if (slot.err != hipSuccess || slot.ptr == nullptr)
    return fail(SLA_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(slot.err));
  *base = static_cast<char*>(slot.ptr);
  return SLA_OK;
}

// The forward's regions for the B*H problems of d, packed (256-byte aligned).
struct FwdLayout {
  size_t qbar, kbar, kgbar, scores, lut, lut_cnt, rbits, states, total;
};
FwdLayout forward_layout(const Dims& d) {
  FwdLayout f{};
  const size_t BH = static_cast<size_t>(d.BH());
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  f.qbar = take(BH * d.T * d.D * 4);
  f.kbar = take(BH * d.T * d.D * 4);
  f.kgbar = take(BH * (d.G > 0 ? d.Tg : 1) * d.D * 4);
  f.scores = take(BH * d.T * d.T * 4);
  f.lut = take(BH * d.T * d.T * 4);
  f.lut_cnt = take(BH * d.T * 4);
  f.rbits = take(BH * d.Tp * (d.Tp / 32) * 4);
  f.states = take(BH * d.Tp * d.NB * 2);
  f.total = off;
  return f;
}

Dims with_problems(const Dims& d, int n) {
  Dims c = d;
  c.B = 1;
  c.H = n;
  return c;
}

}  // namespace

}  // namespace sla

using namespace sla;

extern "C" {

sla_status sla_block_counts(const sla_config* cfg, int32_t* k_c, int32_t* k_n, int32_t* k_m) {
  Dims d;
  SLA_CHECK(make_dims(cfg, &d));
  if (k_c) *k_c = d.kc;
  if (k_n) *k_n = d.kn;
  if (k_m) *k_m = d.km;
  return SLA_OK;
}

size_t sla_workspace_size(const sla_config* cfg) {
  Dims d;
  if (make_dims(cfg, &d) != SLA_OK) return 0;
  return workspace_layout(d).total;
}

size_t sla_saved_size(const sla_config* cfg) {
  Dims d;
  if (make_dims(cfg, &d) != SLA_OK) return 0;
  return saved_layout(d).total;
}

sla_status sla_saved_offsets(const sla_config* cfg, size_t* lse, size_t* den, size_t* y,
                             size_t* hst, size_t* zst) {
  Dims d;
  SLA_CHECK(make_dims(cfg, &d));
  const SavedLayout s = saved_layout(d);
  if (lse) *lse = s.lse;
  if (den) *den = s.den;
  if (y) *y = s.y;
  if (hst) *hst = s.hst;
  if (zst) *zst = s.zst;
  return SLA_OK;
}

sla_status sla_forward(const sla_config* cfg, const void* q, const void* k, const void* v,
                       const void* w, void* o, int8_t* mask, void* saved, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Dims d;
  SLA_CHECK(make_dims(cfg, &d));
  SLA_CHECK(check_forward_ptrs(q, k, v, w, o, mask, saved));
  SLA_CHECK(check_ptr(workspace, "workspace"));
  const WorkspaceLayout wl = workspace_layout(d);
  if (workspace_bytes < wl.total)
    return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is below the required %zu",
                workspace_bytes, wl.total);
  char* ws = static_cast<char*>(workspace);
  const FwdScratch fs{reinterpret_cast<float*>(ws + wl.qbar), reinterpret_cast<float*>(ws + wl.kbar),
                      reinterpret_cast<float*>(ws + wl.kgbar), reinterpret_cast<float*>(ws + wl.scores),
                      reinterpret_cast<int32_t*>(ws + wl.lut), reinterpret_cast<int32_t*>(ws + wl.lut_cnt),
                      reinterpret_cast<uint32_t*>(ws + wl.rbits), reinterpret_cast<uint16_t*>(ws + wl.states)};
  const SavedLayout sl = saved_layout(d);
  char* sv = static_cast<char*>(saved);
  const FwdOut out{static_cast<uint16_t*>(o), mask, reinterpret_cast<float*>(sv + sl.lse),
                   reinterpret_cast<float*>(sv + sl.den), reinterpret_cast<uint16_t*>(sv + sl.y),
                   reinterpret_cast<uint16_t*>(sv + sl.hst), reinterpret_cast<float*>(sv + sl.zst)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return forward_run(d, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(w), out, fs,
                     Stages{static_cast<hipEvent_t*>(cfg->stage_events), s}, s);
}

sla_status sla_forward_static(const sla_config* cfg, const void* q, const void* k,
                              const void* v, const void* w, void* o, int8_t* mask, void* saved,
                              void* stream) {
  Dims d;
  SLA_CHECK(make_dims(cfg, &d));
  SLA_CHECK(check_forward_ptrs(q, k, v, w, o, mask, saved));
  const long long BH = d.BH();
  const size_t one = forward_layout(with_problems(d, 1)).total;
  if (one > SLA_STATIC_SCRATCH_BYTES)
    return fail(SLA_ERR_WORKSPACE,
                "one (batch, head) problem needs %zu bytes of scratch, above the %llu of the "
                "static scratch; use sla_forward with a workspace",
                one, static_cast<unsigned long long>(SLA_STATIC_SCRATCH_BYTES));
  // problems per pass: the most whose packed regions fit the array
  long long per = std::min<long long>(BH, SLA_STATIC_SCRATCH_BYTES / one);
  while (per > 1 && forward_layout(with_problems(d, static_cast<int>(per))).total >
                        SLA_STATIC_SCRATCH_BYTES)
    --per;
  char* base = nullptr;
  SLA_CHECK(static_scratch(&base));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const SavedLayout sl = saved_layout(d);
  char* sv = static_cast<char*>(saved);
  const size_t N = d.N, D = d.D, T = d.T;
  for (long long p0 = 0; p0 < BH; p0 += per) {
    const int n = static_cast<int>(std::min(per, BH - p0));
    const Dims dc = with_problems(d, n);
    const FwdLayout fl = forward_layout(dc);
    const FwdScratch fs{reinterpret_cast<float*>(base + fl.qbar),
                        reinterpret_cast<float*>(base + fl.kbar),
                        reinterpret_cast<float*>(base + fl.kgbar),
                        reinterpret_cast<float*>(base + fl.scores),
                        reinterpret_cast<int32_t*>(base + fl.lut),
                        reinterpret_cast<int32_t*>(base + fl.lut_cnt),
                        reinterpret_cast<uint32_t*>(base + fl.rbits),
                        reinterpret_cast<uint16_t*>(base + fl.states)};
    const size_t p = static_cast<size_t>(p0);
    const FwdOut out{static_cast<uint16_t*>(o) + p * N * D, mask + p * T * T,
                     reinterpret_cast<float*>(sv + sl.lse) + p * N,
                     reinterpret_cast<float*>(sv + sl.den) + p * N,
                     reinterpret_cast<uint16_t*>(sv + sl.y) + p * N * D,
                     reinterpret_cast<uint16_t*>(sv + sl.hst) + p * T * D * D,
                     reinterpret_cast<float*>(sv + sl.zst) + p * T * 2 * D};
    SLA_CHECK(forward_run(dc, static_cast<const uint16_t*>(q) + p * N * D,
                          static_cast<const uint16_t*>(k) + p * N * D,
                          static_cast<const uint16_t*>(v) + p * N * D,
                          static_cast<const uint16_t*>(w), out, fs, Stages{nullptr, s}, s));
  }
  return SLA_OK;
}

sla_status sla_backward(const sla_config* cfg, const void* q, const void* k, const void* v,
                        const void* w, const void* o, const void* d_o, const int8_t* mask,
                        const void* saved, float* dq, float* dk, float* dv, float* dw,
                        void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  SLA_CHECK(make_dims(cfg, &d));
  SLA_CHECK(check_ptr(q, "q"));
  SLA_CHECK(check_ptr(k, "k"));
  SLA_CHECK(check_ptr(v, "v"));
  SLA_CHECK(check_ptr(w, "w"));
  SLA_CHECK(check_ptr(o, "o"));
  SLA_CHECK(check_ptr(d_o, "d_o"));
  SLA_CHECK(check_ptr(mask, "mask"));
  SLA_CHECK(check_ptr(saved, "saved"));
  SLA_CHECK(check_ptr(dq, "dq"));
  SLA_CHECK(check_ptr(dk, "dk"));
  SLA_CHECK(check_ptr(dv, "dv"));
  SLA_CHECK(check_ptr(dw, "dw"));
  SLA_CHECK(check_ptr(workspace, "workspace"));
  const WorkspaceLayout wl = workspace_layout(d);
  if (workspace_bytes < wl.total)
    return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is below the required %zu",
                workspace_bytes, wl.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Stages stg{static_cast<hipEvent_t*>(cfg->stage_events), s};
  const SavedLayout sl = saved_layout(d);
  char* ws = static_cast<char*>(workspace);
  const char* sv = static_cast<const char*>(saved);
  auto* lut = reinterpret_cast<int32_t*>(ws + wl.lut);
  auto* lut_cnt = reinterpret_cast<int32_t*>(ws + wl.lut_cnt);
  auto* col = reinterpret_cast<int32_t*>(ws + wl.col);
  auto* col_cnt = reinterpret_cast<int32_t*>(ws + wl.col_cnt);
  auto* cbits = reinterpret_cast<uint32_t*>(ws + wl.cbits);
  auto* states = reinterpret_cast<uint16_t*>(ws + wl.states);
  auto* dh = reinterpret_cast<uint16_t*>(ws + wl.dstate);
  auto* dz = reinterpret_cast<float*>(ws + wl.dstate_z);
  auto* dsum = reinterpret_cast<float*>(ws + wl.dsum);
  auto* ddel = reinterpret_cast<float*>(ws + wl.ddel);
  auto* dn = reinterpret_cast<uint16_t*>(ws + wl.dn);
  auto* wT = reinterpret_cast<uint16_t*>(ws + wl.wT);
  auto* dwp = reinterpret_cast<float*>(ws + wl.dw_part);
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  const auto* o16 = static_cast<const uint16_t*>(o);
  const auto* do16 = static_cast<const uint16_t*>(d_o);
  const auto* lse = reinterpret_cast<const float*>(sv + sl.lse);
  const auto* den = reinterpret_cast<const float*>(sv + sl.den);
  const auto* y = reinterpret_cast<const uint16_t*>(sv + sl.y);
  const auto* hst = reinterpret_cast<const uint16_t*>(sv + sl.hst);
  const auto* zst = reinterpret_cast<const float*>(sv + sl.zst);
  // the forward ran its linear branch exactly when this holds (same config)
  const bool given = d.mask_mode == SLA_MASK_GIVEN;
  const bool linear = d.global || given || ((d.km > 0 || d.G > 0) && d.kc < d.T);

  SLA_CHECK(stg.begin(SLA_STAGE_BWD_PRE));
  // (the row bits only feed the forward's aggregation: not built here)
  SLA_CHECK(launched(launch_mask_lists(d, mask, lut, lut_cnt, nullptr, col, col_cnt, cbits, s),
                     "mask_lists"));
  SLA_CHECK(launched(launch_w_transpose(d, static_cast<const uint16_t*>(w), wT, s), "w_transpose"));
  SLA_CHECK(launched(launch_bwd_prep(d, o16, do16, wT, den, y, linear, dsum, ddel, dn, dwp, s),
                     "bwd_prep"));
  if (linear) {
    SLA_CHECK(launched(launch_dstate(d, q16, dn, ddel, states, s), "dstate"));
    if (d.global)
      SLA_CHECK(launched(launch_state_total(d, states, dh, dz, s), "state_total"));
    else
      SLA_CHECK(launched(launch_aggregate(d, cbits, states, dh, dz, s), "aggregate_t"));
  }
  SLA_CHECK(stg.end(SLA_STAGE_BWD_PRE));
  SLA_CHECK(stg.begin(SLA_STAGE_BWD_KV));
  SLA_CHECK(launched(launch_bwd_kv(d, q16, k16, v16, do16, lse, dsum, col, col_cnt, dh, dz, linear,
                                   dk, dv, s),
                     "bwd_kv"));
  SLA_CHECK(stg.end(SLA_STAGE_BWD_KV));
  SLA_CHECK(stg.begin(SLA_STAGE_BWD_Q));
  SLA_CHECK(launched(launch_bwd_q(d, q16, k16, v16, do16, lse, dsum, lut, lut_cnt, dn, ddel, hst,
                                  zst, linear, dq, s),
                     "bwd_q"));
  SLA_CHECK(launched(launch_dw_reduce(d, dwp, dw, s), "dw_reduce"));
  SLA_CHECK(stg.end(SLA_STAGE_BWD_Q));
  return SLA_OK;
}

sla_status sla_pool_scores(const sla_config* cfg, const void* q, const void* k, float* scores,
                           void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  SLA_CHECK(make_dims(cfg, &d));
  SLA_CHECK(check_ptr(q, "q"));
  SLA_CHECK(check_ptr(k, "k"));
  SLA_CHECK(check_ptr(scores, "scores"));
  SLA_CHECK(check_ptr(workspace, "workspace"));
  const WorkspaceLayout wl = workspace_layout(d);
  if (workspace_bytes < wl.total)
    return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is below the required %zu",
                workspace_bytes, wl.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto* qbar = reinterpret_cast<float*>(ws + wl.qbar);
  auto* kbar = reinterpret_cast<float*>(ws + wl.kbar);
  SLA_CHECK(launched(launch_pool(d, static_cast<const uint16_t*>(q), qbar, s), "pool_q"));
  SLA_CHECK(launched(launch_pool(d, static_cast<const uint16_t*>(k), kbar, s), "pool_k"));
  SLA_CHECK(launched(launch_scores(d, qbar, kbar, scores, s), "scores"));
  return SLA_OK;
}

sla_status sla_classify(const sla_config* cfg, const float* scores, int8_t* mask, void* stream) {
  Dims d;
  SLA_CHECK(make_dims(cfg, &d));
  SLA_CHECK(check_ptr(scores, "scores"));
  SLA_CHECK(check_ptr(mask, "mask"));
  return launched(launch_classify(d, scores, mask, nullptr, nullptr, nullptr,
                                  static_cast<hipStream_t>(stream)),
                  "classify");
}

sla_status sla_coarse_scores(const sla_config* cfg, const void* q, const void* k, float* coarse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  SLA_CHECK(make_dims(cfg, &d));
  if (d.G == 0) return fail(SLA_ERR_INVALID_ARGUMENT, "select_group is 0 (flat selection)");
  SLA_CHECK(check_ptr(q, "q"));
  SLA_CHECK(check_ptr(k, "k"));
  SLA_CHECK(check_ptr(coarse, "coarse"));
  SLA_CHECK(check_ptr(workspace, "workspace"));
  const WorkspaceLayout wl = workspace_layout(d);
  if (workspace_bytes < wl.total)
    return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is below the required %zu",
                workspace_bytes, wl.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto* qbar = reinterpret_cast<float*>(ws + wl.qbar);
  auto* kbar = reinterpret_cast<float*>(ws + wl.kbar);
  auto* kgbar = reinterpret_cast<float*>(ws + wl.kgbar);
  SLA_CHECK(launched(launch_pool(d, static_cast<const uint16_t*>(q), qbar, s), "pool_q"));
  SLA_CHECK(launched(launch_pool(d, static_cast<const uint16_t*>(k), kbar, s), "pool_k"));
  SLA_CHECK(launched(launch_group_means(d, kbar, kgbar, s), "group_means"));
  return launched(launch_coarse_scores(d, qbar, kgbar, coarse, s), "coarse_scores");
}

sla_status sla_classify_hier(const sla_config* cfg, const float* coarse, const float* scores,
                             int8_t* mask, void* stream) {
  Dims d;
  SLA_CHECK(make_dims(cfg, &d));
  if (d.G == 0) return fail(SLA_ERR_INVALID_ARGUMENT, "select_group is 0 (flat selection)");
  SLA_CHECK(check_ptr(coarse, "coarse"));
  SLA_CHECK(check_ptr(scores, "scores"));
  SLA_CHECK(check_ptr(mask, "mask"));
  return launched(launch_classify_hier(d, nullptr, nullptr, nullptr, coarse, scores, mask, nullptr,
                                       nullptr, nullptr, static_cast<hipStream_t>(stream)),
                  "classify_hier");
}

const char* sla_status_string(sla_status status) {
  switch (status) {
    case SLA_OK: return "ok";
    case SLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SLA_ERR_WORKSPACE: return "workspace too small";
    case SLA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* sla_last_error(void) { return g_last_error; }

}  // extern "C"
