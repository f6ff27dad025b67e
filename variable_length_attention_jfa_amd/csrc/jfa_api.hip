// C-ABI layer of libjfa.so: argument validation, workspace layout, launches.
// Declarations and the contract are in include/jfa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>
#include <vector>
#include <string>

#include "jfa.h"
#include "jfa_common.h"
#include "jfa_kernels.h"

static_assert(sizeof(jfa::PlanHeader) == JFA_PLAN_HEADER_BYTES, "work-list header layout published in jfa.h");
static_assert(jfa::kPlanQueues == JFA_PLAN_QUEUES, "queue count published in jfa.h");

namespace {

using jfa::PlanHeader;

thread_local std::string g_last_error;

jfa_status fail(jfa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

jfa_status ok() {
  g_last_error.clear();
  return JFA_OK;
}

struct DeviceInfo {
  int num_cus = 0;
  bool gfx950 = false;
  hipError_t err = hipSuccess;
};

constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

jfa_status device_info(DeviceInfo** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(JFA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(JFA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t p;
    g_dev[dev].err = hipGetDeviceProperties(&p, dev);
    if (g_dev[dev].err == hipSuccess) {
      g_dev[dev].num_cus = p.multiProcessorCount;
      g_dev[dev].gfx950 = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    }
  });
  DeviceInfo* d = &g_dev[dev];
  if (d->err != hipSuccess) return fail(JFA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(d->err));
  if (!d->gfx950) return fail(JFA_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X)", dev);
  *out = d;
  return JFA_OK;
}

// Optional per-launch timing: HIP events recorded on the launch stream around
// each kernel, read back on jfa_timing_collect().
enum { kKindPlan = 0, kKindFwd = 1, kKindBwdPrep = 2, kKindDkdv = 3, kKindDq = 4, kKindScan = 5, kKindSq = 6, kKindFsq = 7,
       kKindDbias = 8 };
static_assert(kKindDbias + 1 == JFA_TIMING_KINDS, "timing kinds published in the header");
struct TimingRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_tmu;
std::atomic<bool> g_timing{false};
std::vector<TimingRec> g_recs;

std::vector<hipEvent_t> g_event_pool;  // reused events (creation is the costly part)

hipError_t take_event(hipEvent_t* ev) {
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (!g_event_pool.empty()) {
      *ev = g_event_pool.back();
      g_event_pool.pop_back();
      return hipSuccess;
    }
  }
  return hipEventCreate(ev);
}

template <typename F>
hipError_t timed(int kind, hipStream_t st, F&& launch) {
  if (!g_timing.load(std::memory_order_relaxed)) return launch();
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = take_event(&a);
  if (e == hipSuccess) e = take_event(&b);
  if (e == hipSuccess) e = hipEventRecord(a, st);
  if (e != hipSuccess) return e;
  e = launch();
  hipError_t e2 = hipEventRecord(b, st);
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_recs.push_back({kind, a, b});
  }
  return e != hipSuccess ? e : e2;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_sizes(int B, int H, int64_t tq, int64_t tk, int D) {
  return B >= 0 && B <= JFA_MAX_BATCH && H >= 1 && H <= JFA_MAX_HEADS && tq >= 0 && tk >= 0 && tq < (1LL << 31) && tk < (1LL << 31) &&
         (D == 32 || D == 64 || D == 128);
}

// Upper bound on the work items of one pass: sum_b ceil(L_b / tile) <= ceil(T / tile) + B.
int64_t max_items(int B, int H, int64_t total, int tile) { return (int64_t)H * (cdiv64(total, tile) + B); }

// Forward workspace: two list headers (query tiles, short-query chunks), the
// two item lists, the short-query group table [B*H] and per short-query item
// its [64, D] fp32 rows and [64] log2 row sums.
struct FwdLayout {
  size_t hdr = 0, hdr_sq = sizeof(PlanHeader), items = 0, items_sq = 0, gfirst = 0, op = 0, lsep = 0, total = 0;
  int64_t cap = 0, cap_sq = 0;
};
// short_on = false: a layout without the short-query regions (their pass does
// not run), for callers that know it, such as jfa_fwd_noalloc.
FwdLayout fwd_layout(int B, int H, int64_t tq, int64_t tk, int D, bool short_on = true) {
  FwdLayout L;
  L.cap = max_items(B, H, tq, 128);  // smallest forward tile: an upper bound for every variant
  L.cap_sq = short_on ? max_items(B, H, tk, jfa::kSqKC) : 0;
  L.items = 2 * sizeof(PlanHeader);
  L.items_sq = L.items + align_up((size_t)L.cap * 16);
  L.gfirst = L.items_sq + align_up((size_t)L.cap_sq * 16);
  L.op = L.gfirst + align_up((size_t)B * H * 4);
  L.lsep = L.op + align_up((size_t)L.cap_sq * jfa::kSqQMax * D * 4);
  L.total = L.lsep + align_up((size_t)L.cap_sq * jfa::kSqQMax * 4);
  return L;
}

// Backward workspace: three list headers (dK/dV, dQ, short-query passes), the
// row constants [Tq, H] (lse * log2 e, Delta), the three item lists, the
// short-query and dK/dV group tables [B*H], one [64, D] fp32 partial dQ per
// short-query item, the 257 bias-gradient bins of every dK/dV and
// short-query item, and their sums per (block of 4 sequences, head).
struct BwdLayout {
  size_t hdr_kv = 0, hdr_q = sizeof(PlanHeader), hdr_sq = 2 * sizeof(PlanHeader), rowc = 0, items_kv = 0,
         items_q = 0, items_sq = 0, gfirst = 0, gfirst_kv = 0, dqp = 0, dbp_kv = 0, dbp_sq = 0, dbpart = 0, dqacc = 0,
         total = 0;
  int64_t cap_kv = 0, cap_q = 0, cap_sq = 0;
};
BwdLayout bwd_layout(int B, int H, int64_t tq, int64_t tk, int D) {
  BwdLayout L;
  L.cap_kv = max_items(B, H, tk, jfa::kDkvTN);
  L.cap_q = max_items(B, H, tq, jfa::kDqTM);
  L.cap_sq = max_items(B, H, tk, jfa::kSqKC);  // sum_b max(1, ceil(Lk_b / KC)) <= ceil(Tk / KC) + B
  L.rowc = 3 * sizeof(PlanHeader);
  L.items_kv = L.rowc + align_up((size_t)tq * H * 8);
  L.items_q = L.items_kv + align_up((size_t)L.cap_kv * 16);
  L.items_sq = L.items_q + align_up((size_t)L.cap_q * 16);
  L.gfirst = L.items_sq + align_up((size_t)L.cap_sq * 16);
  L.gfirst_kv = L.gfirst + align_up((size_t)B * H * 4);
  L.dqp = L.gfirst_kv + align_up((size_t)B * H * 4);
  L.dbp_kv = L.dqp + align_up((size_t)L.cap_sq * jfa::kSqQMax * D * 4);
  L.dbp_sq = L.dbp_kv + align_up((size_t)L.cap_kv * JFA_BIAS_LEN * 4);
  L.dbpart = L.dbp_sq + align_up((size_t)L.cap_sq * JFA_BIAS_LEN * 4);
  L.dqacc = L.dbpart + align_up((size_t)((B + jfa::kDbSeqBlock - 1) / jfa::kDbSeqBlock) * H * JFA_BIAS_LEN * 4);
  // study builds that fuse dQ into the dK/dV pass (rows of up to 128 bytes):
  // an fp32 accumulator, or one partial plane per key tile (at most
  // ceil(Tk / 128) tiles in any sequence)
  const int mode = jfa::bwd_dq_mode(false, D) ? jfa::bwd_dq_mode(false, D) : jfa::bwd_dq_mode(true, D);
  const size_t plane = align_up((size_t)tq * H * D * 4);
  L.total = L.dqacc + (mode == 1 ? plane : mode == 2 ? plane * (size_t)cdiv64(tk, jfa::kDkvTN) : 0);
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The short-query passes run unless the caller's bound on every sequence's key
// count rules them out (no sequence can have more than kSqKC keys). Without
// them every sequence takes the query-tile and key-tile passes, which are
// exact for any lengths, so a wrong bound costs speed, never correctness.
bool short_pass_on(int max_kv_len) { return !(max_kv_len > 0 && max_kv_len <= jfa::kSqKC); }

jfa_status check_common(const void* q, const void* k, const void* v, const int32_t* qo, const int32_t* ko, int B,
                        int H, int D, int64_t tq, int64_t tk, int max_kv_len, const float* bias, const void* ws) {
  if (max_kv_len < 0) return fail(JFA_ERR_INVALID_ARGUMENT, "max_kv_len must be >= 0 (0: unknown)");
  if (!valid_sizes(B, H, tq, tk, D))
    return fail(JFA_ERR_INVALID_ARGUMENT, "invalid sizes: B=%d (0..%d), H=%d (1..%d), D=%d (32/64/128), total_q=%lld, total_kv=%lld",
                B, JFA_MAX_BATCH, H, JFA_MAX_HEADS, D, (long long)tq, (long long)tk);
  if (!qo || !ko) return fail(JFA_ERR_INVALID_ARGUMENT, "offsets must not be NULL");
  if ((tq > 0 && !q) || (tk > 0 && (!k || !v)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "q/k/v must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(JFA_ERR_INVALID_ARGUMENT, "q/k/v must be 16-byte aligned");
  if (!aligned(qo, 4) || !aligned(ko, 4) || !aligned(bias, 4))
    return fail(JFA_ERR_INVALID_ARGUMENT, "offsets/bias must be 4-byte aligned");
  if (!ws || !aligned(ws, kAlign)) return fail(JFA_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  return JFA_OK;
}

// pad_kv_len: non-null only for the padded-dense baseline (uniform slot
// offsets in qo/ko, true key counts in pad_kv_len); it takes neither the
// short-query passes nor the subtraction of pad terms.
jfa_status fwd_impl(bool f32, const void* q, const void* k, const void* v, const int32_t* qo, const int32_t* ko,
                    int B, int H, int D, int64_t tq, int64_t tk, int max_kv_len, const float* bias, int causal,
                    void* out, float* lse, void* ws, size_t ws_bytes, void* stream, const int32_t* pad_kv_len = nullptr,
                    bool compact = false) {
  jfa_status s = check_common(q, k, v, qo, ko, B, H, D, tq, tk, max_kv_len, bias, ws);
  if (s != JFA_OK) return s;
  if (f32 && D > 64) return fail(JFA_ERR_UNSUPPORTED, "fp32 tensors support D = 32 or 64");
  if ((tq > 0 && (!out || !lse))) return fail(JFA_ERR_INVALID_ARGUMENT, "out/lse must not be NULL");
  if (!aligned(out, 16) || !aligned(lse, 4)) return fail(JFA_ERR_INVALID_ARGUMENT, "out must be 16-byte aligned");
  // compact: the short-query regions only when that pass runs (the caller
  // sized the workspace for this call, not by jfa_fwd_workspace_bytes)
  const FwdLayout L = fwd_layout(B, H, tq, tk, D, !compact || (short_pass_on(max_kv_len) && !pad_kv_len));
  if (ws_bytes < L.total)
    return fail(JFA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  DeviceInfo* dev = nullptr;
  if ((s = device_info(&dev)) != JFA_OK) return s;
  if (B == 0 || tq == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;

  jfa::PlanArgs pa{};
  pa.q_off = qo;
  pa.kv_off = ko;
  pa.B = B;
  pa.H = H;
  pa.causal = causal ? 1 : 0;
  const bool short_on = short_pass_on(max_kv_len) && !pad_kv_len;
  pa.pass[0] = {(int4*)(w + L.items), (PlanHeader*)(w + L.hdr), (long)L.cap, jfa::fwd_tile_rows(f32, D, pad_kv_len != nullptr), jfa::fwd_tile_keys(f32, D),
                jfa::kPassQ, jfa::kPlanQueues, short_on ? jfa::kSqQMax : -1, nullptr};
  pa.pass[1] = {(int4*)(w + L.items_sq), (PlanHeader*)(w + L.hdr_sq), (long)L.cap_sq, jfa::kSqQMax, jfa::kSqKC,
                jfa::kPassSQ, jfa::kPlanQueues, -1, (int*)(w + L.gfirst)};
  hipError_t e = timed(kKindPlan, st, [&] { return jfa::launch_plan(pa, short_on ? 2 : 1, st); });
  if (e != hipSuccess) return fail(JFA_ERR_HIP, "plan launch: %s", hipGetErrorString(e));

  jfa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_off = qo;
  a.kv_off = ko;
  a.bias = bias;
  a.out = out;
  a.lse = lse;
  a.items = (const int4*)(w + L.items);
  a.hdr = (PlanHeader*)(w + L.hdr);
  a.H = H;
  a.causal = causal ? 1 : 0;
  a.scale2 = (float)(1.0 / std::sqrt((double)D) * 1.4426950408889634);
  a.B = B;
  a.gfirst = short_on ? (int*)(w + L.gfirst) : nullptr;
  a.op = (float*)(w + L.op);
  a.lsep = (float*)(w + L.lsep);
  a.kv_len = pad_kv_len;
  jfa::FwdArgs a_sq = a;
  a_sq.items = (const int4*)(w + L.items_sq);
  a_sq.hdr = (PlanHeader*)(w + L.hdr_sq);
  const bool has_bias = bias != nullptr;
  // Short-query chunks first: the query-tile launch then combines them.
  if (short_on)
    e = timed(kKindFsq, st, [&] { return jfa::launch_fsq(f32, D, a_sq, has_bias, (long)L.cap_sq, dev->num_cus, st); });
  if (e == hipSuccess)
    e = timed(kKindFwd, st, [&] {
      return pad_kv_len ? jfa::launch_fwd_padded(D, a, has_bias, (long)L.cap, dev->num_cus, st)
                        : jfa::launch_fwd(f32, D, a, has_bias, (long)L.cap, dev->num_cus, st);
    });
  if (e != hipSuccess) return fail(JFA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return ok();
}

jfa_status bwd_impl(bool f32, const void* q, const void* k, const void* v, const void* out, const float* lse,
                    const void* dout, const int32_t* qo, const int32_t* ko, int B, int H, int D, int64_t tq,
                    int64_t tk, int max_kv_len, const float* bias, int causal, void* dq, void* dk, void* dv,
                    float* dbias, void* ws, size_t ws_bytes, void* stream, const int32_t* pad_kv_len = nullptr) {
  const bool padded = pad_kv_len != nullptr;
  jfa_status s = check_common(q, k, v, qo, ko, B, H, D, tq, tk, max_kv_len, bias, ws);
  if (s != JFA_OK) return s;
  if (f32 && D > 64) return fail(JFA_ERR_UNSUPPORTED, "fp32 tensors support D = 32 or 64");
  if (tq > 0 && (!out || !lse || !dout || !dq)) return fail(JFA_ERR_INVALID_ARGUMENT, "out/lse/dout/dq must not be NULL");
  if (tk > 0 && (!dk || !dv)) return fail(JFA_ERR_INVALID_ARGUMENT, "dk/dv must not be NULL");
  if (dbias && !bias) return fail(JFA_ERR_INVALID_ARGUMENT, "dbias needs a bias");
  if (!aligned(dbias, 4)) return fail(JFA_ERR_INVALID_ARGUMENT, "dbias must be 4-byte aligned");
  if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return fail(JFA_ERR_INVALID_ARGUMENT, "out/dout/dq/dk/dv must be 16-byte aligned");
  const BwdLayout L = bwd_layout(B, H, tq, tk, D);
  if (ws_bytes < L.total)
    return fail(JFA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  DeviceInfo* dev = nullptr;
  if ((s = device_info(&dev)) != JFA_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (B == 0 || (tq == 0 && tk == 0)) {
    if (!dbias) return ok();
    jfa::BwdArgs z{};  // no pairs: the bias gradient is zero (no sequence is read)
    z.H = H;
    z.dbias = dbias;
    const hipError_t e = timed(kKindDbias, st, [&] { return jfa::launch_dbias(z, st); });
    return e == hipSuccess ? ok() : fail(JFA_ERR_HIP, "bias gradient launch: %s", hipGetErrorString(e));
  }
  char* w = (char*)ws;

  jfa::PlanArgs pa{};
  pa.q_off = qo;
  pa.kv_off = ko;
  pa.B = B;
  pa.H = H;
  pa.causal = causal ? 1 : 0;
  const bool short_on = short_pass_on(max_kv_len) && !padded;
  const int short_q = short_on ? jfa::kSqQMax : -1;
  // study builds with dQ fused into the dK/dV pass: the dQ pass gets no items
  // (its launch still sums the short-query partial dQ)
  const int dq_mode = jfa::bwd_dq_mode(f32, D);
  pa.pass[0] = {(int4*)(w + L.items_kv), (PlanHeader*)(w + L.hdr_kv), (long)L.cap_kv, jfa::dkv_tile_rows(f32, D),
                jfa::kDkvTN, jfa::kPassKV, jfa::kPlanQueues, short_q, (int*)(w + L.gfirst_kv)};
  pa.pass[1] = {(int4*)(w + L.items_q), (PlanHeader*)(w + L.hdr_q), dq_mode ? 0L : (long)L.cap_q, jfa::kDqTM,
                jfa::kDqTN, jfa::kPassQ, jfa::kPlanQueues, short_q, nullptr};
  pa.pass[2] = {(int4*)(w + L.items_sq), (PlanHeader*)(w + L.hdr_sq), (long)L.cap_sq, jfa::kSqQMax, jfa::kSqKC,
                jfa::kPassSQ, jfa::kPlanQueues, -1, (int*)(w + L.gfirst)};
  jfa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.dout = dout;
  a.q_off = qo;
  a.kv_off = ko;
  a.bias = bias;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.rowc = (float2*)(w + L.rowc);
  a.H = H;
  a.causal = causal ? 1 : 0;
  a.scale = (float)(1.0 / std::sqrt((double)D));
  a.scale2 = (float)(1.0 / std::sqrt((double)D) * 1.4426950408889634);
  a.tq = (long)tq;
  a.B = B;
  a.gfirst = short_on ? (int*)(w + L.gfirst) : nullptr;
  a.dqp = (float*)(w + L.dqp);
  a.gfirst_kv = (int*)(w + L.gfirst_kv);
  a.dbp_kv = (float*)(w + L.dbp_kv);
  a.dbp_sq = (float*)(w + L.dbp_sq);
  a.dbpart = (float*)(w + L.dbpart);
  a.dbias = dbias;
  a.kv_len = pad_kv_len;
  a.dqacc = dq_mode ? (float*)(w + L.dqacc) : nullptr;
  jfa::BwdArgs a_kv = a, a_q = a, a_sq = a;
  a_kv.items = (const int4*)(w + L.items_kv);
  a_kv.hdr = (PlanHeader*)(w + L.hdr_kv);
  a_q.items = (const int4*)(w + L.items_q);
  a_q.hdr = (PlanHeader*)(w + L.hdr_q);
  a_sq.items = (const int4*)(w + L.items_sq);
  a_sq.hdr = (PlanHeader*)(w + L.hdr_sq);
  const bool has_bias = bias != nullptr;
  // The work lists and Delta (one launch), then the short-query chunks (their
  // partial dQ is summed at the start of the dQ launch), then the split
  // passes.
  hipError_t e = timed(kKindBwdPrep, st, [&] { return jfa::launch_bwd_prep(pa, short_on ? 3 : 2, f32, D, a_kv, st); });
  if (e == hipSuccess && short_on)
    e = timed(kKindSq, st, [&] {
      return jfa::launch_sq(f32, D, a_sq, has_bias, dbias != nullptr, (long)L.cap_sq, dev->num_cus, st);
    });
  if (e == hipSuccess && dq_mode == 1)
    e = timed(kKindDkdv, st, [&] { return jfa::launch_dqacc_zero(a.dqacc, (long)tq * H * D, st); });
  if (e == hipSuccess)
    e = timed(kKindDkdv, st, [&] {
      return jfa::launch_dkdv(f32, D, a_kv, has_bias, dbias != nullptr, (long)L.cap_kv, dev->num_cus, st);
    });
  if (e == hipSuccess && dq_mode)
    e = timed(kKindDq, st, [&] { return jfa::launch_dq_fused_out(f32, D, a, st); });
  if (e == hipSuccess)
    e = timed(kKindDq, st, [&] { return jfa::launch_dq(f32, D, a_q, has_bias, (long)L.cap_q, dev->num_cus, st); });
  if (e == hipSuccess && dbias) e = timed(kKindDbias, st, [&] { return jfa::launch_dbias(a, st); });
  if (e != hipSuccess) return fail(JFA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return ok();
}

// Padded-dense baseline: B fixed-length slots of q_slot query rows and
// kv_slot key rows. Workspace: the slots' offsets [B+1] x 2, then the
// forward's or the backward's workspace for the padded totals.
bool padded_sizes_ok(int B, int H, int64_t q_slot, int64_t kv_slot, int D) {
  return q_slot >= 0 && kv_slot >= 0 && B >= 0 && (int64_t)B * q_slot < (1LL << 31) &&
         (int64_t)B * kv_slot < (1LL << 31) && valid_sizes(B, H, (int64_t)B * q_slot, (int64_t)B * kv_slot, D);
}
size_t padded_offsets_bytes(int B) { return 2 * align_up((size_t)(B + 1) * 4); }
size_t padded_ws_bytes(int B, int H, int64_t q_slot, int64_t kv_slot, int D) {
  const int64_t tq = (int64_t)B * q_slot, tk = (int64_t)B * kv_slot;
  const size_t f = fwd_layout(B, H, tq, tk, D).total, b = bwd_layout(B, H, tq, tk, D).total;
  return padded_offsets_bytes(B) + (f > b ? f : b);
}

// Checks the slot sizes and the workspace, then writes the slot offsets at
// its start. *rest receives the part left for the pass itself.
jfa_status padded_setup(int B, int H, int q_slot, int kv_slot, int D, void* ws, size_t ws_bytes, void* stream,
                        char** rest, size_t* rest_bytes) {
  if (!padded_sizes_ok(B, H, q_slot, kv_slot, D))
    return fail(JFA_ERR_INVALID_ARGUMENT, "invalid sizes: B=%d, H=%d, D=%d, q_slot=%d, kv_slot=%d (B * slot < 2^31)", B,
                H, D, q_slot, kv_slot);
  if (!ws || !aligned(ws, kAlign)) return fail(JFA_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  const size_t need = padded_ws_bytes(B, H, q_slot, kv_slot, D);
  if (ws_bytes < need) return fail(JFA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  DeviceInfo* dev = nullptr;
  jfa_status s = device_info(&dev);
  if (s != JFA_OK) return s;
  char* w = (char*)ws;
  int* qo = (int*)w;
  int* ko = (int*)(w + align_up((size_t)(B + 1) * 4));
  hipError_t e = timed(kKindPlan, (hipStream_t)stream,
                       [&] { return jfa::launch_slot_offsets(B, q_slot, kv_slot, qo, ko, (hipStream_t)stream); });
  if (e != hipSuccess) return fail(JFA_ERR_HIP, "slot offsets launch: %s", hipGetErrorString(e));
  *rest = w + padded_offsets_bytes(B);
  *rest_bytes = ws_bytes - padded_offsets_bytes(B);
  return JFA_OK;
}

bool tile_of(int kernel, int D, int dtype, int* tm, int* tn) {
  switch (kernel) {
    case JFA_KERNEL_FWD:
      *tm = jfa::fwd_tile_rows(dtype == JFA_DTYPE_F32, D);
      *tn = jfa::fwd_tile_keys(dtype == JFA_DTYPE_F32, D);
      return true;
    case JFA_KERNEL_BWD_DKDV: *tm = jfa::dkv_tile_rows(dtype == JFA_DTYPE_F32, D); *tn = jfa::kDkvTN; return true;
    case JFA_KERNEL_BWD_DQ: *tm = jfa::kDqTM; *tn = jfa::kDqTN; return true;
    case JFA_KERNEL_BWD_SQ:
    case JFA_KERNEL_FWD_SQ: *tm = jfa::kSqQMax; *tn = jfa::kSqKC; return true;
    default: return false;
  }
}

// ---------------------------------------------------------------------------
// Allocation-free forward. Its scratch (work-list headers, items, short-query
// chunk rows) is this file-scope device array; each GPU the library runs on
// holds its own copy until the process ends. Host code never passes the
// array's name to a kernel (in host code it is a host-side stand-in, not a
// device address): the device address is fetched once per device with
// hipGetSymbolAddress, with that device current, and kept in
// g_scratch_ptr. The plan kernel rewrites every header field and ticket the
// kernels read, so nothing needs clearing between calls; calls that overlap
// on one GPU share the array and race.
constexpr size_t kNoAllocScratchBytes = (size_t)JFA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

jfa_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(JFA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(JFA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::call_once(g_scratch_once[dev], [dev]() {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess)
    return fail(JFA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(g_scratch_err[dev]));
  *out = g_scratch_ptr[dev];
  return JFA_OK;
}

}  // namespace

extern "C" {

jfa_status jfa_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                           const int32_t* kv_offsets, int B, int H, int D, int64_t total_q,
                           int64_t total_kv, int max_kv_len, const float* bias, int causal, void* out,
                           float* lse, void* stream) {
  if (max_kv_len < 0) return fail(JFA_ERR_INVALID_ARGUMENT, "max_kv_len must be >= 0 (0: unknown)");
  if (!valid_sizes(B, H, total_q, total_kv, D))
    return fail(JFA_ERR_INVALID_ARGUMENT, "invalid sizes: B=%d, H=%d, D=%d, total_q=%lld, total_kv=%lld", B, H, D,
                (long long)total_q, (long long)total_kv);
  const size_t need = fwd_layout(B, H, total_q, total_kv, D, short_pass_on(max_kv_len)).total;
  if (need > kNoAllocScratchBytes)
    return fail(JFA_ERR_WORKSPACE,
                "jfa_fwd_noalloc: this call needs %zu bytes of scratch, more than its fixed %zu; pass a key-count "
                "bound of at most 1024 (max_kv_len) if it holds, or call jfa_fwd with a workspace",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  jfa_status s = scratch_ptr(&ws);
  if (s != JFA_OK) return s;
  return fwd_impl(false, q, k, v, q_offsets, kv_offsets, B, H, D, total_q, total_kv, max_kv_len, bias, causal, out,
                  lse, ws, kNoAllocScratchBytes, stream, nullptr, /*compact=*/true);
}

size_t jfa_fwd_workspace_bytes(int B, int H, int64_t total_q, int64_t total_kv, int D, int causal) {
  (void)causal;
  if (!valid_sizes(B, H, total_q, total_kv, D)) return 0;
  return fwd_layout(B, H, total_q, total_kv, D).total;
}

size_t jfa_bwd_workspace_bytes(int B, int H, int64_t total_q, int64_t total_kv, int D, int causal) {
  (void)causal;
  if (!valid_sizes(B, H, total_q, total_kv, D)) return 0;
  return bwd_layout(B, H, total_q, total_kv, D).total;
}

jfa_status jfa_fwd(const void* q, const void* k, const void* v, const int32_t* q_offsets, const int32_t* kv_offsets,
                   int B, int H, int D, int64_t total_q, int64_t total_kv, int max_kv_len, const float* bias,
                   int causal, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(false, q, k, v, q_offsets, kv_offsets, B, H, D, total_q, total_kv, max_kv_len, bias, causal, out,
                  lse, workspace, workspace_bytes, stream);
}

jfa_status jfa_fwd_f32(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                       const int32_t* kv_offsets, int B, int H, int D, int64_t total_q, int64_t total_kv,
                       int max_kv_len, const float* bias, int causal, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return fwd_impl(true, q, k, v, q_offsets, kv_offsets, B, H, D, total_q, total_kv, max_kv_len, bias, causal, out,
                  lse, workspace, workspace_bytes, stream);
}

jfa_status jfa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
                   const int32_t* q_offsets, const int32_t* kv_offsets, int B, int H, int D, int64_t total_q,
                   int64_t total_kv, int max_kv_len, const float* bias, int causal, void* dq, void* dk, void* dv,
                   float* dbias, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(false, q, k, v, out, lse, dout, q_offsets, kv_offsets, B, H, D, total_q, total_kv, max_kv_len, bias,
                  causal, dq, dk, dv, dbias, workspace, workspace_bytes, stream);
}

jfa_status jfa_bwd_f32(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, const int32_t* q_offsets, const int32_t* kv_offsets, int B, int H, int D,
                       int64_t total_q, int64_t total_kv, int max_kv_len, const float* bias, int causal, void* dq,
                       void* dk, void* dv, float* dbias, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(true, q, k, v, out, lse, dout, q_offsets, kv_offsets, B, H, D, total_q, total_kv, max_kv_len, bias,
                  causal, dq, dk, dv, dbias, workspace, workspace_bytes, stream);
}

size_t jfa_padded_workspace_bytes(int B, int H, int q_slot, int kv_slot, int D) {
  if (!padded_sizes_ok(B, H, q_slot, kv_slot, D)) return 0;
  return padded_ws_bytes(B, H, q_slot, kv_slot, D);
}

jfa_status jfa_fwd_padded(const void* q, const void* k, const void* v, const int32_t* kv_lens, int B, int q_slot,
                          int kv_slot, int H, int D, const float* bias, int causal, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && (!kv_lens || !aligned(kv_lens, 4)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "kv_lens must be non-NULL and 4-byte aligned");
  char* rest = nullptr;
  size_t rest_bytes = 0;
  jfa_status s = padded_setup(B, H, q_slot, kv_slot, D, workspace, workspace_bytes, stream, &rest, &rest_bytes);
  if (s != JFA_OK) return s;
  const int32_t* qo = (const int32_t*)workspace;
  const int32_t* ko = (const int32_t*)((char*)workspace + align_up((size_t)(B + 1) * 4));
  return fwd_impl(false, q, k, v, qo, ko, B, H, D, (int64_t)B * q_slot, (int64_t)B * kv_slot, 0, bias, causal, out,
                  lse, rest, rest_bytes, stream, B > 0 ? kv_lens : nullptr);
}

jfa_status jfa_bwd_padded(const void* q, const void* k, const void* v, const void* out, const float* lse,
                          const void* dout, const int32_t* kv_lens, int B, int q_slot, int kv_slot, int H, int D,
                          const float* bias, int causal, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (B > 0 && (!kv_lens || !aligned(kv_lens, 4)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "kv_lens must be non-NULL and 4-byte aligned");
  char* rest = nullptr;
  size_t rest_bytes = 0;
  jfa_status s = padded_setup(B, H, q_slot, kv_slot, D, workspace, workspace_bytes, stream, &rest, &rest_bytes);
  if (s != JFA_OK) return s;
  const int32_t* qo = (const int32_t*)workspace;
  const int32_t* ko = (const int32_t*)((char*)workspace + align_up((size_t)(B + 1) * 4));
  return bwd_impl(false, q, k, v, out, lse, dout, qo, ko, B, H, D, (int64_t)B * q_slot, (int64_t)B * kv_slot, 0,
                  bias, causal, dq, dk, dv, nullptr, rest, rest_bytes, stream, B > 0 ? kv_lens : nullptr);
}

jfa_status jfa_offsets_from_lengths(const int32_t* lengths, int B, int32_t* offsets, void* stream) {
  if (B < 0) return fail(JFA_ERR_INVALID_ARGUMENT, "B must be >= 0");
  if (!offsets || (B > 0 && !lengths)) return fail(JFA_ERR_INVALID_ARGUMENT, "lengths/offsets must not be NULL");
  DeviceInfo* dev = nullptr;
  jfa_status s = device_info(&dev);
  if (s != JFA_OK) return s;
  hipError_t e = timed(kKindScan, (hipStream_t)stream, [&] { return jfa::launch_scan(lengths, B, offsets, (hipStream_t)stream); });
  if (e != hipSuccess) return fail(JFA_ERR_HIP, "scan launch: %s", hipGetErrorString(e));
  return ok();
}

jfa_status jfa_tile_config(int kernel, int D, int dtype, int* tile_m, int* tile_n) {
  if (!tile_m || !tile_n) return fail(JFA_ERR_INVALID_ARGUMENT, "tile_m/tile_n must not be NULL");
  if (!(D == 32 || D == 64 || D == 128)) return fail(JFA_ERR_INVALID_ARGUMENT, "D must be 32, 64 or 128");
  if (dtype != JFA_DTYPE_BF16 && dtype != JFA_DTYPE_F32) return fail(JFA_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (!tile_of(kernel, D, dtype, tile_m, tile_n)) return fail(JFA_ERR_INVALID_ARGUMENT, "unknown kernel id %d", kernel);
  return ok();
}

size_t jfa_plan_workspace_bytes(int B, int H, int64_t total_q, int64_t total_kv, int D, int dtype, int kernel) {
  int tm, tn;
  if (!valid_sizes(B, H, total_q, total_kv, D) || (dtype != JFA_DTYPE_BF16 && dtype != JFA_DTYPE_F32) ||
      !tile_of(kernel, D, dtype, &tm, &tn))
    return 0;
  const bool sq = kernel == JFA_KERNEL_BWD_SQ || kernel == JFA_KERNEL_FWD_SQ;
  const int64_t cap = kernel == JFA_KERNEL_BWD_DKDV || sq ? max_items(B, H, total_kv, tn) : max_items(B, H, total_q, tm);
  return sizeof(PlanHeader) + align_up((size_t)cap * 16) + (sq ? align_up((size_t)B * H * 4) : 0);
}

jfa_status jfa_build_plan(const int32_t* q_offsets, const int32_t* kv_offsets, int B, int H, int D, int dtype,
                          int causal, int kernel, void* workspace, size_t workspace_bytes, void* stream) {
  int tm, tn;
  if (B < 0 || B > JFA_MAX_BATCH || H < 1 || !(D == 32 || D == 64 || D == 128) ||
      (dtype != JFA_DTYPE_BF16 && dtype != JFA_DTYPE_F32))
    return fail(JFA_ERR_INVALID_ARGUMENT, "invalid sizes");
  if (!tile_of(kernel, D, dtype, &tm, &tn)) return fail(JFA_ERR_INVALID_ARGUMENT, "unknown kernel id %d", kernel);
  if (!q_offsets || !kv_offsets) return fail(JFA_ERR_INVALID_ARGUMENT, "offsets must not be NULL");
  if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < sizeof(PlanHeader))
    return fail(JFA_ERR_WORKSPACE, "workspace must be non-NULL, 256-byte aligned and at least 256 bytes");
  DeviceInfo* dev = nullptr;
  jfa_status s = device_info(&dev);
  if (s != JFA_OK) return s;
  char* w = (char*)workspace;
  jfa::PlanArgs pa{};
  pa.q_off = q_offsets;
  pa.kv_off = kv_offsets;
  pa.B = B;
  pa.H = H;
  pa.causal = causal ? 1 : 0;
  // Layout: header, items, and for the short-query pass the [B*H] group table
  // after the largest list the sizes allow.
  const bool sq = kernel == JFA_KERNEL_BWD_SQ || kernel == JFA_KERNEL_FWD_SQ;
  const size_t tail = sq ? align_up((size_t)B * H * 4) : 0;
  if (workspace_bytes < sizeof(PlanHeader) + tail) return fail(JFA_ERR_WORKSPACE, "workspace too small");
  const int kind = kernel == JFA_KERNEL_BWD_DKDV ? jfa::kPassKV : (sq ? jfa::kPassSQ : jfa::kPassQ);
  const int short_q = sq ? -1 : jfa::kSqQMax;
  pa.pass[0] = {(int4*)(w + sizeof(PlanHeader)), (PlanHeader*)w,
                (long)((workspace_bytes - sizeof(PlanHeader) - tail) / 16), tm, tn, kind, jfa::kPlanQueues, short_q,
                tail ? (int*)(w + workspace_bytes - tail) : nullptr};
  hipError_t e = jfa::launch_plan(pa, 1, (hipStream_t)stream);
  if (e != hipSuccess) return fail(JFA_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
  return ok();
}

jfa_status jfa_timing_enable(int enable) {
  g_timing.store(enable != 0);
  return ok();
}

jfa_status jfa_timing_collect(double* total_ms, int64_t* launches, int n_kinds) {
  if (n_kinds < 0 || (n_kinds > 0 && (!total_ms || !launches)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "total_ms/launches must hold n_kinds entries");
  for (int i = 0; i < n_kinds; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  std::vector<TimingRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    recs.swap(g_recs);
  }
  hipError_t first = hipSuccess;
  for (const TimingRec& r : recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e == hipSuccess && r.kind < n_kinds) {
      total_ms[r.kind] += ms;
      launches[r.kind] += 1;
    }
    if (e != hipSuccess && first == hipSuccess) first = e;
  }
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    for (const TimingRec& r : recs) {
      g_event_pool.push_back(r.a);
      g_event_pool.push_back(r.b);
    }
  }
  if (first != hipSuccess) return fail(JFA_ERR_HIP, "timing events: %s", hipGetErrorString(first));
  return ok();
}

const char* jfa_status_string(jfa_status status) {
  switch (status) {
    case JFA_OK: return "ok";
    case JFA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case JFA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case JFA_ERR_UNSUPPORTED: return "unsupported device or configuration";
    case JFA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* jfa_last_error(void) { return g_last_error.c_str(); }

int jfa_abi_version(void) { return JFA_ABI_VERSION; }

}  // extern "C"
