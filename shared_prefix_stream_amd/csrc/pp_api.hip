// C ABI of libppattn: argument validation (host only, before any HIP call),
// workspace carving, kernel launches on the caller's stream, status codes.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "pp_internal.h"

namespace pp {
thread_local StageEvents g_stage_events;
}

namespace {
pp_status_t fail(pp_status_t st, const char* fmt, ...);
}

namespace pp {
// (for the other translation units: the calling thread's error message)
pp_status_t set_error(pp_status_t st, const char* msg) { return fail(st, "%s", msg); }
}

namespace {

thread_local char g_err[512] = "";

pp_status_t fail(pp_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

pp_status_t ok() {
  g_err[0] = '\0';
  return PP_OK;
}

// Once-per-device cache of the compute-unit count (the only global state).
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_num_cus[kMaxDevices];

bool num_cus(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::call_once(g_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = -1;
    g_num_cus[dev] = n;
  });
  *out = g_num_cus[dev];
  return *out > 0;
}

size_t elem_size(pp_dtype_t dt) { return dt == PP_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

pp_status_t check_shape(int64_t seq_len, int32_t P, int32_t H, int32_t d, pp_dtype_t dtype) {
  if (dtype != PP_BF16 && dtype != PP_F32) return fail(PP_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (d != 64 && d != 128) return fail(PP_ERR_UNSUPPORTED, "head dim d=%d not supported (64 or 128)", d);
  if (seq_len < 1 || seq_len > PP_MAX_SEQ_LEN)
    return fail(PP_ERR_INVALID_ARG, "seq_len=%lld out of range [1, %lld]", (long long)seq_len, (long long)PP_MAX_SEQ_LEN);
  if (P < 1 || P > PP_MAX_STREAMS) return fail(PP_ERR_INVALID_ARG, "P=%d out of range [1, %d]", P, PP_MAX_STREAMS);
  if (H < 1 || H > PP_MAX_HEADS) return fail(PP_ERR_INVALID_ARG, "H=%d out of range [1, %d]", H, PP_MAX_HEADS);
  return PP_OK;
}

// Split counts are chosen for the device's compute-unit count, capped at
// the 256 CUs of an MI355X; the workspace is sized for 256 CUs, an upper
// bound because split counts never shrink as the CU count grows.  So the
// workspace size is a host-only function of the shape.
constexpr int kSizingCus = 256;

struct Plan {
  pp::DocPlan doc;
  int batched_splits;
};

// B requests of P streams, H query heads in groups of G per key/value head:
// the document kernel sees P * G queries per key/value head and B * H / G
// (key/value head, request) pairs; the baseline B * P streams of H heads.
Plan plan_for(int64_t seq_len, int32_t P, int32_t H, int32_t d, pp_dtype_t dtype, int cus, int32_t B = 1,
              int32_t G = 1) {
  if (cus > kSizingCus) cus = kSizingCus;
  Plan pl;
  pl.doc = pp::choose_doc_plan(seq_len, P * G, B * (H / G), d, dtype, cus);
  pl.batched_splits = pp::choose_batched_splits(seq_len, B * P, H, cus);
  return pl;
}

size_t required_bytes(int64_t seq_len, int32_t P, int32_t H, int32_t d, pp_dtype_t dtype, int32_t B = 1,
                      int32_t G = 1) {
  const Plan pl = plan_for(seq_len, P, H, d, dtype, kSizingCus, B, G);
  const int n = pl.doc.n_splits > pl.batched_splits ? pl.doc.n_splits : pl.batched_splits;
  return pp::workspace_bytes_for(n, (int64_t)B * P, H, d, seq_len, B);
}

enum class Path { kParallel, kBatched };

// A visibility plan computed earlier by pp_attn_plan (device buffers).
struct ExternalPlan {
  const int32_t* doc_len;
  const int32_t* counts;
  const int32_t* slots;
  int64_t capacity;
};

// The append part of an appending decode step (the step's new query, key
// and value per stream, the caches it writes, the rotary base).
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  double rope_base;
};

// bt (several requests, grouped key/value heads) comes with the multi and
// appending entry points only, which have checked B, G and seq_lens; H is
// the number of query heads.
pp_status_t decode_impl(Path path, const void* q, const void* k, const void* v, const int32_t* sid, int64_t seq_len,
                        int32_t P, int32_t H, int32_t d, float scale, void* out, pp_dtype_t dtype, void* workspace,
                        size_t workspace_bytes, void* hip_stream, void* const* events = nullptr,
                        const ExternalPlan* xp = nullptr, const AppendArgs* ap = nullptr,
                        pp::Batch bt = pp::Batch()) {
  pp_status_t st = check_shape(seq_len, P, H, d, dtype);
  if (st != PP_OK) return st;
  if (!q || !k || !v || !sid || !out) return fail(PP_ERR_INVALID_ARG, "null q, k_cache, v_cache, stream_id or out");
  if (!isfinite(scale)) return fail(PP_ERR_INVALID_ARG, "scale is not finite");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sid) || !aligned16(out))
    return fail(PP_ERR_INVALID_ARG, "q, k_cache, v_cache, stream_id and out must be 16-byte aligned");
  const size_t es = elem_size(dtype);
  const int32_t B = bt.B, G = bt.G, Hkv = H / G;
  bt.kv_stride = seq_len * Hkv * d;
  bt.id_stride = seq_len;
  const size_t nq = (size_t)B * P * H * d * es, nkv = (size_t)B * seq_len * Hkv * d * es,
               nid = (size_t)B * seq_len * 4;
  if (overlaps(out, nq, q, nq) || overlaps(out, nq, k, nkv) || overlaps(out, nq, v, nkv) ||
      overlaps(out, nq, sid, nid) || overlaps(out, nq, workspace, workspace_bytes))
    return fail(PP_ERR_INVALID_ARG, "out overlaps an input or the workspace");
  if (overlaps(workspace, workspace_bytes, q, nq) || overlaps(workspace, workspace_bytes, k, nkv) ||
      overlaps(workspace, workspace_bytes, v, nkv) || overlaps(workspace, workspace_bytes, sid, nid))
    return fail(PP_ERR_INVALID_ARG, "workspace overlaps an input");
  // a caller's plan: head (doc_len per request, then with an append their
  // seq_len), counts [B][P], slots [B][P][capacity]
  const size_t nh = (size_t)(ap ? 2 : 1) * B * 4, nc = (size_t)B * P * 4,
               ns = xp ? (size_t)B * P * (size_t)(xp->capacity > 0 ? xp->capacity : 0) * 4 : 0;
  if (xp) {
    if (!xp->doc_len || !xp->counts) return fail(PP_ERR_INVALID_ARG, "null plan_doc_len or plan_counts");
    if (xp->capacity < 0 || (xp->capacity > 0 && !xp->slots))
      return fail(PP_ERR_INVALID_ARG, "plan_slots is null or plan_capacity negative");
    if (overlaps(out, nq, xp->doc_len, nh) || overlaps(out, nq, xp->counts, nc) || overlaps(out, nq, xp->slots, ns) ||
        overlaps(workspace, workspace_bytes, xp->doc_len, nh) || overlaps(workspace, workspace_bytes, xp->counts, nc) ||
        overlaps(workspace, workspace_bytes, xp->slots, ns))
      return fail(PP_ERR_INVALID_ARG, "a plan buffer overlaps out or the workspace");
  }
  if (ap) {  // (always with a caller's plan)
    if (P > seq_len) return fail(PP_ERR_INVALID_ARG, "P=%d exceeds max_seq_len=%lld", P, (long long)seq_len);
    if (!ap->k_new || !ap->v_new) return fail(PP_ERR_INVALID_ARG, "null k_new or v_new");
    if (!aligned16(ap->k_new) || !aligned16(ap->v_new))
      return fail(PP_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
    if (!isfinite(ap->rope_base)) return fail(PP_ERR_INVALID_ARG, "rope_base is not finite");
    // the caches are written: nothing read in the step may share their bytes
    const size_t nn = (size_t)B * P * Hkv * d * es;  // new keys (values) of the step
    for (const void* w : {k, v})
      if (overlaps(w, nkv, q, nq) || overlaps(w, nkv, ap->k_new, nn) || overlaps(w, nkv, ap->v_new, nn) ||
          overlaps(w, nkv, sid, nid) || overlaps(w, nkv, workspace, workspace_bytes) ||
          overlaps(w, nkv, xp->doc_len, nh) || overlaps(w, nkv, xp->counts, nc) || overlaps(w, nkv, xp->slots, ns))
        return fail(PP_ERR_INVALID_ARG, "k_cache or v_cache overlaps another argument");
    if (overlaps(k, nkv, v, nkv)) return fail(PP_ERR_INVALID_ARG, "k_cache and v_cache overlap");
    if (overlaps(out, nq, ap->k_new, nn) || overlaps(out, nq, ap->v_new, nn) ||
        overlaps(workspace, workspace_bytes, ap->k_new, nn) || overlaps(workspace, workspace_bytes, ap->v_new, nn))
      return fail(PP_ERR_INVALID_ARG, "k_new or v_new overlaps out or the workspace");
  }
  const size_t need = required_bytes(seq_len, P, H, d, dtype, B, G);
  if (!workspace || workspace_bytes < need)
    return fail(PP_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0, need);
  int cus = 0;
  if (!num_cus(&cus)) return fail(PP_ERR_HIP, "could not query the current device's compute-unit count");
  const Plan pl = plan_for(seq_len, P, H, d, dtype, cus, B, G);
  if ((int64_t)pl.doc.n_ptiles * B > 65535)
    return fail(PP_ERR_INVALID_ARG, "B * query tiles = %lld exceeds the grid", (long long)pl.doc.n_ptiles * B);

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const float c = (float)((double)scale * 1.4426950408889634074);  // log2(e): softmax in base 2
  const int n_splits = path == Path::kParallel ? pl.doc.n_splits : pl.batched_splits;
  // the keys and values a step may read (K and V up to the bound seq_len):
  // past the last-level cache they are streamed with the non-temporal hint
  const bool stream_nt = 2.0 * (double)nkv > pp::kLastLevelCacheBytes;
  pp::Workspace ws = pp::carve_workspace(workspace, n_splits, (int64_t)B * P, H, d, seq_len, B);
  if (xp) {  // the caller's plan (read only) in place of the plan kernel's
    ws.plan = const_cast<int32_t*>(xp->doc_len);
    ws.counts = const_cast<int32_t*>(xp->counts);
    ws.slots = const_cast<int32_t*>(xp->slots);
    ws.cap = xp->capacity;
  }
  if (ap && !bt.seq_lens) ws.dyn_len = xp->doc_len + 1;  // {doc_len, seq_len} of the step

  // optional profiling: stage i's kernel is bound to events[2i] (its start)
  // and events[2i + 1] (its end)
  auto stage = [&](int i) {
    if (events)
      pp::g_stage_events = {static_cast<hipEvent_t>(events[2 * i]), static_cast<hipEvent_t>(events[2 * i + 1])};
  };
  auto unstage = [&]() { pp::g_stage_events = pp::StageEvents(); };
  hipError_t e = hipSuccess;
  if (!xp) {
    stage(0);
    e = pp::launch_plan(sid, seq_len, P, ws.plan, ws.counts, ws.slots, ws.cap, stream, bt, ws.rows);
    unstage();
  }
  if (e == hipSuccess && ap) {  // new keys and values into the caches, rotated queries into the workspace
    e = pp::launch_append_rope(q, ap->k_new, ap->v_new, const_cast<void*>(k), const_cast<void*>(v), P, H, Hkv, d, dtype,
                               ap->rope_base, ws.plan, ws.counts, seq_len, ws.q_rot, stream, B, bt.kv_stride,
                               bt.active);
    q = ws.q_rot;
  }
  if (e == hipSuccess) {
    stage(1);
    e = path == Path::kParallel
            ? pp::launch_doc(pl.doc, q, k, v, seq_len, P, Hkv, d, dtype, c, ws, stream, false, bt, nullptr, stream_nt)
            : pp::launch_batched_doc(n_splits, q, k, v, seq_len, P, H, d, dtype, c, ws, stream, bt);
    unstage();
  }
  if (e == hipSuccess) {
    stage(2);
    e = pp::launch_tail_merge(n_splits, q, k, v, sid, seq_len, P, H, d, dtype, c, ws, out, stream, bt, stream_nt);
    unstage();
  }
  if (e != hipSuccess) return fail(PP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Prefill workspace: the one-stream plan (document length), then one
// partial state per (slot, head) of the causal document kernel (one split).
constexpr int64_t kPrefillMaxLen = (int64_t)65535 * 256;  // query tiles per head fit the grid

size_t prefill_bytes(int64_t T, int32_t H, int32_t d) {
  return 256 /*base alignment slack*/ + 512 /*plan, counts*/ + pp::align_up((size_t)T * H * sizeof(float2), 256) +
         pp::align_up((size_t)T * H * d * sizeof(float), 256);
}

pp::Workspace carve_prefill(void* ws, int64_t T, int32_t H) {
  uintptr_t at = pp::align_up((uintptr_t)ws, 256);
  pp::Workspace w;
  w.plan = reinterpret_cast<int32_t*>(at);
  w.counts = reinterpret_cast<int32_t*>(at + 256);
  w.slots = nullptr;
  w.cap = 0;
  at += 512;
  w.part_ml = reinterpret_cast<float2*>(at);
  at += pp::align_up((size_t)T * H * sizeof(float2), 256);
  w.part_o = reinterpret_cast<float*>(at);
  w.q_rot = nullptr;
  return w;
}

pp_status_t check_prefill_shape(int64_t seq_len, int32_t H, int32_t d, pp_dtype_t dtype) {
  pp_status_t st = check_shape(seq_len, 1, H, d, dtype);
  if (st != PP_OK) return st;
  if (seq_len > kPrefillMaxLen)
    return fail(PP_ERR_INVALID_ARG, "prefill seq_len=%lld exceeds %lld", (long long)seq_len, (long long)kPrefillMaxLen);
  return PP_OK;
}

// Scratch of pp_attn_plan: the two-pass plan's chunk rows (and the base
// alignment), at least PP_PLAN_WORKSPACE_BYTES.
size_t plan_scratch_bytes(int64_t seq_len, int32_t P) {
  const size_t r = pp::plan_rows_bytes(seq_len, P, 1);
  const size_t n = r ? 256 + r : 0;
  return n > PP_PLAN_WORKSPACE_BYTES ? n : (size_t)PP_PLAN_WORKSPACE_BYTES;
}

}  // namespace

extern "C" {

size_t pp_attn_plan_workspace_bytes(int64_t seq_len, int32_t P) {
  if (seq_len < 1 || seq_len > PP_MAX_SEQ_LEN || P < 1 || P > PP_MAX_STREAMS) return 0;
  ok();
  return plan_scratch_bytes(seq_len, P);
}

int pp_abi_version(void) { return PP_ABI_VERSION; }

const char* pp_status_string(pp_status_t s) {
  switch (s) {
    case PP_OK: return "PP_OK";
    case PP_ERR_INVALID_ARG: return "PP_ERR_INVALID_ARG: invalid argument";
    case PP_ERR_UNSUPPORTED: return "PP_ERR_UNSUPPORTED: unsupported head dimension or dtype";
    case PP_ERR_WORKSPACE: return "PP_ERR_WORKSPACE: workspace missing or too small";
    case PP_ERR_HIP: return "PP_ERR_HIP: HIP runtime error";
  }
  return "unknown pp_status_t";
}

const char* pp_last_error_message(void) { return g_err; }

size_t pp_attn_workspace_bytes(int64_t seq_len, int32_t P, int32_t H, int32_t d, pp_dtype_t dtype) {
  if (check_shape(seq_len, P, H, d, dtype) != PP_OK) return 0;
  ok();
  return required_bytes(seq_len, P, H, d, dtype);
}

pp_status_t pp_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* stream_id,
                           int64_t seq_len, int32_t P, int32_t H, int32_t d, float scale, void* out,
                           pp_dtype_t dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return decode_impl(Path::kParallel, q, k_cache, v_cache, stream_id, seq_len, P, H, d, scale, out, dtype, workspace,
                     workspace_bytes, hip_stream);
}

pp_status_t pp_attn_decode_batched(const void* q, const void* k_cache, const void* v_cache, const int32_t* stream_id,
                                   int64_t seq_len, int32_t P, int32_t H, int32_t d, float scale, void* out,
                                   pp_dtype_t dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return decode_impl(Path::kBatched, q, k_cache, v_cache, stream_id, seq_len, P, H, d, scale, out, dtype, workspace,
                     workspace_bytes, hip_stream);
}

pp_status_t pp_attn_decode_planned(const void* q, const void* k_cache, const void* v_cache, const int32_t* stream_id,
                                   int64_t seq_len, int32_t P, int32_t H, int32_t d, float scale, void* out,
                                   pp_dtype_t dtype, const int32_t* plan_doc_len, const int32_t* plan_counts,
                                   const int32_t* plan_slots, int64_t plan_capacity, void* workspace,
                                   size_t workspace_bytes, void* hip_stream) {
  const ExternalPlan xp{plan_doc_len, plan_counts, plan_slots, plan_capacity};
  return decode_impl(Path::kParallel, q, k_cache, v_cache, stream_id, seq_len, P, H, d, scale, out, dtype, workspace,
                     workspace_bytes, hip_stream, nullptr, &xp);
}

pp_status_t pp_step_plan_multi(int32_t* stream_id, const int32_t* base_len, const int32_t* active,
                               int64_t max_seq_len, int32_t B, int32_t P, int32_t* plan_head, int32_t* plan_counts,
                               int32_t* plan_slots, int64_t plan_capacity, void* hip_stream) {
  if (B < 1 || B > PP_MAX_REQUESTS) return fail(PP_ERR_INVALID_ARG, "B=%d out of range [1, %d]", B, PP_MAX_REQUESTS);
  if (max_seq_len < 1 || max_seq_len > PP_MAX_SEQ_LEN)
    return fail(PP_ERR_INVALID_ARG, "max_seq_len=%lld out of range", (long long)max_seq_len);
  if (P < 1 || P > PP_MAX_STREAMS || P > max_seq_len)
    return fail(PP_ERR_INVALID_ARG, "P=%d out of range [1, min(%d, max_seq_len)]", P, PP_MAX_STREAMS);
  if (!stream_id || !base_len || !plan_head || !plan_counts) return fail(PP_ERR_INVALID_ARG, "null pointer");
  if (plan_capacity < 0 || (plan_capacity > 0 && !plan_slots))
    return fail(PP_ERR_INVALID_ARG, "plan_slots is null or plan_capacity negative");
  if (!aligned16(stream_id)) return fail(PP_ERR_INVALID_ARG, "stream_id must be 16-byte aligned");
  const size_t nid = (size_t)B * max_seq_len * 4, nc = (size_t)B * P * 4,
               ns = (size_t)B * P * (size_t)plan_capacity * 4, nb = (size_t)B * 4, na = active ? nc : 0;
  const void* outs[3] = {plan_head, plan_counts, plan_slots};
  const size_t nout[3] = {2 * nb, nc, ns};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], nout[i], stream_id, nid) || overlaps(outs[i], nout[i], base_len, nb) ||
        overlaps(outs[i], nout[i], active, na))
      return fail(PP_ERR_INVALID_ARG, "a plan buffer overlaps stream_id, base_len or active");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], nout[i], outs[j], nout[j])) return fail(PP_ERR_INVALID_ARG, "plan buffers overlap");
  }
  if (overlaps(base_len, nb, stream_id, nid) || overlaps(active, na, stream_id, nid))
    return fail(PP_ERR_INVALID_ARG, "base_len or active overlaps stream_id");
  pp::Batch bt;
  bt.B = B;
  bt.id_stride = max_seq_len;
  bt.active = active;
  hipError_t e = pp::launch_plan_append(stream_id, base_len, max_seq_len, P, plan_head, plan_counts, plan_slots,
                                        plan_capacity, static_cast<hipStream_t>(hip_stream), bt);
  if (e != hipSuccess) return fail(PP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

pp_status_t pp_step_plan(int32_t* stream_id, const int32_t* base_len, int64_t max_seq_len, int32_t P,
                         int32_t* plan_head, int32_t* plan_counts, int32_t* plan_slots, int64_t plan_capacity,
                         void* hip_stream) {
  return pp_step_plan_multi(stream_id, base_len, nullptr, max_seq_len, 1, P, plan_head, plan_counts, plan_slots,
                            plan_capacity, hip_stream);
}

pp_status_t pp_attn_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                  const int32_t* stream_id, int64_t max_seq_len, int32_t P, int32_t Hq, int32_t Hkv,
                                  int32_t d, float scale, double rope_base, const int32_t* plan_head,
                                  const int32_t* plan_counts, const int32_t* plan_slots, int64_t plan_capacity,
                                  void* out, pp_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                  void* hip_stream) {
  if (Hkv < 1 || Hq % Hkv != 0) return fail(PP_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const ExternalPlan xp{plan_head, plan_counts, plan_slots, plan_capacity};
  const AppendArgs ap{k_new, v_new, rope_base};
  pp::Batch bt;
  bt.G = Hq / Hkv;
  return decode_impl(Path::kParallel, q, k_cache, v_cache, stream_id, max_seq_len, P, Hq, d, scale, out, dtype,
                     workspace, workspace_bytes, hip_stream, nullptr, &xp, &ap, bt);
}

pp_status_t pp_attn_decode_append_multi(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                        void* v_cache, const int32_t* stream_id, const int32_t* active,
                                        int64_t max_seq_len, int32_t B, int32_t P, int32_t Hq, int32_t Hkv, int32_t d,
                                        float scale, double rope_base, const int32_t* plan_head,
                                        const int32_t* plan_counts, const int32_t* plan_slots, int64_t plan_capacity,
                                        void* out, pp_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                        void* hip_stream) {
  if (B < 1 || B > PP_MAX_REQUESTS) return fail(PP_ERR_INVALID_ARG, "B=%d out of range [1, %d]", B, PP_MAX_REQUESTS);
  if (Hkv < 1 || Hq % Hkv != 0) return fail(PP_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (!plan_head) return fail(PP_ERR_INVALID_ARG, "null plan_head");
  const ExternalPlan xp{plan_head, plan_counts, plan_slots, plan_capacity};
  const AppendArgs ap{k_new, v_new, rope_base};
  pp::Batch bt;
  bt.B = B;
  bt.G = Hq / Hkv;
  bt.seq_lens = plan_head + B;  // each request's step length, from the step's plan
  bt.active = active;
  return decode_impl(Path::kParallel, q, k_cache, v_cache, stream_id, max_seq_len, P, Hq, d, scale, out, dtype,
                     workspace, workspace_bytes, hip_stream, nullptr, &xp, &ap, bt);
}

size_t pp_attn_multi_workspace_bytes(int64_t max_seq_len, int32_t B, int32_t P, int32_t Hq, int32_t Hkv, int32_t d,
                                     pp_dtype_t dtype) {
  if (check_shape(max_seq_len, P, Hq, d, dtype) != PP_OK) return 0;
  if (B < 1 || B > PP_MAX_REQUESTS || Hkv < 1 || Hq % Hkv != 0) return 0;
  ok();
  return required_bytes(max_seq_len, P, Hq, d, dtype, B, Hq / Hkv);
}

static pp_status_t multi_impl(Path path, const void* q, const void* k, const void* v, const int32_t* sid,
                              const int32_t* seq_lens, const int32_t* active, int64_t max_seq_len, int32_t B,
                              int32_t P, int32_t Hq, int32_t Hkv, int32_t d, float scale, void* out,
                              pp_dtype_t dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (B < 1 || B > PP_MAX_REQUESTS) return fail(PP_ERR_INVALID_ARG, "B=%d out of range [1, %d]", B, PP_MAX_REQUESTS);
  if (Hkv < 1 || Hq < 1 || Hq % Hkv != 0)
    return fail(PP_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if ((int64_t)B * P > PP_MAX_STREAMS * (int64_t)PP_MAX_REQUESTS)
    return fail(PP_ERR_INVALID_ARG, "B * P too large");
  if (!seq_lens) return fail(PP_ERR_INVALID_ARG, "null seq_lens");
  pp::Batch bt;
  bt.B = B;
  bt.G = Hq / Hkv;
  bt.seq_lens = seq_lens;
  bt.active = active;
  const size_t nq = (size_t)B * P * Hq * d * elem_size(dtype);
  if (overlaps(out, nq, seq_lens, (size_t)B * 4) || overlaps(workspace, workspace_bytes, seq_lens, (size_t)B * 4))
    return fail(PP_ERR_INVALID_ARG, "seq_lens overlaps out or the workspace");
  if (overlaps(out, nq, active, (size_t)B * P * 4) || overlaps(workspace, workspace_bytes, active, (size_t)B * P * 4))
    return fail(PP_ERR_INVALID_ARG, "active overlaps out or the workspace");
  return decode_impl(path, q, k, v, sid, max_seq_len, P, Hq, d, scale, out, dtype, workspace, workspace_bytes,
                     hip_stream, nullptr, nullptr, nullptr, bt);
}

pp_status_t pp_attn_decode_multi(const void* q, const void* k_cache, const void* v_cache, const int32_t* stream_id,
                                 const int32_t* seq_lens, const int32_t* active, int64_t max_seq_len, int32_t B,
                                 int32_t P, int32_t Hq, int32_t Hkv, int32_t d, float scale, void* out,
                                 pp_dtype_t dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return multi_impl(Path::kParallel, q, k_cache, v_cache, stream_id, seq_lens, active, max_seq_len, B, P, Hq, Hkv, d,
                    scale, out, dtype, workspace, workspace_bytes, hip_stream);
}

pp_status_t pp_attn_decode_multi_batched(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* stream_id, const int32_t* seq_lens, const int32_t* active,
                                         int64_t max_seq_len, int32_t B, int32_t P, int32_t Hq, int32_t Hkv,
                                         int32_t d, float scale, void* out, pp_dtype_t dtype, void* workspace,
                                         size_t workspace_bytes, void* hip_stream) {
  return multi_impl(Path::kBatched, q, k_cache, v_cache, stream_id, seq_lens, active, max_seq_len, B, P, Hq, Hkv, d,
                    scale, out, dtype, workspace, workspace_bytes, hip_stream);
}

size_t pp_attn_prefill_workspace_bytes(int64_t seq_len, int32_t H, int32_t d, pp_dtype_t dtype) {
  if (check_prefill_shape(seq_len, H, d, dtype) != PP_OK) return 0;
  ok();
  return prefill_bytes(seq_len, H, d);
}

pp_status_t pp_attn_prefill(const void* q, const void* k, const void* v, const int32_t* stream_id, int64_t seq_len,
                            int32_t Hq, int32_t Hkv, int32_t d, float scale, void* out, pp_dtype_t dtype,
                            void* workspace, size_t workspace_bytes, void* hip_stream) {
  pp_status_t st = check_prefill_shape(seq_len, Hq, d, dtype);
  if (st != PP_OK) return st;
  if (Hkv < 1 || Hq % Hkv != 0) return fail(PP_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (!q || !k || !v || !stream_id || !out) return fail(PP_ERR_INVALID_ARG, "null q, k, v, stream_id or out");
  if (!isfinite(scale)) return fail(PP_ERR_INVALID_ARG, "scale is not finite");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(stream_id) || !aligned16(out))
    return fail(PP_ERR_INVALID_ARG, "q, k, v, stream_id and out must be 16-byte aligned");
  const size_t n = (size_t)seq_len * Hq * d * elem_size(dtype), nkv = (size_t)seq_len * Hkv * d * elem_size(dtype),
               nid = (size_t)seq_len * 4;
  if (overlaps(out, n, q, n) || overlaps(out, n, k, nkv) || overlaps(out, n, v, nkv) ||
      overlaps(out, n, stream_id, nid) || overlaps(out, n, workspace, workspace_bytes))
    return fail(PP_ERR_INVALID_ARG, "out overlaps an input or the workspace");
  if (overlaps(workspace, workspace_bytes, q, n) || overlaps(workspace, workspace_bytes, k, nkv) ||
      overlaps(workspace, workspace_bytes, v, nkv) || overlaps(workspace, workspace_bytes, stream_id, nid))
    return fail(PP_ERR_INVALID_ARG, "workspace overlaps an input");
  const size_t need = prefill_bytes(seq_len, Hq, d);
  if (!workspace || workspace_bytes < need)
    return fail(PP_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0, need);
  int cus = 0;
  if (!num_cus(&cus)) return fail(PP_ERR_HIP, "could not query the current device's compute-unit count");
  if (cus > kSizingCus) cus = kSizingCus;
  pp::DocPlan pl = pp::choose_doc_plan(seq_len, (int)seq_len, Hq, d, dtype, cus);
  pl.n_splits = 1;  // the causal document kernel covers each query tile's prefix in one workgroup
  const int tile = pp::doc_query_tile(pl, dtype);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const float c = (float)((double)scale * 1.4426950408889634074);
  const pp::Workspace ws = carve_prefill(workspace, seq_len, Hq);
  // grouped key/value heads: the causal document kernel runs one workgroup
  // row per query head (query tiles stay aligned with slots), each reading
  // its group's key/value head; the per-slot kernel maps heads the same way
  pp::Batch doc_bt, rest_bt;
  doc_bt.kv_group = Hq / Hkv;
  rest_bt.G = Hq / Hkv;
  // the document length (a one-stream plan with no list), the causal
  // document part, then everything else per query slot
  hipError_t e = pp::launch_plan(stream_id, seq_len, 1, ws.plan, ws.counts, nullptr, 0, stream);
  if (e == hipSuccess)
    e = pp::launch_doc(pl, q, k, v, seq_len, (int)seq_len, Hq, d, dtype, c, ws, stream, true, doc_bt, out);
  if (e == hipSuccess)
    e = pp::launch_prefill_rest(1, tile, q, k, v, stream_id, seq_len, Hq, d, dtype, c, ws, out, stream, rest_bt);
  if (e != hipSuccess) return fail(PP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

pp_status_t pp_attn_decode_profiled(int32_t batched, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* stream_id, int64_t seq_len, int32_t P, int32_t H, int32_t d,
                                    float scale, void* out, pp_dtype_t dtype, void* workspace,
                                    size_t workspace_bytes, void* hip_stream, void* const* events,
                                    int32_t n_events) {
  if (!events || n_events < PP_PROFILE_EVENTS)
    return fail(PP_ERR_INVALID_ARG, "need %d events, got %d", PP_PROFILE_EVENTS, events ? n_events : 0);
  for (int i = 0; i < PP_PROFILE_EVENTS; ++i)
    if (!events[i]) return fail(PP_ERR_INVALID_ARG, "events[%d] is null", i);
  return decode_impl(batched ? Path::kBatched : Path::kParallel, q, k_cache, v_cache, stream_id, seq_len, P, H, d,
                     scale, out, dtype, workspace, workspace_bytes, hip_stream, events);
}

pp_status_t pp_attn_plan(const int32_t* stream_id, int64_t seq_len, int32_t P, int32_t* doc_len_out,
                         int32_t* tail_count_out, int32_t* tail_slots_out, int64_t tail_capacity, void* workspace,
                         size_t workspace_bytes, void* hip_stream) {
  if (seq_len < 1 || seq_len > PP_MAX_SEQ_LEN)
    return fail(PP_ERR_INVALID_ARG, "seq_len=%lld out of range", (long long)seq_len);
  if (P < 1 || P > PP_MAX_STREAMS) return fail(PP_ERR_INVALID_ARG, "P=%d out of range", P);
  if (!stream_id || !doc_len_out || !tail_count_out) return fail(PP_ERR_INVALID_ARG, "null pointer");
  if (tail_capacity < 0 || (tail_capacity > 0 && !tail_slots_out))
    return fail(PP_ERR_INVALID_ARG, "tail_slots_out is null or tail_capacity negative");
  if (!aligned16(stream_id)) return fail(PP_ERR_INVALID_ARG, "stream_id must be 16-byte aligned");
  const size_t need = plan_scratch_bytes(seq_len, P);
  if (!workspace || workspace_bytes < need)
    return fail(PP_ERR_WORKSPACE, "pp_attn_plan needs %zu bytes of workspace", need);
  const size_t nid = (size_t)seq_len * 4, nc = (size_t)P * 4, ns = (size_t)P * (size_t)tail_capacity * 4;
  if (overlaps(workspace, workspace_bytes, stream_id, nid) || overlaps(workspace, workspace_bytes, doc_len_out, 4) ||
      overlaps(workspace, workspace_bytes, tail_count_out, nc) ||
      overlaps(workspace, workspace_bytes, tail_slots_out, ns))
    return fail(PP_ERR_INVALID_ARG, "workspace overlaps stream_id or an output");
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  // the workspace holds the per-chunk rows of the two-pass plan; the plan
  // itself is written straight into the caller's buffers
  int32_t* rows = pp::plan_rows_bytes(seq_len, P, 1)
                      ? reinterpret_cast<int32_t*>(pp::align_up((uintptr_t)workspace, 256))
                      : nullptr;
  hipError_t e = pp::launch_plan(stream_id, seq_len, P, doc_len_out, tail_count_out, tail_slots_out, tail_capacity,
                                 stream, pp::Batch(), rows);
  if (e != hipSuccess) return fail(PP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
