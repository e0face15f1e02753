// C ABI of libppattn: argument validation (host only, before any HIP call),
// workspace carving, kernel launches on the caller's stream, status codes.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "pp_internal.h"

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

Plan plan_for(int64_t seq_len, int32_t P, int32_t H, int32_t d, pp_dtype_t dtype, int cus) {
  if (cus > kSizingCus) cus = kSizingCus;
  Plan pl;
  pl.doc = pp::choose_doc_plan(seq_len, P, H, d, dtype, cus);
  pl.batched_splits = pp::choose_batched_splits(seq_len, P, H, cus);
  return pl;
}

size_t required_bytes(int64_t seq_len, int32_t P, int32_t H, int32_t d, pp_dtype_t dtype) {
  const Plan pl = plan_for(seq_len, P, H, d, dtype, kSizingCus);
  const int n = pl.doc.n_splits > pl.batched_splits ? pl.doc.n_splits : pl.batched_splits;
  return pp::workspace_bytes_for(n, P, H, d, seq_len);
}

enum class Path { kParallel, kBatched };

// A visibility plan computed earlier by pp_attn_plan (device buffers).
struct ExternalPlan {
  const int32_t* doc_len;
  const int32_t* counts;
  const int32_t* slots;
  int64_t capacity;
};

pp_status_t decode_impl(Path path, const void* q, const void* k, const void* v, const int32_t* sid, int64_t seq_len,
                        int32_t P, int32_t H, int32_t d, float scale, void* out, pp_dtype_t dtype, void* workspace,
                        size_t workspace_bytes, void* hip_stream, void* const* events = nullptr,
                        const ExternalPlan* xp = nullptr) {
  pp_status_t st = check_shape(seq_len, P, H, d, dtype);
  if (st != PP_OK) return st;
  if (!q || !k || !v || !sid || !out) return fail(PP_ERR_INVALID_ARG, "null q, k_cache, v_cache, stream_id or out");
  if (!isfinite(scale)) return fail(PP_ERR_INVALID_ARG, "scale is not finite");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sid) || !aligned16(out))
    return fail(PP_ERR_INVALID_ARG, "q, k_cache, v_cache, stream_id and out must be 16-byte aligned");
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)P * H * d * es, nkv = (size_t)seq_len * H * d * es, nid = (size_t)seq_len * 4;
  if (overlaps(out, nq, q, nq) || overlaps(out, nq, k, nkv) || overlaps(out, nq, v, nkv) ||
      overlaps(out, nq, sid, nid) || overlaps(out, nq, workspace, workspace_bytes))
    return fail(PP_ERR_INVALID_ARG, "out overlaps an input or the workspace");
  if (overlaps(workspace, workspace_bytes, q, nq) || overlaps(workspace, workspace_bytes, k, nkv) ||
      overlaps(workspace, workspace_bytes, v, nkv) || overlaps(workspace, workspace_bytes, sid, nid))
    return fail(PP_ERR_INVALID_ARG, "workspace overlaps an input");
  if (xp) {
    if (!xp->doc_len || !xp->counts) return fail(PP_ERR_INVALID_ARG, "null plan_doc_len or plan_counts");
    if (xp->capacity < 0 || (xp->capacity > 0 && !xp->slots))
      return fail(PP_ERR_INVALID_ARG, "plan_slots is null or plan_capacity negative");
    const size_t ns = (size_t)P * (size_t)xp->capacity * 4;
    if (overlaps(out, nq, xp->doc_len, 4) || overlaps(out, nq, xp->counts, (size_t)P * 4) ||
        overlaps(out, nq, xp->slots, ns) || overlaps(workspace, workspace_bytes, xp->doc_len, 4) ||
        overlaps(workspace, workspace_bytes, xp->counts, (size_t)P * 4) ||
        overlaps(workspace, workspace_bytes, xp->slots, ns))
      return fail(PP_ERR_INVALID_ARG, "a plan buffer overlaps out or the workspace");
  }
  const size_t need = required_bytes(seq_len, P, H, d, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(PP_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0, need);
  int cus = 0;
  if (!num_cus(&cus)) return fail(PP_ERR_HIP, "could not query the current device's compute-unit count");
  const Plan pl = plan_for(seq_len, P, H, d, dtype, cus);

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const float c = (float)((double)scale * 1.4426950408889634074);  // log2(e): softmax in base 2
  const int n_splits = path == Path::kParallel ? pl.doc.n_splits : pl.batched_splits;
  pp::Workspace ws = pp::carve_workspace(workspace, n_splits, P, H, seq_len);
  if (xp) {  // the caller's plan (read only) in place of the plan kernel's
    ws.plan = const_cast<int32_t*>(xp->doc_len);
    ws.counts = const_cast<int32_t*>(xp->counts);
    ws.slots = const_cast<int32_t*>(xp->slots);
    ws.cap = xp->capacity;
  }

  // optional profiling events around the launches
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), stream) : hipSuccess;
  };
  hipError_t e = mark(0);
  if (e == hipSuccess && !xp) e = pp::launch_plan(sid, seq_len, P, ws.plan, ws.counts, ws.slots, ws.cap, stream);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess) {
    e = path == Path::kParallel ? pp::launch_doc(pl.doc, q, k, v, seq_len, P, H, d, dtype, c, ws, stream)
                                : pp::launch_batched_doc(n_splits, q, k, v, seq_len, P, H, d, dtype, c, ws, stream);
  }
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess) e = pp::launch_tail_merge(n_splits, q, k, v, sid, seq_len, P, H, d, dtype, c, ws, out, stream);
  if (e == hipSuccess) e = mark(3);
  if (e != hipSuccess) return fail(PP_ERR_HIP, "kernel launch or event record failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

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
  if (!workspace || workspace_bytes < PP_PLAN_WORKSPACE_BYTES)
    return fail(PP_ERR_WORKSPACE, "pp_attn_plan needs %d bytes of workspace", (int)PP_PLAN_WORKSPACE_BYTES);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  // the workspace argument is reserved: the plan is written straight into
  // the caller's buffers
  hipError_t e = pp::launch_plan(stream_id, seq_len, P, doc_len_out, tail_count_out, tail_slots_out, tail_capacity,
                                 stream);
  if (e != hipSuccess) return fail(PP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
