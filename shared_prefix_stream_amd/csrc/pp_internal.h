// Internal declarations shared by the HIP translation units of libppattn.
// gfx950 (CDNA4) only: 64-wide wavefronts, MFMA bf16 16x16x32, 160 KB LDS.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "ppattn.h"

namespace pp {

// ------------------------------------------------------------ launching ---
// Events that the next kernel launch of this host thread binds to its own
// start and end (hipExtLaunchKernel), so that hipEventElapsedTime gives that
// kernel's execution time alone; both null for ordinary launches.  Set only
// by the profiling entry point around one launch at a time.
struct StageEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
extern thread_local StageEvents g_stage_events;

// Sets the calling thread's pp_last_error_message() and returns st.
pp_status_t set_error(pp_status_t st, const char* msg);

template <typename Tup, size_t... I>
inline void kernel_arg_ptrs(Tup& t, void** argv, std::index_sequence<I...>) {
  ((argv[I] = (void*)&std::get<I>(t)), ...);
}

// Launch of kernel k (no dynamic LDS) with its arguments converted to the
// kernel's parameter types; returns the launch status.
template <typename... Params, typename... Args>
inline hipError_t launch_kernel(void (*k)(Params...), dim3 grid, dim3 block, hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  std::tuple<Params...> t(std::forward<Args>(args)...);
  void* argv[sizeof...(Params) > 0 ? sizeof...(Params) : 1];
  kernel_arg_ptrs(t, argv, std::index_sequence_for<Params...>{});
  const StageEvents ev = g_stage_events;
  if (!ev.start && !ev.stop)  // (the plain launch costs the host less time)
    return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, stream);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, stream, ev.start, ev.stop, 0);
}

// Lazy rescaling threshold (log2 units): the running maximum used as the
// softmax reference is only raised when a score (or a tile's maximum)
// exceeds it by more than this, so exp2(x - m) <= 2^kLazyTau and the
// accumulators are rescaled rarely.  The merges use the same (m, l, O), so
// the result is unchanged up to rounding.
constexpr float kLazyTau = 8.0f;

// ----------------------------------------------------------------- types ---
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// A launch over B independent requests (each its own document, streams,
// ids and caches, laid out one after another) whose Hq query heads share
// Hkv = Hq / G key/value heads: query head hq reads key/value head hq / G.
// The single-request, one-head-per-key step is B = 1, G = 1.  Stream s of
// request b is stream b * P + s of the launch (q, out, counts, lists and
// partials are indexed that way).
struct Batch {
  int B = 1;
  int G = 1;
  int64_t kv_stride = 0;               // elements between requests' K (and V) caches
  int64_t id_stride = 0;               // ids between requests' stream_id arrays
  const int32_t* seq_lens = nullptr;   // per-request lengths on the device (else seq_len for all)
  const int32_t* active = nullptr;     // per launch stream: 0 = retired (sees nothing, output 0); null: all
  // document kernel without folding (the causal prefill): grid.y runs over
  // query heads and head h reads key/value head h / kv_group
  int kv_group = 1;
};

__device__ __forceinline__ bool stream_active(const Batch& bt, int s) {
  return !bt.active || __builtin_amdgcn_readfirstlane(bt.active[s]) != 0;
}

// Length of request b's sequence: its device value clamped to [0, bound],
// or the host value when there is none.
__device__ __forceinline__ int64_t request_len(const Batch& bt, int b, int64_t bound) {
  if (!bt.seq_lens) return bound;
  const int64_t n = __builtin_amdgcn_readfirstlane(bt.seq_lens[b]);
  return n < 0 ? 0 : (n > bound ? bound : n);
}

// Workspace layout (byte offsets from a 256-byte aligned base):
//   [0, PL)           int32 plan[b] = doc_len of request b (length of its
//                     leading id-0 run); PL = 256 bytes, more for B > 64
//   [256, +CNT)       int32 counts[P]: visible slots past the prefix, per stream
//   [.., +SL)         int32 slots[P][cap]: their ascending slot indices (the
//                     first cap of them; a stream with more gathers them itself;
//                     cap = min(seq_len, 2048) rounded up to a multiple of 4)
//   [.., +ML)         float2 part_ml[n_splits][P][H]  (m in log2 units, l)
//   [.., +O)          float  part_o [n_splits][P][H][d] (unnormalised)
//   [.., +QR)         the step's rotated queries [P][H][d] (appending step
//                     only; room for 4-byte elements)
//   [.., +RW)         the two-pass plan's chunk rows (plan_rows_bytes)
struct Workspace {
  int32_t* plan;
  int32_t* counts;
  int32_t* slots;
  int64_t cap;
  float2* part_ml;
  float* part_o;
  void* q_rot;
  int32_t* rows = nullptr;  // two-pass plan scratch (null: P too large for it)
  // appending step: the step's length lives on the device (plan[1]); the
  // host-side seq_len is then only an upper bound
  const int32_t* dyn_len = nullptr;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Per-stream slot-list capacity kept in the workspace: at most 2048 (a
// multiple of 4, so that every list starts 16-byte aligned).
constexpr int64_t kListCapMax = 2048;
inline int64_t list_cap_for(int64_t seq_len) {
  const int64_t c = seq_len < kListCapMax ? seq_len : kListCapMax;
  return (c + 3) & ~(int64_t)3;
}

inline size_t plan_bytes_for(int64_t B) { return align_up((size_t)(B < 2 ? 2 : B) * 4, 256); }

// Two-pass plan: the ids are cut into at most 64 chunks of a multiple of 1024
// slots; each chunk gets a head of kRowHead ints (first non-zero id, zero
// ids, zero ids after the first non-zero one, -) and the count of each
// stream's id.
constexpr int kRowMaxP = 1024;  // streams per request the two-pass plan handles
constexpr int kRowHead = 4;
inline int plan_row_chunks(int64_t seq_len) {
  const int64_t n = (seq_len + 1023) / 1024;
  return (int)(n < 1 ? 1 : (n > 64 ? 64 : n));
}
inline int64_t plan_row_chunk_len(int64_t seq_len) {
  const int64_t nc = plan_row_chunks(seq_len);
  const int64_t per = (seq_len + nc - 1) / nc;
  return (per + 1023) / 1024 * 1024;
}
// chunks per request rounded up to a multiple of 4: per request the rows
// are [stride][kRowHead] chunk heads then [P][stride] per-stream counts, so
// each stream's counts over all chunks are a few 16-byte loads
__host__ __device__ inline int plan_row_stride(int nc) { return (nc + 3) & ~3; }
// Which plan a launch takes.  The two passes are two small launches, each
// with a fixed cost of ~5 us on an MI355X whatever its work (measured: 5 us
// to count 32 chunks, 9 us to place them, at 16k + 15k slots and 256
// streams), while one workgroup per stream over all ids costs ~10 us there
// but grows with P x seq_len; past 2^24 stream-slots the two passes win.
inline bool use_two_pass_plan(int64_t seq_len, int64_t P) {
  return P <= kRowMaxP && P * seq_len > ((int64_t)1 << 24);
}
inline size_t plan_rows_bytes(int64_t seq_len, int64_t P, int64_t B) {
  return P > kRowMaxP ? 0 : align_up((size_t)B * plan_row_stride(plan_row_chunks(seq_len)) * (P + kRowHead) * 4, 256);
}

// P: streams of the launch (all requests), H: query heads.
inline size_t workspace_bytes_for(int n_splits, int64_t P, int64_t H, int64_t d, int64_t seq_len, int64_t B = 1) {
  const size_t cnt = align_up((size_t)P * 4, 256);
  const size_t sl = align_up((size_t)P * list_cap_for(seq_len) * 4, 256);
  const size_t ml = align_up((size_t)n_splits * P * H * sizeof(float2), 256);
  const size_t o = align_up((size_t)n_splits * P * H * d * sizeof(float), 256);
  const size_t qr = align_up((size_t)P * H * d * 4, 256);
  const size_t rw = plan_rows_bytes(seq_len, P / B, B);
  return 256 /*base alignment slack*/ + plan_bytes_for(B) + cnt + sl + ml + o + qr + rw;
}

inline Workspace carve_workspace(void* ws, int n_splits, int64_t P, int64_t H, int64_t d, int64_t seq_len,
                                 int64_t B = 1) {
  uintptr_t at = align_up((uintptr_t)ws, 256);
  Workspace w;
  w.cap = list_cap_for(seq_len);
  w.plan = reinterpret_cast<int32_t*>(at);
  at += plan_bytes_for(B);
  w.counts = reinterpret_cast<int32_t*>(at);
  at += align_up((size_t)P * 4, 256);
  w.slots = reinterpret_cast<int32_t*>(at);
  at += align_up((size_t)P * w.cap * 4, 256);
  w.part_ml = reinterpret_cast<float2*>(at);
  at += align_up((size_t)n_splits * P * H * sizeof(float2), 256);
  w.part_o = reinterpret_cast<float*>(at);
  at += align_up((size_t)n_splits * P * H * d * sizeof(float), 256);
  w.q_rot = reinterpret_cast<void*>(at);
  at += align_up((size_t)P * H * d * 4, 256);
  w.rows = plan_rows_bytes(seq_len, P / B, B) ? reinterpret_cast<int32_t*>(at) : nullptr;
  return w;
}

// --------------------------------------------------------- device helpers ---
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// round-to-nearest-even fp32 -> bf16 pair (one v_cvt_pk_bf16_f32 on gfx950)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// sum over aligned groups of G lanes (G a power of two, <= 64)
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Reductions across the four 16-lane rows of a wave with the gfx950 VALU
// lane swaps (no LDS round trip): permlane16_swap(x, x) returns, on every
// lane, {x of the even 16-lane row, x of the odd row} of its row pair (lane
// and lane ^ 16); permlane32_swap likewise {lower half, upper half} for lane
// and lane ^ 32.  Both lanes of a pair therefore compute the same value.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of G lanes (G in {8, 16, 32, 64}) with DPP lane
// moves fused into the adds (16-lane rows) and lane swaps across rows: no
// LDS round trip.  Every lane of a group ends with the group's sum.
template <int G>
__device__ __forceinline__ float group_sum_dpp(float v) {
  static_assert(G == 8 || G == 16 || G == 32 || G == 64, "group size");
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // lane ^ 1
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // lane ^ 2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));  // half-row mirror
  if constexpr (G >= 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));  // row mirror
  if constexpr (G >= 32) v = sum_xor16(v);
  if constexpr (G >= 64) v = sum_xor32(v);
  return v;
}


// ---------------------------------------------------- document prefix ---
// The plan kernel stores the document prefix length in plan[0]; consumers
// read it with one (wave-uniform) load.
__device__ __forceinline__ int load_doc_len(const int32_t* __restrict__ plan) {
  return __builtin_amdgcn_readfirstlane(plan[0]);
}

// ------------------------------------------------- visibility compaction ---
// Ascending compaction of the slots j in [from, seq_len) that stream s sees
// past the document prefix: sid[j] == s1 (= s + 1, its own slots) or
// sid[j] == 0 (document slots after the prefix).  [Parallel Prompting
// project page, "How it works", item 1: a stream sees the document and its
// own earlier tokens only.]
//
// All NT threads of the workgroup call it together.  The scan goes in
// chunks of NT*U slots; thread t owns the contiguous run of U slots starting
// at chunk_base + t*U, read as 16-byte int4 granules (the caller guarantees
// sid is 16-byte aligned; loads are unconditional at clamped granules, and a
// granule that straddles seq_len lies in one page with a valid element; its
// extra entries are ignored).  Matches go to list[0..cap) in slot order via
// one workgroup-wide exclusive scan per chunk: deterministic, no atomics.
// When more than cap slots match, the first cap are kept and *next is the
// slot after the last kept one; otherwise *next = seq_len.  `scan` is LDS
// scratch of NT/64 + 2 ints.
template <int NT, int U>
__device__ int collect_visible(const int32_t* __restrict__ sid, int64_t from, int64_t seq_len, int s1,
                               int* list, int cap, int64_t* next, int* scan) {
  static_assert(NT % 64 == 0 && U % 4 == 0 && U <= 64, "bad shape");
  constexpr int G = U / 4;  // int4 granules per thread
  constexpr int NW = NT / 64;
  constexpr int64_t CHUNK = (int64_t)NT * U;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int count = 0;
  int64_t cb = from & ~(int64_t)3;                        // granule-aligned chunk base
  const int64_t last_gran = (seq_len - 1) & ~(int64_t)3;  // last granule holding a slot < seq_len
  int64_t nxt = seq_len;
  while (cb < seq_len) {
    if (count == cap) {  // full at a chunk boundary: resume at this chunk
      nxt = cb;
      break;
    }
    const int64_t j0 = cb + (int64_t)tid * U;
    uint64_t match = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t jg = j0 + 4 * g;
      const int4 x = *reinterpret_cast<const int4*>(sid + (jg < last_gran ? jg : last_gran));
      const int ids[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // bitwise (not short-circuit) operators: the element is always read,
        // so the 16-byte load is never split into guarded narrower loads
        const int64_t j = jg + e;
        const unsigned vis = (unsigned)(j >= from) & (unsigned)(j < seq_len) &
                             ((unsigned)(ids[e] == 0) | (unsigned)(ids[e] == s1));
        match |= (uint64_t)vis << (4 * g + e);
      }
    }
    const int c = __popcll(match);
    int incl = c;  // wave-inclusive prefix of c
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) scan[wave] = incl;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int w = 0; w < NW; ++w) {
        const int t = scan[w];
        scan[w] = run;
        run += t;
      }
      scan[NW] = run;
    }
    __syncthreads();
    const int total = scan[NW];
    int pos = count + scan[wave] + incl - c;
    uint64_t mm = match;
    while (mm) {
      const int u = __ffsll((long long)mm) - 1;
      mm &= mm - 1;
      if (pos < cap) list[pos] = (int)(j0 + u);
      if (pos == cap - 1) scan[NW + 1] = (int)(j0 + u + 1);  // resume point after the last kept slot
      ++pos;
    }
    __syncthreads();
    if (count + total > cap) {  // uniform: every thread read the same total
      count = cap;
      nxt = scan[NW + 1];
      break;
    }
    count += total;
    cb += CHUNK;
    __syncthreads();  // scan[] is reused by the next chunk
  }
  *next = nxt;
  __syncthreads();  // list[] complete for every thread; scan[] free again
  return count;
}

// ---------------------------------------------------------- host launchers ---
// Each returns hipSuccess or the launch error.  All enqueue on `stream`.

// Visibility plan: doc_len into plan[0]; for every stream s, the number of
// slots j in [doc_len, seq_len) it sees (counts[s]) and the first cap of
// them in ascending order (slots[s*cap ...]).  With `rows` (plan_rows_bytes
// of scratch) and P <= kRowMaxP: two passes over chunks of the ids, O(T)
// work; otherwise one workgroup per stream over all ids.
hipError_t launch_plan(const int32_t* sid, int64_t seq_len, int P, int32_t* plan, int32_t* counts, int32_t* slots,
                       int64_t cap, hipStream_t stream, const Batch& bt = Batch(), int32_t* rows = nullptr);

// The same for a decode step that appends one slot per stream: the step
// starts at *base_len (device), stream s's new slot is *base_len + s and gets
// id s + 1 (written here), the plan covers seq_len = *base_len + P and
// plan[1] = seq_len.  max_len bounds seq_len; a base past it gives an empty
// plan.
hipError_t launch_plan_append(int32_t* sid, const int32_t* base_len, int64_t max_len, int P, int32_t* plan,
                              int32_t* counts, int32_t* slots, int64_t cap, hipStream_t stream,
                              const Batch& bt = Batch());

// Rotary embedding of the step's new queries and keys at their shared
// positions (from the plan), and the new keys and values written to the
// cache slots [seq_len - P, seq_len); the rotated queries go to q_rot.
// rope_base <= 0: no rotation.
hipError_t launch_append_rope(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              int P, int Hq, int Hkv, int d, pp_dtype_t dtype, double rope_base, const int32_t* plan,
                              const int32_t* counts, int64_t max_len, void* q_rot, hipStream_t stream, int B = 1,
                              int64_t kv_stride = 0, const int32_t* active = nullptr);

// Document part, all P queries of a head at once: split-K partial softmax
// states over [0, doc_len).  Returns the number of splits it will use via
// choose_doc_splits (host side, shape only).
// Last-level cache of the device (MI355X: 256 MB of Infinity Cache, shared
// by its XCDs).  A decode step whose key/value reads exceed it cannot keep
// them cached until the next step, so the rows each workgroup reads once
// are loaded with the non-temporal hint: they then do not evict what the
// step reads again (split partials, queries, slot lists) or force
// write-backs of dirty lines.  Smaller steps load them normally and may find
// them cached on the next call.
constexpr double kLastLevelCacheBytes = 256.0 * 1024 * 1024;

struct DocPlan {
  int n_splits;
  int qb;        // 16-query blocks per wave (bf16 MFMA path)
  int nw;        // waves per workgroup (bf16 MFMA path)
  int n_ptiles;  // query tiles per head
};
DocPlan choose_doc_plan(int64_t seq_len, int P, int H, int d, pp_dtype_t dtype, int num_cus);
// Queries per workgroup of the document kernel for this plan (its query tile).
int doc_query_tile(const DocPlan& plan, pp_dtype_t dtype);
// causal: prefill -- query i is slot i and query tile pt sees the document
// slots j < min((pt + 1) * tile, doc_len) with j <= i (one split); with out
// given, the rows of document slots (complete there) are written to it.
// (P: streams per request, H: key/value heads; the grid covers bt.B requests)
// stream_nt: load key/value tiles that only one workgroup reads with the
// non-temporal hint (see kLastLevelCacheBytes).
hipError_t launch_doc(const DocPlan& plan, const void* q, const void* k, const void* v, int64_t seq_len, int P,
                      int H, int d, pp_dtype_t dtype, float scale_log2, const Workspace& ws, hipStream_t stream,
                      bool causal = false, const Batch& bt = Batch(), void* out = nullptr, bool stream_nt = false);

// Per-question document part (the "batched requests" baseline): every
// stream reads the document itself.
int choose_batched_splits(int64_t seq_len, int P, int H, int num_cus);
// (P: streams per request, H: query heads)
hipError_t launch_batched_doc(int n_splits, const void* q, const void* k, const void* v, int64_t seq_len, int P,
                              int H, int d, pp_dtype_t dtype, float scale_log2, const Workspace& ws,
                              hipStream_t stream, const Batch& bt = Batch());

// Own-slot gather for every stream, then the fixed-order merge of the doc
// partials and the stream's own partial; writes out.
// (P: streams per request, H: query heads)
// stream_nt: load the own-slot rows with the non-temporal hint where no
// other workgroup reads them (no grouped heads).
hipError_t launch_tail_merge(int n_splits, const void* q, const void* k, const void* v,
                             const int32_t* sid, int64_t seq_len, int P, int H, int d, pp_dtype_t dtype,
                             float scale_log2, const Workspace& ws, void* out, hipStream_t stream,
                             const Batch& bt = Batch(), bool stream_nt = false);

// Prefill: for every query slot i in [doc_len, seq_len), the visible slots
// the document kernel (causal, query tile `tile`) left out -- j in
// [min((i / tile + 1) * tile, doc_len), i] with id 0 or id[i] -- compacted
// from stream_id, gathered, merged with the document partial of row i, and
// out[i] written (document slots were written by the document kernel).
hipError_t launch_prefill_rest(int n_splits, int tile, const void* q, const void* k, const void* v,
                               const int32_t* sid, int64_t seq_len, int H, int d, pp_dtype_t dtype, float scale_log2,
                               const Workspace& ws, void* out, hipStream_t stream, const Batch& bt = Batch());

}  // namespace pp
