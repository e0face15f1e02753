// Internal declarations shared by the HIP translation units of libppattn.
// gfx950 (CDNA4) only: 64-wide wavefronts, MFMA bf16 16x16x32, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ppattn.h"

namespace pp {

// ----------------------------------------------------------------- types ---
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Workspace layout (byte offsets from a 256-byte aligned base):
//   [0, 256)              int32 doc_len (leading run of id-0 slots)
//   [256, 256 + ML)       float2 part_ml[n_splits][P][H]  (m in log2 units, l)
//   [..., + O)            float  part_o [n_splits][P][H][d] (unnormalised)
struct Workspace {
  int32_t* doc_len;
  float2* part_ml;
  float* part_o;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline size_t workspace_bytes_for(int n_splits, int64_t P, int64_t H, int64_t d) {
  size_t ml = align_up((size_t)n_splits * P * H * sizeof(float2), 256);
  size_t o = align_up((size_t)n_splits * P * H * d * sizeof(float), 256);
  return 256 /*base alignment slack*/ + 256 /*doc_len*/ + ml + o;
}

inline Workspace carve_workspace(void* ws, int n_splits, int64_t P, int64_t H) {
  uintptr_t base = align_up((uintptr_t)ws, 256);
  Workspace w;
  w.doc_len = reinterpret_cast<int32_t*>(base);
  w.part_ml = reinterpret_cast<float2*>(base + 256);
  size_t ml = align_up((size_t)n_splits * P * H * sizeof(float2), 256);
  w.part_o = reinterpret_cast<float*>(base + 256 + ml);
  return w;
}

// --------------------------------------------------------- device helpers ---
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(unsigned short, a) |
         ((uint32_t)__builtin_bit_cast(unsigned short, b) << 16);
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

// ------------------------------------------------- visibility compaction ---
// Ascending compaction of the slots j in [from, seq_len) that stream s sees
// past the document prefix: sid[j] == s1 (= s + 1, its own slots) or
// sid[j] == 0 (document slots after the prefix).  [Parallel Prompting
// project page, "How it works", item 1: a stream sees the document and its
// own earlier tokens only.]
//
// All NT threads of the workgroup call it together.  Work goes in chunks of
// kCollectChunk slots; thread t owns the contiguous run of U = chunk / NT
// slots starting at chunk_base + t*U, read as 16-byte int4 granules (the
// caller guarantees sid is 16-byte aligned; a granule that straddles
// seq_len lies in one page with a valid element, and its extra entries are
// ignored).  Matches are written to list[0..) in slot order using one
// workgroup-wide exclusive scan per chunk, so the order is deterministic and
// no atomics are used.  Collection stops before a chunk whose matches would
// not fit in `cap` (cap >= kCollectChunk), returning the count and the first
// slot not yet examined in *next.  `scan` is LDS scratch of NT/64 + 1 ints.
constexpr int kCollectChunk = 4096;

template <int NT>
__device__ int collect_visible(const int32_t* __restrict__ sid, int64_t from, int64_t seq_len, int s1,
                               int* list, int cap, int64_t* next, int* scan) {
  static_assert(NT % 64 == 0 && kCollectChunk % (4 * NT) == 0, "bad workgroup size");
  constexpr int U = kCollectChunk / NT;  // slots per thread per chunk
  constexpr int G = U / 4;               // int4 granules per thread
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int count = 0;
  int64_t cb = from & ~(int64_t)3;  // granule-aligned chunk base
  while (cb < seq_len) {
    const int64_t j0 = cb + (int64_t)tid * U;
    int ids[U];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      int4 x = make_int4(-1, -1, -1, -1);
      if (j0 + 4 * g < seq_len) x = *reinterpret_cast<const int4*>(sid + j0 + 4 * g);
      ids[4 * g + 0] = x.x;
      ids[4 * g + 1] = x.y;
      ids[4 * g + 2] = x.z;
      ids[4 * g + 3] = x.w;
    }
    unsigned match = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = j0 + u;
      const bool vis = (j >= from) && (j < seq_len) && (ids[u] == 0 || ids[u] == s1);
      match |= (vis ? 1u : 0u) << u;
    }
    const int c = __popc(match);
    // workgroup exclusive scan of c
    int incl = c;
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
    if (count + total > cap) {
      __syncthreads();
      break;  // uniform: every thread read the same total
    }
    int pos = count + scan[wave] + incl - c;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (match & (1u << u)) list[pos++] = (int)(j0 + u);
    count += total;
    cb += kCollectChunk;
    __syncthreads();  // scan[] is reused by the next chunk
  }
  *next = cb < seq_len ? cb : seq_len;
  __syncthreads();  // list[] complete for every thread
  return count;
}

// ---------------------------------------------------------- host launchers ---
// Each returns hipSuccess or the launch error.  All enqueue on `stream`.

// doc_len = leading run of id-0 slots of stream_id[0, seq_len).
hipError_t launch_plan_doclen(const int32_t* sid, int64_t seq_len, int32_t* doc_len, hipStream_t stream);

// Integer plan inspection (pp_attn_plan).
hipError_t launch_plan_lists(const int32_t* sid, int64_t seq_len, int P, const int32_t* doc_len,
                             int32_t* counts, int32_t* slots, int64_t cap, hipStream_t stream);

// Document part, all P queries of a head at once: split-K partial softmax
// states over [0, doc_len).  Returns the number of splits it will use via
// choose_doc_splits (host side, shape only).
struct DocPlan {
  int n_splits;
  int qb;        // 16-query blocks per wave (bf16 MFMA path)
  int n_ptiles;  // query tiles per head
};
DocPlan choose_doc_plan(int64_t seq_len, int P, int H, int d, pp_dtype_t dtype, int num_cus);
hipError_t launch_doc(const DocPlan& plan, const void* q, const void* k, const void* v, int P, int H,
                      int d, pp_dtype_t dtype, float scale_log2, const Workspace& ws, hipStream_t stream);

// Per-question document part (the "batched requests" baseline): every
// stream reads the document itself.
int choose_batched_splits(int64_t seq_len, int P, int H, int num_cus);
hipError_t launch_batched_doc(int n_splits, const void* q, const void* k, const void* v, int P, int H,
                              int d, pp_dtype_t dtype, float scale_log2, const Workspace& ws,
                              hipStream_t stream);

// Own-slot gather for every stream, then the fixed-order merge of the doc
// partials and the stream's own partial; writes out.
hipError_t launch_tail_merge(int n_splits, const void* q, const void* k, const void* v,
                             const int32_t* sid, int64_t seq_len, int P, int H, int d, pp_dtype_t dtype,
                             float scale_log2, const Workspace& ws, void* out, hipStream_t stream);

}  // namespace pp
