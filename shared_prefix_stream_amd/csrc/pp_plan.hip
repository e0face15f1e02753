// Integer visibility plan on the device.
//
// Parallel Prompting packs the shared document first in the request and
// every stream's question and answer slots after it (project page,
// illustration: the document and all questions go into one sequence).  The
// leading run of document slots (id 0) is the part every stream sees; its
// length is found here on the device, so the host never reads device data.
#include "pp_internal.h"

namespace pp {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanIds = 16;                              // ids per thread per chunk (4 int4 loads)
constexpr int64_t kPlanChunk = (int64_t)kPlanThreads * kPlanIds;

// Workgroup b scans chunks b, b + kPlanWGs, ... in increasing order and
// records the first slot whose id is not 0; it stops at the first chunk that
// holds one.  Loads are unconditional (clamped granules), one round trip per
// chunk.
__global__ __launch_bounds__(kPlanThreads) void plan_doclen_kernel(const int32_t* __restrict__ sid,
                                                                   int64_t seq_len,
                                                                   int32_t* __restrict__ parts) {
  __shared__ int found;
  const int tid = threadIdx.x;
  if (tid == 0) found = 0x7fffffff;
  __syncthreads();
  const int64_t last_gran = (seq_len - 1) & ~(int64_t)3;
  for (int64_t cb = (int64_t)blockIdx.x * kPlanChunk; cb < seq_len; cb += kPlanWGs * kPlanChunk) {
    const int64_t j0 = cb + (int64_t)tid * kPlanIds;
    int first = 0x7fffffff;
#pragma unroll
    for (int g = kPlanIds / 4 - 1; g >= 0; --g) {
      const int64_t jg = j0 + 4 * g;
      const int4 x = *reinterpret_cast<const int4*>(sid + (jg < last_gran ? jg : last_gran));
      const int ids[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        // bitwise test so every element is read (the load is never split)
        const unsigned hit = (unsigned)(jg + e < seq_len) & (unsigned)(ids[e] != 0);
        first = hit ? (int)(jg + e) : first;
      }
    }
    if (first != 0x7fffffff) atomicMin(&found, first);
    __syncthreads();
    const bool done = found != 0x7fffffff;
    __syncthreads();  // every thread has read `found` before it can change again
    if (done) break;
  }
  if (tid == 0) parts[blockIdx.x] = found;
}

constexpr int kListThreads = 256;
constexpr int kListScanU = 64;
constexpr int kListCap = 2048;

// One workgroup per stream: the same ascending compaction the tail kernel
// runs, written out for inspection.
__global__ __launch_bounds__(kListThreads) void plan_lists_kernel(const int32_t* __restrict__ sid,
                                                                  int64_t seq_len,
                                                                  const int32_t* __restrict__ parts,
                                                                  int32_t* __restrict__ doc_len_out,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ slots, int64_t cap) {
  __shared__ int list[kListCap];
  __shared__ int scan[kListThreads / 64 + 2];
  const int s = blockIdx.x;
  const int doc_len = doc_prefix_from_parts(parts, seq_len);
  if (s == 0 && threadIdx.x == 0) *doc_len_out = doc_len;
  int64_t from = doc_len;
  int64_t total = 0;
  while (from < seq_len) {
    int64_t next;
    const int n = collect_visible<kListThreads, kListScanU>(sid, from, seq_len, s + 1, list, kListCap, &next, scan);
    for (int i = threadIdx.x; i < n; i += kListThreads)
      if (total + i < cap) slots[(int64_t)s * cap + total + i] = list[i];
    total += n;
    from = next;
    __syncthreads();  // list[] is refilled by the next round
  }
  if (threadIdx.x == 0) counts[s] = (int32_t)total;
}

}  // namespace

hipError_t launch_plan_doclen(const int32_t* sid, int64_t seq_len, int32_t* parts, hipStream_t stream) {
  plan_doclen_kernel<<<kPlanWGs, kPlanThreads, 0, stream>>>(sid, seq_len, parts);
  return hipGetLastError();
}

hipError_t launch_plan_lists(const int32_t* sid, int64_t seq_len, int P, const int32_t* parts, int32_t* doc_len,
                             int32_t* counts, int32_t* slots, int64_t cap, hipStream_t stream) {
  plan_lists_kernel<<<P, kListThreads, 0, stream>>>(sid, seq_len, parts, doc_len, counts, slots, cap);
  return hipGetLastError();
}

}  // namespace pp
