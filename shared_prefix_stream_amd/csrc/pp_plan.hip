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

constexpr int kPlanThreads = 1024;
constexpr int kPlanUnroll = 16;

// doc_len = index of the first slot whose id is not 0 (or seq_len).  One
// workgroup scans in chunks of 16K slots, 16 independent loads per thread
// in flight, and stops at the first chunk that holds a non-zero id.
__global__ __launch_bounds__(kPlanThreads) void plan_doclen_kernel(const int32_t* __restrict__ sid,
                                                                   int64_t seq_len,
                                                                   int32_t* __restrict__ doc_len) {
  __shared__ int found;
  const int tid = threadIdx.x;
  if (tid == 0) found = 0x7fffffff;
  __syncthreads();
  for (int64_t base = 0; base < seq_len; base += (int64_t)kPlanThreads * kPlanUnroll) {
    int ids[kPlanUnroll];
#pragma unroll
    for (int u = 0; u < kPlanUnroll; ++u) {
      const int64_t j = base + (int64_t)u * kPlanThreads + tid;
      ids[u] = j < seq_len ? sid[j] : 0;
    }
    int first = 0x7fffffff;
#pragma unroll
    for (int u = kPlanUnroll - 1; u >= 0; --u)
      if (ids[u] != 0) first = (int)(base + (int64_t)u * kPlanThreads + tid);
    if (first != 0x7fffffff) atomicMin(&found, first);
    __syncthreads();
    const bool done = found != 0x7fffffff;
    __syncthreads();  // every thread has read `found` before the next chunk
    if (done) break;
  }
  if (tid == 0) *doc_len = found == 0x7fffffff ? (int32_t)seq_len : found;
}

constexpr int kListThreads = 256;

// One workgroup per stream: the same ascending compaction the tail kernel
// runs, written out for inspection.
__global__ __launch_bounds__(kListThreads) void plan_lists_kernel(const int32_t* __restrict__ sid,
                                                                  int64_t seq_len,
                                                                  const int32_t* __restrict__ doc_len,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ slots, int64_t cap) {
  __shared__ int list[kCollectChunk];
  __shared__ int scan[kListThreads / 64 + 1];
  const int s = blockIdx.x;
  int64_t from = *doc_len;
  int64_t total = 0;
  while (from < seq_len) {
    int64_t next;
    const int n = collect_visible<kListThreads>(sid, from, seq_len, s + 1, list, kCollectChunk, &next, scan);
    for (int i = threadIdx.x; i < n; i += kListThreads)
      if (total + i < cap) slots[(int64_t)s * cap + total + i] = list[i];
    total += n;
    from = next;
    __syncthreads();  // list[] is refilled by the next round
  }
  if (threadIdx.x == 0) counts[s] = (int32_t)total;
}

}  // namespace

hipError_t launch_plan_doclen(const int32_t* sid, int64_t seq_len, int32_t* doc_len, hipStream_t stream) {
  plan_doclen_kernel<<<1, kPlanThreads, 0, stream>>>(sid, seq_len, doc_len);
  return hipGetLastError();
}

hipError_t launch_plan_lists(const int32_t* sid, int64_t seq_len, int P, const int32_t* doc_len,
                             int32_t* counts, int32_t* slots, int64_t cap, hipStream_t stream) {
  plan_lists_kernel<<<P, kListThreads, 0, stream>>>(sid, seq_len, doc_len, counts, slots, cap);
  return hipGetLastError();
}

}  // namespace pp
