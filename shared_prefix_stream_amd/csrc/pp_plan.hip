// Integer visibility plan on the device.
//
// Parallel Prompting packs the shared document first in the request and
// every stream's question and answer slots after it (project page,
// illustration: the document and all questions go into one sequence).  The
// leading run of document slots (id 0) is the part every stream sees and is
// handled as one dense block; past it, each stream sees only its own slots
// and any later document slot ("How it works", item 1).  One workgroup per
// stream finds the prefix length and compacts that stream's visible slots,
// once per step, for the gather kernel.  Nothing is read back on the host.
#include "pp_internal.h"

namespace pp {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanNW = kPlanThreads / 64;                       // 16 waves: 4 per SIMD hide latency
constexpr int kPlanG = 8;                                        // granule rows per wave per round
constexpr int64_t kPlanWaveSpan = (int64_t)64 * kPlanG * 4;      // 2K slots per wave per round
constexpr int64_t kPlanChunk = kPlanWaveSpan * kPlanNW;          // 32K slots per workgroup per round

// Workgroup = one stream.  In a round wave w owns the 2K slots starting at
// wb = chunk_base + 2K*w, as 8 rows of 256: lane l, row g holds the int4
// granule of slots wb + 4*(64g + l) .. +3 (coalesced 1 KB wave-wide loads,
// all in flight, unconditional at clamped granules).  Per round:
//   1. while the document prefix is open: the first non-zero id of the
//      chunk (wave minimum, then workgroup minimum) closes it;
//   2. the slots j >= doc_len the stream sees (id 0 or s+1) are ranked in
//      slot order -- within a row by ballots, across rows and waves by
//      running totals -- and stored at slots[s*cap + rank] (ranks >= cap
//      are counted only).
// One global round trip per 32K slots; no atomics decide positions.
//
// APPEND (a decode step that appends one slot per stream): request b's
// step starts at base = base_len[b], stream s's new slot is base + s, and
// the plan covers seq_len = base + P, where the `seq_len` argument is only
// the largest allowed length.  The ids of [base, base + P) are taken as
// s + 1 whatever memory holds (other workgroups may be writing them),
// workgroup (s, b) stores its own, and plan[B + b] = seq_len (plan[1] for
// one request).  A base outside [0, limit - P] gives an empty plan
// (plan[b] = plan[B + b] = 0, no counts, nothing written): an idle request.
//
// Several requests (grid.y = B, single-request layout otherwise): workgroup
// (s, b) plans stream s of request b over that request's ids and length;
// plan[b] is its document length, its counts and lists are those of launch
// stream b * P + s.
template <bool APPEND>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ sid, int64_t seq_len,
                                                            int32_t* __restrict__ plan, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ slots, int64_t cap,
                                                            int32_t* sid_out, const int32_t* base_len, Batch bt) {
  __shared__ int found;
  __shared__ int wsum[kPlanNW];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y;
  const int s = blockIdx.x;                     // stream within the request
  const int sl = b * (int)gridDim.x + s;        // stream of the launch
  sid += b * bt.id_stride;
  if constexpr (APPEND) sid_out += b * bt.id_stride;
  if constexpr (!APPEND) seq_len = request_len(bt, b, seq_len);
  const unsigned live = stream_active(bt, sl) ? 1u : 0u;  // a retired stream lists nothing
  const int s1 = s + 1;
  const uint64_t below = (1ull << lane) - 1ull;  // lanes before this one
  int64_t app = seq_len;  // first appended slot
  if constexpr (APPEND) {
    // head: doc_len of the B requests, then their seq_len
    const int64_t bb = __builtin_amdgcn_readfirstlane(base_len[b]);
    const int64_t P = gridDim.x;
    if (bb < 0 || bb > seq_len - P) {  // an idle request: empty plan, no ids
      if (tid == 0) {
        counts[sl] = 0;
        if (s == 0) plan[b] = plan[gridDim.y + b] = 0;
      }
      return;
    }
    app = bb;
    seq_len = bb + P;
  }
  if (tid == 0) found = 0x7fffffff;
  __syncthreads();
  const int64_t last_gran = (seq_len - 1) & ~(int64_t)3;
  int64_t doc_len = -1;  // unknown until a non-zero id is seen
  int64_t total = 0;
  for (int64_t cb = 0; cb < seq_len; cb += kPlanChunk) {
    const int64_t wb = cb + wave * kPlanWaveSpan;  // this wave's first slot
    int4 x[kPlanG];
#pragma unroll
    for (int g = 0; g < kPlanG; ++g) {
      const int64_t jg = wb + 4 * (64 * g + lane);
      const int64_t jl = jg < last_gran ? jg : last_gran;
      x[g] = *reinterpret_cast<const int4*>(sid + jl);
      if constexpr (APPEND) {
        x[g].x = jl >= app ? (int)(jl - app) + 1 : x[g].x;
        x[g].y = jl + 1 >= app ? (int)(jl + 1 - app) + 1 : x[g].y;
        x[g].z = jl + 2 >= app ? (int)(jl + 2 - app) + 1 : x[g].z;
        x[g].w = jl + 3 >= app ? (int)(jl + 3 - app) + 1 : x[g].w;
      }
    }
    // slot wb + 4*(64g + lane) + e is valid iff 4*(64g + lane) + e < hi
    const int hi = (int)max<int64_t>(min<int64_t>(seq_len - wb, kPlanWaveSpan), 0);
    // 1. document prefix
    if (doc_len < 0) {
      // this wave's first non-zero id: the first row whose ballot is
      // non-empty, its first lane, then that lane's first element
      int first = 0x7fffffff;
#pragma unroll
      for (int g = 0; g < kPlanG; ++g) {
        const int r0 = 4 * (64 * g + lane);
        const unsigned valid = (1u << min(max(hi - r0, 0), 4)) - 1u;
        const unsigned nz = (((unsigned)(x[g].x != 0)) | ((unsigned)(x[g].y != 0) << 1) |
                             ((unsigned)(x[g].z != 0) << 2) | ((unsigned)(x[g].w != 0) << 3)) & valid;
        const uint64_t b = __builtin_amdgcn_ballot_w64(nz != 0);
        if (first == 0x7fffffff && b != 0) {  // uniform
          const int l0 = __builtin_ctzll(b);
          first = 4 * (64 * g + l0) + __builtin_ctz((unsigned)__builtin_amdgcn_readlane((int)nz, l0));
        }
      }
      if (lane == 0 && first != 0x7fffffff) atomicMin(&found, (int)(wb + first));
      __syncthreads();
      const int f = found;
      __syncthreads();  // every thread has read `found` before it can change again
      if (f != 0x7fffffff) doc_len = f;
      else if (cb + kPlanChunk >= seq_len) doc_len = seq_len;  // no non-document slot at all
      if (doc_len < 0) continue;  // the whole chunk is document (uniform)
    }
    // 2. visible slots past the prefix, ranked in slot order: r in [lo, hi)
    const int lo = (int)max<int64_t>(min<int64_t>(doc_len - wb, kPlanWaveSpan), 0);
    unsigned m[kPlanG];
    int row_base[kPlanG];
    int wave_total = 0;
#pragma unroll
    for (int g = 0; g < kPlanG; ++g) {
      const int ids[4] = {x[g].x, x[g].y, x[g].z, x[g].w};
      m[g] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * (64 * g + lane) + e;
        const unsigned vis = (unsigned)(r >= lo) & (unsigned)(r < hi) & live &
                             ((unsigned)(ids[e] == 0) | (unsigned)(ids[e] == s1));
        m[g] |= vis << e;
      }
      row_base[g] = wave_total;
#pragma unroll
      for (int e = 0; e < 4; ++e) wave_total += __popcll(__builtin_amdgcn_ballot_w64((m[g] >> e) & 1u));
    }
    if (lane == 0) wsum[wave] = wave_total;
    __syncthreads();
    int before = 0, chunk_total = 0;
#pragma unroll
    for (int w = 0; w < kPlanNW; ++w) {
      const int t = wsum[w];
      before += w < wave ? t : 0;
      chunk_total += t;
    }
    if (wave_total > 0) {  // uniform
#pragma unroll
      for (int g = 0; g < kPlanG; ++g) {
        // matches of this row in earlier lanes (all four bits), then own bits
        int rank = row_base[g];
#pragma unroll
        for (int e = 0; e < 4; ++e) rank += __popcll(__builtin_amdgcn_ballot_w64((m[g] >> e) & 1u) & below);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((m[g] >> e) & 1u) {
            const int64_t pos = total + before + rank;
            if (pos < cap) slots[(int64_t)sl * cap + pos] = (int32_t)(wb + 4 * (64 * g + lane) + e);
            ++rank;
          }
        }
      }
    }
    total += chunk_total;
    // wsum[] is rewritten next round (the last round needs no barrier: it
    // would only wait for this round's stores)
    if (cb + kPlanChunk < seq_len) __syncthreads();
  }
  if (tid == 0) {
    counts[sl] = (int32_t)total;
    if (s == 0) plan[b] = (int32_t)(doc_len < 0 ? seq_len : doc_len);
    if constexpr (APPEND) {
      sid_out[app + s] = s1;
      if (s == 0) plan[gridDim.y + b] = (int32_t)seq_len;
    }
  }
}

}  // namespace

hipError_t launch_plan(const int32_t* sid, int64_t seq_len, int P, int32_t* plan, int32_t* counts, int32_t* slots,
                       int64_t cap, hipStream_t stream, const Batch& bt) {
  plan_kernel<false><<<dim3(P, bt.B), kPlanThreads, 0, stream>>>(sid, seq_len, plan, counts, slots, cap, nullptr,
                                                                 nullptr, bt);
  return hipGetLastError();
}

hipError_t launch_plan_append(int32_t* sid, const int32_t* base_len, int64_t max_len, int P, int32_t* plan,
                              int32_t* counts, int32_t* slots, int64_t cap, hipStream_t stream, const Batch& bt) {
  plan_kernel<true><<<dim3(P, bt.B), kPlanThreads, 0, stream>>>(sid, max_len, plan, counts, slots, cap, sid, base_len,
                                                                bt);
  return hipGetLastError();
}

}  // namespace pp
