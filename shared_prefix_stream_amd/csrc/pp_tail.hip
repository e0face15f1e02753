// Per-stream part of one decode step, and the final merge.
//
// After the document, a stream sees only its own slots (its question and
// its earlier answer tokens) plus any document slot placed later (Parallel
// Prompting project page, "How it works", item 1).  Instead of testing the
// stream rule on every slot for every stream -- which makes each stream scan
// its siblings' answers, the cost the project page's "More results" section
// blames for the smaller gain on long answers -- the plan kernel has listed
// the slots each stream sees (ascending) and this kernel gathers only those
// rows.  A stream whose list did not fit the plan's capacity compacts it
// here, in chunks (one workgroup-wide scan per 16K slots).
//
// Workgroup = one stream x one group of GW heads (a contiguous GW*d-element
// slice of every K/V row, so each wave-wide 16-byte load is 1 KB contiguous).
// Its 4 waves are substreams.  Substream w first merges the document split
// partial states w, w+4, w+8, ... (written by the document kernel, or by the
// per-question baseline) -- their loads are issued at kernel start, so they
// overlap the list loads -- then folds in list entries [w*U, w*U + U),
// [w*U + 4U, ...), ... with an online softmax.  The four states are merged
// in substream order and the output slice is written.  Every step has a
// fixed order, so the result is bitwise reproducible.  Splitting streams by
// head group gives P * H/GW small workgroups, which spread streams of
// different tail lengths evenly over the CUs.
#include <math.h>

#include "pp_internal.h"

namespace pp {
namespace {

constexpr int kTailThreads = 256;  // 4 waves = 4 token substreams of one head group
constexpr int kTailNTS = kTailThreads / 64;
constexpr int kTailU = 4;          // list entries per substream step (loads in flight)
constexpr int kTailScanU = 64;     // stream ids per thread per compaction chunk (16K-slot chunks)
constexpr int kTailCap = 2048;     // visible slots compacted per round
constexpr int kMergeBatch = 2;     // document split partials a substream loads at once
constexpr int kTailNI = 2;         // 16-byte vectors per lane per K row

template <typename T, int D>
struct TailShape {
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte vector
  static constexpr int LPH = D / VEC;              // lanes sharing one head
  static constexpr int HPI = 64 / LPH;             // heads per wave-wide vector load
  static constexpr int GW = kTailNI * HPI;         // heads per workgroup
};

template <typename T>
__device__ __forceinline__ void to_f32(const u32x4& w, float* f);
template <>
__device__ __forceinline__ void to_f32<uint16_t>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}
template <>
__device__ __forceinline__ void to_f32<float>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}

template <typename T>
__device__ __forceinline__ u32x4 from_f32(const float* f);
template <>
__device__ __forceinline__ u32x4 from_f32<uint16_t>(const float* f) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}
template <>
__device__ __forceinline__ u32x4 from_f32<float>(const float* f) {
  return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
}

// (M, Ls, A) <- merge with (m2, l2, A2); states with m = -inf are empty.
// Branch-free, so loads of later states are not held behind this one.
template <int VEC>
__device__ __forceinline__ void merge_state(float& M, float& Ls, float* A, float m2, float l2, const float* A2) {
  const float Mn = fmaxf(M, m2);
  const float ref = Mn == -INFINITY ? 0.f : Mn;  // both empty: weights exp2(-inf) = 0
  const float a = fast_exp2(M - ref), b = fast_exp2(m2 - ref);
  Ls = Ls * a + l2 * b;
#pragma unroll
  for (int e = 0; e < VEC; ++e) A[e] = A[e] * a + A2[e] * b;
  M = Mn;
}

// PREFILL: blockIdx.x is a query slot i (q, out and the partials have one
// row per slot), and its list is compacted here from stream_id: the slots
// j in [min((i / tile + 1) * tile, doc_len), i] with id 0 or id[i] -- what
// the causal document kernel did not cover of i's visible set.  Slots below
// doc_len are complete in the document kernel, which wrote them.
//
// NT (decode without grouped heads): a stream's rows are read by its own
// workgroups only, each its own slice, once per step: they are loaded
// non-temporal, so that they do not evict what the step reads again.
template <typename T, int D, bool PREFILL, bool NT = false>
// (at most 128 VGPRs: four workgroups per CU)
__global__ __launch_bounds__(kTailThreads, 4) void tail_merge_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ sid,
    int64_t seq_len, int P, int H, float c, const int32_t* __restrict__ plan, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ slots, int64_t cap, int n_splits, const float* __restrict__ part_o,
    const float2* __restrict__ part_ml, T* __restrict__ out, const int32_t* __restrict__ dyn_len, int tile,
    Batch bt) {
  using S = TailShape<T, D>;
  constexpr int VEC = S::VEC, LPH = S::LPH, HPI = S::HPI, GW = S::GW;
  constexpr int RED = kTailNI * (VEC + 2);  // floats per lane in the substream merge

  __shared__ int list[kTailCap];
  __shared__ int scan[kTailNTS + 2];
  __shared__ float red[(kTailNTS - 1) * RED * 64];

  // s: stream of the launch; sr: the same stream within its request b
  // (several requests: each has its own ids, caches and document length;
  // grouped key/value heads: query head h reads key/value head h / G)
  const int s = blockIdx.x, hg = blockIdx.y;
  const int b = PREFILL ? 0 : s / P, sr = PREFILL ? s : s % P;
  const int Pt = PREFILL ? P : P * bt.B;
  sid += b * bt.id_stride;
  k += b * bt.kv_stride;
  v += b * bt.kv_stride;
  plan += b;
  // (the substream index is wave-uniform; readfirstlane lets the compiler know)
  const int tid = threadIdx.x, ts = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t row = (int64_t)(H / bt.G) * D;  // key/value heads
  if (PREFILL && s < load_doc_len(plan)) return;  // a document slot: written by the document kernel
  if (!PREFILL && !stream_active(bt, s)) {  // a retired stream: zeros, no work (workgroup-uniform)
    const int head0 = hg * S::GW;
    const int nel = (min(H, head0 + S::GW) - head0) * D;
    T* o = out + ((int64_t)s * H + head0) * D;
    for (int e = tid * VEC; e < nel; e += kTailThreads * VEC) *reinterpret_cast<u32x4*>(o + e) = u32x4{0u, 0u, 0u, 0u};
    return;
  }

  // lane covers head head[i], dims d0[i] .. +VEC of its 16-byte vector i;
  // lanes of heads past H use head 0 for their (unconditional) loads and
  // discard the results
  int head[kTailNI], safe_head[kTailNI], d0[kTailNI];
  bool valid[kTailNI];
#pragma unroll
  for (int i = 0; i < kTailNI; ++i) {
    head[i] = hg * GW + i * HPI + lane / LPH;
    d0[i] = (lane % LPH) * VEC;
    valid[i] = head[i] < H;
    safe_head[i] = valid[i] ? head[i] : 0;
  }

  float qv[kTailNI][VEC], mm[kTailNI], ll[kTailNI], acc[kTailNI][VEC];
#pragma unroll
  for (int i = 0; i < kTailNI; ++i) {
    to_f32<T>(*reinterpret_cast<const u32x4*>(q + ((int64_t)s * H + safe_head[i]) * D + d0[i]), qv[i]);
    mm[i] = -INFINITY;
    ll[i] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[i][e] = 0.f;
  }

  // ---- this substream's share of the document split partials ---------------
  // splits ts, ts + NTS, ...; loaded kMergeBatch at a time (indices past the
  // last split re-read split 0 and are skipped), merged in split order
  for (int sp0 = ts; sp0 < n_splits; sp0 += kTailNTS * kMergeBatch) {
    float2 ml[kMergeBatch][kTailNI];
    float o2[kMergeBatch][kTailNI][VEC];
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const int spb = sp0 + b * kTailNTS;
      const int sp = spb < n_splits ? spb : 0;
#pragma unroll
      for (int i = 0; i < kTailNI; ++i) {
        const int64_t sh = ((int64_t)sp * Pt + s) * H + safe_head[i];
        ml[b][i] = part_ml[sh];
        const float* src = part_o + sh * D + d0[i];
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const float4 x = *reinterpret_cast<const float4*>(src + e);
          o2[b][i][e] = x.x;
          o2[b][i][e + 1] = x.y;
          o2[b][i][e + 2] = x.z;
          o2[b][i][e + 3] = x.w;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b)
      if (sp0 + b * kTailNTS < n_splits)
#pragma unroll
        for (int i = 0; i < kTailNI; ++i) merge_state<VEC>(mm[i], ll[i], acc[i], ml[b][i].x, ml[b][i].y, o2[b][i]);
  }

  // ---- own slots (and late document slots), gathered ------------------------
  // fold list entries [0, n) of `lst` into this substream's state
  auto gather = [&](const int* lst, int n) {
    for (int base = ts * kTailU; base < n; base += kTailNTS * kTailU) {
      // unconditional loads (entries past the end re-read the last one) so
      // that all of them are in flight together
      u32x4 kr[kTailU][kTailNI], vr[kTailU][kTailNI];
#pragma unroll
      for (int u = 0; u < kTailU; ++u) {
        const int j = lst[min(base + u, n - 1)];
#pragma unroll
        for (int i = 0; i < kTailNI; ++i) {
          const int64_t off = (int64_t)j * row + (int64_t)(safe_head[i] / bt.G) * D + d0[i];
          if constexpr (NT) {
            kr[u][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
            vr[u][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
          } else {
            kr[u][i] = *reinterpret_cast<const u32x4*>(k + off);
            vr[u][i] = *reinterpret_cast<const u32x4*>(v + off);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kTailU; ++u) {
        if (base + u >= n) break;  // uniform across the wave
#pragma unroll
        for (int i = 0; i < kTailNI; ++i) {
          float kf[VEC], vf[VEC];
          to_f32<T>(kr[u][i], kf);
          to_f32<T>(vr[u][i], vf);
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) dot = fmaf(qv[i][e], kf[e], dot);
          dot = group_sum_dpp<LPH>(dot);
          const float t = dot * c;
          const float mn = fmaxf(mm[i], t);
          const float alpha = fast_exp2(mm[i] - mn);
          const float p = fast_exp2(t - mn);
          ll[i] = ll[i] * alpha + p;
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[i][e] = fmaf(p, vf[e], acc[i][e] * alpha);
          mm[i] = mn;
        }
      }
    }
  };
  // (wave-uniform: stated so the gather loop's control stays on the scalar unit)
  if constexpr (PREFILL) {
    const int s1 = __builtin_amdgcn_readfirstlane(sid[s]);
    int64_t from = min<int64_t>((int64_t)(s / tile + 1) * tile, load_doc_len(plan));
    const int64_t len = (int64_t)s + 1;
    while (from < len) {
      int64_t next;
      const int n = collect_visible<kTailThreads, kTailScanU>(sid, from, len, s1, list, kTailCap, &next, scan);
      gather(list, n);
      from = next;
      __syncthreads();  // list[] is refilled by the next round
    }
  } else {
  const int count = __builtin_amdgcn_readfirstlane(counts[s]);
  if (count <= cap) {
    gather(slots + (int64_t)s * cap, count);  // the plan's list (global, L2-resident)
  } else {
    // list longer than the plan kept: compact it here, chunk by chunk
    // (an appending step's length is on the device; seq_len bounds it)
    const int64_t len = dyn_len ? min<int64_t>(__builtin_amdgcn_readfirstlane(dyn_len[0]), seq_len)
                                : request_len(bt, b, seq_len);
    int64_t from = load_doc_len(plan);
    while (from < len) {
      int64_t next;
      const int n = collect_visible<kTailThreads, kTailScanU>(sid, from, len, sr + 1, list, kTailCap, &next, scan);
      gather(list, n);
      from = next;
      __syncthreads();  // list[] is refilled by the next round
    }
  }
  }

  // ---- merge token substreams (fixed order 0, 1, ..., NTS-1) -----------------
  if (ts > 0) {
    float* r = red + (size_t)(ts - 1) * RED * 64;
#pragma unroll
    for (int i = 0; i < kTailNI; ++i) {
      r[(i * (VEC + 2) + 0) * 64 + lane] = mm[i];
      r[(i * (VEC + 2) + 1) * 64 + lane] = ll[i];
#pragma unroll
      for (int e = 0; e < VEC; ++e) r[(i * (VEC + 2) + 2 + e) * 64 + lane] = acc[i][e];
    }
  }
  __syncthreads();
  if (ts != 0) return;
#pragma unroll
  for (int t2 = 1; t2 < kTailNTS; ++t2) {
    const float* r = red + (size_t)(t2 - 1) * RED * 64;
#pragma unroll
    for (int i = 0; i < kTailNI; ++i) {
      float a2[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) a2[e] = r[(i * (VEC + 2) + 2 + e) * 64 + lane];
      merge_state<VEC>(mm[i], ll[i], acc[i], r[(i * (VEC + 2)) * 64 + lane], r[(i * (VEC + 2) + 1) * 64 + lane], a2);
    }
  }

  // ---- write ----------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < kTailNI; ++i) {
    if (!valid[i]) continue;
    float res[VEC];
    const float inv = ll[i] > 0.f ? 1.f / ll[i] : 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) res[e] = ll[i] > 0.f ? acc[i][e] * inv : 0.f;
    *reinterpret_cast<u32x4*>(out + ((int64_t)s * H + head[i]) * D + d0[i]) = from_f32<T>(res);
  }
}

template <typename T, int D, bool PREFILL = false>
hipError_t launch_tail_t(int n_splits, const void* q, const void* k, const void* v, const int32_t* sid,
                         int64_t seq_len, int P, int H, float c, const Workspace& ws, void* out, hipStream_t stream,
                         int tile = 0, const Batch& bt = Batch(), bool stream_nt = false) {
  using S = TailShape<T, D>;
  const dim3 grid(P * bt.B, (H + S::GW - 1) / S::GW);
  auto go = [&](auto kern) {
    return launch_kernel(kern, grid, dim3(kTailThreads), stream, static_cast<const T*>(q), static_cast<const T*>(k),
                         static_cast<const T*>(v), sid, seq_len, P, H, c, ws.plan, ws.counts, ws.slots, ws.cap,
                         n_splits, ws.part_o, ws.part_ml, static_cast<T*>(out), ws.dyn_len, tile, bt);
  };
  // (grouped heads: the query heads of a key/value head read the same rows)
  if constexpr (!PREFILL)
    if (stream_nt && bt.G == 1) return go(tail_merge_kernel<T, D, false, true>);
  return go(tail_merge_kernel<T, D, PREFILL>);
}

}  // namespace

hipError_t launch_tail_merge(int n_splits, const void* q, const void* k, const void* v, const int32_t* sid,
                             int64_t seq_len, int P, int H, int d, pp_dtype_t dtype, float c, const Workspace& ws,
                             void* out, hipStream_t stream, const Batch& bt, bool stream_nt) {
  const bool nt = stream_nt;
  if (dtype == PP_BF16)
    return d == 128 ? launch_tail_t<uint16_t, 128>(n_splits, q, k, v, sid, seq_len, P, H, c, ws, out, stream, 0, bt, nt)
                    : launch_tail_t<uint16_t, 64>(n_splits, q, k, v, sid, seq_len, P, H, c, ws, out, stream, 0, bt, nt);
  return d == 128 ? launch_tail_t<float, 128>(n_splits, q, k, v, sid, seq_len, P, H, c, ws, out, stream, 0, bt, nt)
                  : launch_tail_t<float, 64>(n_splits, q, k, v, sid, seq_len, P, H, c, ws, out, stream, 0, bt, nt);
}

hipError_t launch_prefill_rest(int n_splits, int tile, const void* q, const void* k, const void* v,
                               const int32_t* sid, int64_t seq_len, int H, int d, pp_dtype_t dtype, float c,
                               const Workspace& ws, void* out, hipStream_t stream, const Batch& bt) {
  const int P = (int)seq_len;  // one query per slot
  if (dtype == PP_BF16)
    return d == 128
               ? launch_tail_t<uint16_t, 128, true>(n_splits, q, k, v, sid, seq_len, P, H, c, ws, out, stream, tile, bt)
               : launch_tail_t<uint16_t, 64, true>(n_splits, q, k, v, sid, seq_len, P, H, c, ws, out, stream, tile, bt);
  return d == 128 ? launch_tail_t<float, 128, true>(n_splits, q, k, v, sid, seq_len, P, H, c, ws, out, stream, tile, bt)
                  : launch_tail_t<float, 64, true>(n_splits, q, k, v, sid, seq_len, P, H, c, ws, out, stream, tile, bt);
}

}  // namespace pp
