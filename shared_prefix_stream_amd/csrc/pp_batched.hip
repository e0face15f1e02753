// Per-question baseline ("batched requests"): the document part of the
// step computed as P independent requests, each one query against the whole
// document.  This is what a serving engine does when every question is its
// own request sharing a prefix-cached document: each decode step reads the
// document's keys and values once per question (Parallel Prompting project
// page, illustration "Inside decode step", and "How it works").
//
// Kernel: flash-decoding GEMV.  Workgroup = (stream s, head h, split); its 4
// waves sweep the split's document slots, each 16-byte lane load holding VEC
// elements of one slot's row, LPK lanes per slot (so one wave-wide load
// covers KPI slots).  Each lane group keeps its own online-softmax state
// (no cross-lane work per slot beyond the dot-product reduction); states are
// merged across lane groups and waves at the end, in a fixed order, and
// written as the split's partial state.  The tail kernel then gathers the
// stream's own slots and merges, exactly as for pp_attn_decode.  Workgroups
// are dispatched request-major (head fastest, stream outermost), as a
// per-request decode launch orders them; nothing co-schedules different
// requests onto the same document tiles on purpose.  With grouped key/value
// heads each query head reads its group's key/value head; with several
// Parallel Prompting requests (grid.z = B * P) each stream reads its own
// request's document.
#include <math.h>

#include "pp_internal.h"

namespace pp {
namespace {

constexpr int kBThreads = 256;
constexpr int kBU = 8;  // slots in flight per lane group

template <typename T>
__device__ __forceinline__ void to_f32b(const u32x4& w, float* f);
template <>
__device__ __forceinline__ void to_f32b<uint16_t>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}
template <>
__device__ __forceinline__ void to_f32b<float>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}

template <int VEC>
__device__ __forceinline__ void merge_b(float& M, float& Ls, float* A, float m2, float l2, const float* A2) {
  const float Mn = fmaxf(M, m2);
  const float ref = Mn == -INFINITY ? 0.f : Mn;  // both empty: weights exp2(-inf) = 0
  const float a = fast_exp2(M - ref), b = fast_exp2(m2 - ref);
  Ls = Ls * a + l2 * b;
#pragma unroll
  for (int e = 0; e < VEC; ++e) A[e] = A[e] * a + A2[e] * b;
  M = Mn;
}

template <typename T, int D>
__global__ __launch_bounds__(kBThreads) void batched_doc_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int P, int H, float c,
    const int32_t* __restrict__ plan, int64_t seq_len, int n_splits, float* __restrict__ part_o,
    float2* __restrict__ part_ml, Batch bt) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LPK = D / VEC;   // lanes per slot
  constexpr int KPI = 64 / LPK;  // slots per wave-wide load
  constexpr int NW = kBThreads / 64;
  __shared__ float red[NW][VEC + 2][LPK];

  const int h = blockIdx.x, split = blockIdx.y, s = blockIdx.z;  // s: stream of the launch
  if (!stream_active(bt, s)) return;                               // retired: the merge writes zeros
  const int b = s / P;                                             // its request
  // (the wave index is wave-uniform; readfirstlane lets the compiler know)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int kg = lane / LPK, dl = lane % LPK;
  const int64_t L = min<int64_t>(load_doc_len(plan + b), seq_len);
  const int64_t j_begin = split * L / n_splits, j_end = (split + 1) * L / n_splits;
  const int64_t row = (int64_t)(H / bt.G) * D;  // key/value heads
  const int hk = h / bt.G;
  k += b * bt.kv_stride;
  v += b * bt.kv_stride;

  float qv[VEC];
  to_f32b<T>(*reinterpret_cast<const u32x4*>(q + ((int64_t)s * H + h) * D + dl * VEC), qv);
  float m = -INFINITY, l = 0.f, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  for (int64_t blk = j_begin; blk < j_end; blk += (int64_t)NW * kBU * KPI) {
    u32x4 kr[kBU], vr[kBU];
#pragma unroll
    for (int u = 0; u < kBU; ++u) {
      // unconditional load (slots past the split's end re-read its last slot
      // and are skipped below), so all of them are in flight together
      const int64_t j = min(blk + (int64_t)(wave * kBU + u) * KPI + kg, j_end - 1);
      const int64_t off = j * row + (int64_t)hk * D + dl * VEC;
      kr[u] = *reinterpret_cast<const u32x4*>(k + off);
      vr[u] = *reinterpret_cast<const u32x4*>(v + off);
    }
#pragma unroll
    for (int u = 0; u < kBU; ++u) {
      const int64_t j = blk + (int64_t)(wave * kBU + u) * KPI + kg;
      float kf[VEC], vf[VEC];
      to_f32b<T>(kr[u], kf);
      to_f32b<T>(vr[u], vf);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) dot = fmaf(qv[e], kf[e], dot);
      dot = group_sum<LPK>(dot);
      if (j < j_end) {
        const float t = dot * c;
        const float mn = fmaxf(m, t);
        const float alpha = fast_exp2(m - mn);
        const float p = fast_exp2(t - mn);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = fmaf(p, vf[e], acc[e] * alpha);
        m = mn;
      }
    }
  }

  // merge the KPI lane-group states of this wave (lane groups 0,1 | 2,3 | ...)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    float a2[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) a2[e] = __shfl_xor(acc[e], off);
    // lower group first, so every lane computes the same ordered merge
    if (lane & off) {
      float mt = m2, lt = l2, at[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) at[e] = a2[e];
      merge_b<VEC>(mt, lt, at, m, l, acc);
      m = mt;
      l = lt;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = at[e];
    } else {
      merge_b<VEC>(m, l, acc, m2, l2, a2);
    }
  }
  if (kg == 0) {
    red[wave][0][dl] = m;
    red[wave][1][dl] = l;
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[wave][2 + e][dl] = acc[e];
  }
  __syncthreads();
  if (wave != 0 || kg != 0) return;
  for (int w = 1; w < NW; ++w) {
    float a2[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) a2[e] = red[w][2 + e][dl];
    merge_b<VEC>(m, l, acc, red[w][0][dl], red[w][1][dl], a2);
  }
  const int64_t sh = ((int64_t)split * bt.B * P + s) * H + h;
  if (dl == 0) part_ml[sh] = make_float2(m, l);
#pragma unroll
  for (int e = 0; e < VEC; e += 4)
    *reinterpret_cast<float4*>(part_o + sh * D + dl * VEC + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
}

}  // namespace

int choose_batched_splits(int64_t seq_len, int P, int H, int num_cus) {
  const int64_t pairs = (int64_t)P * H;
  int64_t want = ((int64_t)num_cus * 8 + pairs - 1) / pairs;
  const int64_t max_by_len = (seq_len + 1023) / 1024;
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  if (want > 64) want = 64;
  return (int)want;
}

hipError_t launch_batched_doc(int n_splits, const void* q, const void* k, const void* v, int64_t seq_len, int P,
                              int H, int d, pp_dtype_t dtype, float c, const Workspace& ws, hipStream_t stream,
                              const Batch& bt) {
  const dim3 grid(H, n_splits, P * bt.B);  // dispatch order: heads, then splits, stream outermost
#define PP_B_LAUNCH(TT, DD)                                                                                   \
  launch_kernel(batched_doc_kernel<TT, DD>, grid, dim3(kBThreads), stream, static_cast<const TT*>(q),           \
                static_cast<const TT*>(k), static_cast<const TT*>(v), P, H, c, ws.plan, seq_len, n_splits,      \
                ws.part_o, ws.part_ml, bt)
  if (dtype == PP_BF16) return d == 128 ? PP_B_LAUNCH(uint16_t, 128) : PP_B_LAUNCH(uint16_t, 64);
  return d == 128 ? PP_B_LAUNCH(float, 128) : PP_B_LAUNCH(float, 64);
#undef PP_B_LAUNCH
}

}  // namespace pp
