// The append part of one layer of a decode step.
//
// A decode step appends one token per stream (Parallel Prompting project
// page, "How it works": each step appends one token per stream and keeps a
// fixed shape).  Positions are shared (same page, item 2): every stream's
// positions start right after the document, as if its question were the
// only one, so the new token of stream s sits at the number of slots it sees
// before itself -- the document prefix plus its earlier visible slots past
// it -- which the step's plan already holds: pos_s = doc_len + counts[s] - 1
// (the new slot is the last one stream s sees).
//
// One workgroup per stream: the rotary embedding (rotate-half pairs
// (i, i + d/2), angle pos * base^(-2i/d)) of the new query and key, the
// rotated key and the value written to the stream's new cache slot, the
// rotated query to the workspace for the attention kernels that follow.
// The angles are formed in double precision (a position of 10^5 times a
// frequency near 1 leaves fp32 with ~10^-2 rad of error); the rotation
// itself is fp32 and rounds once to the element type.
#include <math.h>

#include "pp_internal.h"

namespace pp {
namespace {

constexpr int kAppendThreads = 256;

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* f);
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float* f) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  f[0] = bf16_bits_to_f32(w.x & 0xffffu);
  f[1] = bf16_bits_to_f32(w.x >> 16);
  f[2] = bf16_bits_to_f32(w.y & 0xffffu);
  f[3] = bf16_bits_to_f32(w.y >> 16);
}
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* f) {
  const float4 w = *reinterpret_cast<const float4*>(p);
  f[0] = w.x;
  f[1] = w.y;
  f[2] = w.z;
  f[3] = w.w;
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float* f);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const float* f) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}

// plan = {doc_len, seq_len} of the step (from the appending plan kernel);
// the step's new slots are [seq_len - P, seq_len).  An empty or out-of-range
// plan writes nothing.  Hq query heads, Hkv key/value heads (Hq = Hkv
// without grouping): the queries have Hq rows per stream, the new keys and
// values Hkv.
template <typename T, int D>
__global__ __launch_bounds__(kAppendThreads) void append_rope_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new, T* __restrict__ k_cache,
    T* __restrict__ v_cache, int Hq, int Hkv, double rope_base, const int32_t* __restrict__ plan,
    const int32_t* __restrict__ counts, int64_t max_len, T* __restrict__ q_rot) {
  constexpr int HALF = D / 2;
  constexpr int C4 = HALF / 4;  // chunks of 4 pairs per head
  __shared__ float cs[HALF], sn[HALF];
  const int s = blockIdx.x, P = gridDim.x, tid = threadIdx.x;
  const int64_t seq_len = __builtin_amdgcn_readfirstlane(plan[1]);
  if (seq_len < P || seq_len > max_len) return;
  const int64_t slot = seq_len - P + s;
  const bool rot = rope_base > 0.0;
  if (rot) {
    if (tid < HALF) {
      const int64_t pos = (int64_t)plan[0] + counts[s] - 1;
      const double theta = exp2(-(2.0 * tid / D) * log2(rope_base));
      double sv, cv;
      sincos((double)pos * theta, &sv, &cv);
      cs[tid] = (float)cv;
      sn[tid] = (float)sv;
    }
    __syncthreads();
  }
  // rows [0, nh) of D elements from src, each pair (i, i + D/2) rotated, to dst
  auto rotate = [&](const T* src, T* dst, int nh) {
    for (int it = tid; it < nh * C4; it += kAppendThreads) {
      const int h = it / C4, i0 = (it % C4) * 4;
      const int64_t lo = (int64_t)h * D + i0, hi = lo + HALF;
      float a[4], b4[4];
      load4<T>(src + lo, a);
      load4<T>(src + hi, b4);
      if (rot) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = cs[i0 + e], sv = sn[i0 + e];
          const float x = a[e], y = b4[e];
          a[e] = fmaf(x, c, -y * sv);
          b4[e] = fmaf(y, c, x * sv);
        }
      }
      store4<T>(dst + lo, a);
      store4<T>(dst + hi, b4);
    }
  };
  const int64_t qoff = (int64_t)s * Hq * D, knoff = (int64_t)s * Hkv * D, koff = slot * Hkv * D;
  rotate(q + qoff, q_rot + qoff, Hq);
  rotate(k_new + knoff, k_cache + koff, Hkv);
  constexpr int VE = 16 / (int)sizeof(T);  // elements per 16-byte vector
  for (int it = tid; it < Hkv * D / VE; it += kAppendThreads)
    *reinterpret_cast<u32x4*>(v_cache + koff + (int64_t)it * VE) =
        *reinterpret_cast<const u32x4*>(v_new + knoff + (int64_t)it * VE);
}

}  // namespace

hipError_t launch_append_rope(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              int P, int Hq, int Hkv, int d, pp_dtype_t dtype, double rope_base, const int32_t* plan,
                              const int32_t* counts, int64_t max_len, void* q_rot, hipStream_t stream) {
#define PP_APPEND_LAUNCH(TT, DD)                                                                              \
  append_rope_kernel<TT, DD><<<P, kAppendThreads, 0, stream>>>(                                               \
      static_cast<const TT*>(q), static_cast<const TT*>(k_new), static_cast<const TT*>(v_new),                \
      static_cast<TT*>(k_cache), static_cast<TT*>(v_cache), Hq, Hkv, rope_base, plan, counts, max_len,       \
      static_cast<TT*>(q_rot))
  if (dtype == PP_BF16) {
    if (d == 128) PP_APPEND_LAUNCH(uint16_t, 128);
    else PP_APPEND_LAUNCH(uint16_t, 64);
  } else {
    if (d == 128) PP_APPEND_LAUNCH(float, 128);
    else PP_APPEND_LAUNCH(float, 64);
  }
#undef PP_APPEND_LAUNCH
  return hipGetLastError();
}

}  // namespace pp
