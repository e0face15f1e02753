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
// frequency near 1 leaves fp32 with ~10^-2 rad of error) and reduced modulo
// 2*pi there; the sine and cosine of the reduced angle (|r| <= pi, rounded
// to fp32: about 2^-22 rad off) are fp32, as is the rotation, which rounds
// once to the element type.  A double sincos of the unreduced angle takes
// the slow large-argument path on every new token past the first few
// thousand positions.
#include <math.h>

#include "pp_internal.h"

namespace pp {
namespace {

constexpr int kAppendThreads = 256;

// 16 bytes of elements <-> floats (8 bf16 or 4 fp32)
template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& w, float* f);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}
template <typename T>
__device__ __forceinline__ u32x4 pack16(const float* f);
template <>
__device__ __forceinline__ u32x4 pack16<uint16_t>(const float* f) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}
template <>
__device__ __forceinline__ u32x4 pack16<float>(const float* f) {
  return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
}

// Workgroup (s, b): stream s of request b.  plan = {doc_len[B], seq_len[B]}
// of the step (from the appending plan kernel); request b's new slots are
// [seq_len[b] - P, seq_len[b]).  An empty or out-of-range plan writes
// nothing (an idle request).  Hq query heads, Hkv key/value heads (Hq = Hkv
// without grouping): the queries have Hq rows per stream, the new keys and
// values Hkv; request b's caches start kv_stride elements after request
// b - 1's.  A retired stream (active[s] == 0) lists nothing, so it has no
// position: its query is rotated (the attention discards it) but its key and
// value are not written.
//
// A rotation item is VE consecutive pairs (i, i + d/2) of one row: two
// 16-byte vectors.  Each thread loads its first kPre items and value
// vectors before anything else, so that one memory round trip (overlapping
// the angles) precedes the rotation; rows past that (many heads) are
// loaded in the loop.
template <typename T, int D>
__global__ __launch_bounds__(kAppendThreads) void append_rope_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new, T* __restrict__ k_cache,
    T* __restrict__ v_cache, int Hq, int Hkv, double rope_base, const int32_t* __restrict__ plan,
    const int32_t* __restrict__ counts, int64_t max_len, T* __restrict__ q_rot, int64_t kv_stride,
    const int32_t* __restrict__ active) {
  constexpr int HALF = D / 2;
  constexpr int VE = 16 / (int)sizeof(T);  // elements per 16-byte vector
  constexpr int CV = HALF / VE;            // rotation items per row
  constexpr int kPre = 4;                  // items (and value vectors) per thread loaded up front
  __shared__ float cs[HALF], sn[HALF];
  const int s = blockIdx.x, P = gridDim.x, b = blockIdx.y, B = gridDim.y, tid = threadIdx.x;
  const int sl = b * P + s;  // stream of the launch
  k_cache += b * kv_stride;
  v_cache += b * kv_stride;
  // rotation items: the Hq query rows of the stream, then its Hkv key rows
  const bool live = !active || active[sl] != 0;
  const int nq = Hq * CV, nr = live ? (Hq + Hkv) * CV : nq, nv = live ? Hkv * D / VE : 0;
  const int64_t qoff = (int64_t)sl * Hq * D, knoff = (int64_t)sl * Hkv * D;
  auto row_off = [&](int it) -> int64_t {  // offset of item it within its rows
    const int r = it < nq ? it : it - nq;
    return (int64_t)(r / CV) * D + (r % CV) * VE;
  };
  auto src = [&](int it) -> const T* { return (it < nq ? q + qoff : k_new + knoff) + row_off(it); };
  // Only the destination slot and the angle depend on the plan: every input
  // this thread needs first is loaded before it.
  u32x4 av[kPre], bv[kPre], vv[kPre];
#pragma unroll
  for (int p = 0; p < kPre; ++p) {
    const int it = tid + p * kAppendThreads, iv = it;
    if (it < nr) {
      av[p] = *reinterpret_cast<const u32x4*>(src(it));
      bv[p] = *reinterpret_cast<const u32x4*>(src(it) + HALF);
    }
    if (iv < nv) vv[p] = *reinterpret_cast<const u32x4*>(v_new + knoff + (int64_t)iv * VE);
  }
  const int32_t doc_len = plan[b], count = counts[sl];
  const int64_t seq_len = __builtin_amdgcn_readfirstlane(plan[B + b]);
  if (seq_len < P || seq_len > max_len) return;  // (uniform over the workgroup)
  const int64_t slot = seq_len - P + s, koff = slot * Hkv * D;
  const bool rot = rope_base > 0.0;
  if (rot) {
    if (tid < HALF) {
      const int64_t pos = (int64_t)doc_len + count - 1;
      const double theta = exp2(-(2.0 * tid / D) * log2(rope_base));
      const double x = (double)pos * theta;
      constexpr double kTwoPi = 6.283185307179586476925286766559;
      const float r = (float)fma(-rint(x * (1.0 / kTwoPi)), kTwoPi, x);
      float sv, cv;
      sincosf(r, &sv, &cv);
      cs[tid] = cv;
      sn[tid] = sv;
    }
    __syncthreads();
  }
  auto rotate_store = [&](int it, const u32x4& aw, const u32x4& bw) {
    float a[VE], b4[VE];
    unpack16<T>(aw, a);
    unpack16<T>(bw, b4);
    if (rot) {
      const int i0 = (it % CV) * VE;
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float c = cs[i0 + e], sv = sn[i0 + e];
        const float x = a[e], y = b4[e];
        a[e] = fmaf(x, c, -y * sv);
        b4[e] = fmaf(y, c, x * sv);
      }
    }
    T* dst = (it < nq ? q_rot + qoff : k_cache + koff) + row_off(it);
    *reinterpret_cast<u32x4*>(dst) = pack16<T>(a);
    *reinterpret_cast<u32x4*>(dst + HALF) = pack16<T>(b4);
  };
#pragma unroll
  for (int p = 0; p < kPre; ++p) {
    const int it = tid + p * kAppendThreads;
    if (it < nr) rotate_store(it, av[p], bv[p]);
  }
  for (int it = tid + kPre * kAppendThreads; it < nr; it += kAppendThreads)
    rotate_store(it, *reinterpret_cast<const u32x4*>(src(it)), *reinterpret_cast<const u32x4*>(src(it) + HALF));
#pragma unroll
  for (int p = 0; p < kPre; ++p) {
    const int iv = tid + p * kAppendThreads;
    if (iv < nv) *reinterpret_cast<u32x4*>(v_cache + koff + (int64_t)iv * VE) = vv[p];
  }
  for (int iv = tid + kPre * kAppendThreads; iv < nv; iv += kAppendThreads)
    *reinterpret_cast<u32x4*>(v_cache + koff + (int64_t)iv * VE) =
        *reinterpret_cast<const u32x4*>(v_new + knoff + (int64_t)iv * VE);
}

}  // namespace

hipError_t launch_append_rope(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              int P, int Hq, int Hkv, int d, pp_dtype_t dtype, double rope_base, const int32_t* plan,
                              const int32_t* counts, int64_t max_len, void* q_rot, hipStream_t stream, int B,
                              int64_t kv_stride, const int32_t* active) {
#define PP_APPEND_LAUNCH(TT, DD)                                                                              \
  append_rope_kernel<TT, DD><<<dim3(P, B), kAppendThreads, 0, stream>>>(                                      \
      static_cast<const TT*>(q), static_cast<const TT*>(k_new), static_cast<const TT*>(v_new),                \
      static_cast<TT*>(k_cache), static_cast<TT*>(v_cache), Hq, Hkv, rope_base, plan, counts, max_len,       \
      static_cast<TT*>(q_rot), kv_stride, active)
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
