// Document part of one decode step: the document's K/V are read once for
// all P streams of a head.
//
// Parallel Prompting's point (project page, illustration "Inside decode
// step" and "How it works"): P per-question requests do P vector x matrix
// products against the document keys, reading them P times; packing the P
// streams into one request turns that into one matrix x matrix product that
// reads the document once per step.  On gfx950 that product runs on the
// matrix cores: for a head h and a tile of NK document slots,
//     S^T[key][query] = K_tile[key][:] . Q[query][:]        (MFMA bf16)
//     O^T[dim][query] += V_tile^T[dim][key] . P^T[key][query] (MFMA bf16)
// with an online softmax between them (flash-decoding), split over the
// document ("split-K") so that H x splits workgroups fill the chip.  Each
// split leaves a partial softmax state (m, l, O) per (stream, head); the
// tail kernel merges them in a fixed order.
//
// Every document slot is visible to every stream, so no mask is evaluated
// here beyond the split's slot range; slots outside it are zero-filled in
// LDS, never loaded.
#include <math.h>

#include "pp_internal.h"

namespace pp {
namespace {

constexpr int kDocThreads = 256;  // 4 waves; wave w owns queries [w*16*QB, (w+1)*16*QB)

// Document slots per tile: 64, or 32 for the widest query tile at d = 128,
// whose accumulators (64 queries x 128 dims per wave) leave room for no more.
template <int D, int QB>
constexpr int doc_tile_keys() { return (D == 128 && QB == 4) ? 32 : 64; }

// ---- LDS layouts -----------------------------------------------------------
// K tile: [NK keys][D dims] bf16, 16-byte chunks XOR-swizzled per row so
// that the 16 rows read by one MFMA A-operand load fall in distinct banks.
// V tile: stored transposed, [D dims][NK keys] bf16 (rows of 2*NK bytes), so a
// lane can read the 8 consecutive keys of one dim that the P.V MFMA needs
// as its A operand; 16-byte granules XOR-swizzled per row.

// 4-bit row pattern f(r) with: f bijective on even r, on odd r, on r<8 and
// on r>=8 (r = 0..15).  Used for 128-byte rows where two rows share one
// 256-byte bank line.
__device__ __forceinline__ int swz_rows128(int r) { return ((r >> 1) & 3) | (((r & 1) ^ ((r >> 3) & 1)) << 2); }

// K-row swizzle.  The 16 keys of one QK MFMA A operand are
// {32c + 8(r>>2) + 4b + (r&3)} (r = 0..15), i.e. they differ in key bits
// 0,1,3,4; the swizzle maps those bits to distinct granules.
template <int D>
__device__ __forceinline__ int swz_k(int key) {
  const int r = (key & 3) | (((key >> 3) & 3) << 2);
  if constexpr (D == 128) {
    return r;  // 16 chunks per 256-byte row
  } else {
    return swz_rows128(r);  // 8 chunks per 128-byte row
  }
}

// V^T-row swizzle (16-byte granule index within a row of NK keys).
template <int NK>
__device__ __forceinline__ int swz_vt(int row) {
  if constexpr (NK == 64) {
    return swz_rows128(row & 15);  // 8 granules per 128-byte row
  } else {
    return ((row >> 2) & 3) ^ (row & 2);  // 4 granules per 64-byte row
  }
}

// Physical key (within a tile) of row r of 16-key MFMA block kb.  Chosen so
// that the QK accumulator rows a lane holds for key blocks 2c and 2c+1 are
// exactly the 8 consecutive keys 32c + 8g .. 32c + 8g + 7 that the same lane
// supplies as the P.V MFMA operand (g = lane / 16).
__device__ __forceinline__ int key_of(int kb, int r) { return 32 * (kb >> 1) + 8 * (r >> 2) + 4 * (kb & 1) + (r & 3); }

template <int D, int QB>
__global__ __launch_bounds__(kDocThreads) void doc_mfma_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int P,
    int H, float c, const int32_t* __restrict__ doc_len_ptr, int n_splits, float* __restrict__ part_o,
    float2* __restrict__ part_ml) {
  constexpr int kNK = doc_tile_keys<D, QB>();
  constexpr int KC = D / 32;            // QK contraction steps (32 dims each)
  constexpr int DB = D / 16;            // 16-dim output blocks
  constexpr int KB = kNK / 16;          // 16-key blocks per tile
  constexpr int CH = kNK / 32;          // P.V contraction steps (32 keys each)
  constexpr int ROWB = D * 2;           // bytes per K row in LDS
  constexpr int VTB = kNK * 2;          // bytes per V^T row in LDS
  constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
  constexpr int NLD = kNK * CPR / kDocThreads;  // 16-byte loads per thread per tile (K and V each)
  constexpr int KPT = NLD;              // V keys per thread (same dim chunk)
  static_assert(NLD == 2 || NLD == 4, "tile shape");

  __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][kNK * ROWB];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v[2][D * VTB];

  const int split = blockIdx.x, h = blockIdx.y, pt = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int L = *doc_len_ptr;
  const int n_tiles = (L + kNK - 1) / kNK;
  const int t0 = (int)((int64_t)split * n_tiles / n_splits);
  const int t1 = (int)((int64_t)(split + 1) * n_tiles / n_splits);
  const int key_end = min(t1 * kNK, L);
  const int q0 = pt * (64 * QB) + wave * (16 * QB);
  const int64_t row = (int64_t)H * D;  // elements between consecutive slots

  // Q fragments (B operand of S^T = K Q^T): lane (query ln, group lg) holds
  // dims kc*32 + 8*lg .. +8 of its query.  Padding queries are zero.
  bf16x8 qf[QB][KC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int p = q0 + qb * 16 + ln;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (p < P) {
        qf[qb][kc] = *reinterpret_cast<const bf16x8*>(q + ((int64_t)p * H + h) * D + kc * 32 + lg * 8);
      } else {
        qf[qb][kc] = bf16x8{};
      }
    }
  }

  f32x4 o[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (t0 < t1) {
    u32x4 kreg[NLD], vreg[NLD];

    // global -> registers for tile t (coalesced 16-byte loads; rows past
    // key_end are zero and never read from memory)
    auto gload = [&](int t) {
      const int kbase = t * kNK;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int cidx = tid + i * kDocThreads;
        const int key = cidx / CPR, col = cidx % CPR;
        const int gk = kbase + key;
        kreg[i] = gk < key_end ? *reinterpret_cast<const u32x4*>(k + (int64_t)gk * row + (int64_t)h * D + col * 8)
                               : u32x4{0u, 0u, 0u, 0u};
      }
      const int dc = tid % CPR, kq = tid / CPR;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int gk = kbase + kq * KPT + i;
        vreg[i] = gk < key_end ? *reinterpret_cast<const u32x4*>(v + (int64_t)gk * row + (int64_t)h * D + dc * 8)
                               : u32x4{0u, 0u, 0u, 0u};
      }
    };

    // registers -> LDS buffer b (K swizzled, V transposed + swizzled)
    auto lstore = [&](int b) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int cidx = tid + i * kDocThreads;
        const int key = cidx / CPR, col = cidx % CPR;
        *reinterpret_cast<u32x4*>(&lds_k[b][key * ROWB + ((col ^ swz_k<D>(key)) * 16)]) = kreg[i];
      }
      const int dc = tid % CPR, kq = tid / CPR;
      // vreg[i] holds dims dc*8 .. +8 of key kq*KPT + i; dword w = dims 2w (lo), 2w+1 (hi)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int dim = dc * 8 + 2 * w + half;
          uint32_t pk[KPT / 2];
#pragma unroll
          for (int j = 0; j < KPT / 2; ++j) {
            const uint32_t a = vreg[2 * j][w], bb = vreg[2 * j + 1][w];
            pk[j] = half == 0 ? ((a & 0xffffu) | (bb << 16)) : ((a >> 16) | (bb & 0xffff0000u));
          }
          const int key0 = kq * KPT;              // first key written
          const int gi = key0 / 8;                // 16-byte granule within the row
          const int off = (key0 % 8) * 2;         // byte offset within the granule
          unsigned char* dst = &lds_v[b][dim * VTB + ((gi ^ swz_vt<kNK>(dim)) * 16) + off];
          if constexpr (KPT == 4) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pk[0], pk[1]);
          } else {
            *reinterpret_cast<uint32_t*>(dst) = pk[0];
          }
        }
      }
    };

    gload(t0);
    lstore(0);
    __syncthreads();

    for (int t = t0; t < t1; ++t) {
      const int b = (t - t0) & 1;
      if (t + 1 < t1) gload(t + 1);
      const int kbase = t * kNK;

      // ---- S^T = K Q^T -----------------------------------------------------
      f32x4 s[QB][KB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int key = key_of(kb, ln);
          const int col = kc * 4 + lg;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&lds_k[b][key * ROWB + ((col ^ swz_k<D>(key)) * 16)]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[qb][kc], s[qb][kb], 0, 0, 0);
        }
      }

      // ---- online softmax (log2 domain); lane holds keys of its group lg ----
      uint32_t pb[QB][CH][4];  // P^T as packed bf16 pairs: the P.V B operand
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 32 * (kb >> 1) + 8 * lg + 4 * (kb & 1) + i;
            const float x = (kbase + key < key_end) ? s[qb][kb][i] * c : -INFINITY;
            s[qb][kb][i] = x;
            tmax = fmaxf(tmax, x);
          }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mn = fmaxf(m[qb], tmax);  // finite: every tile has a valid key
        const float alpha = fast_exp2(m[qb] - mn);
        m[qb] = mn;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(s[qb][kb][i] - mn);
            s[qb][kb][i] = p;
            psum += p;
          }
        l[qb] = l[qb] * alpha + psum;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
          pb[qb][ch][0] = pack_bf16x2(s[qb][2 * ch][0], s[qb][2 * ch][1]);
          pb[qb][ch][1] = pack_bf16x2(s[qb][2 * ch][2], s[qb][2 * ch][3]);
          pb[qb][ch][2] = pack_bf16x2(s[qb][2 * ch + 1][0], s[qb][2 * ch + 1][1]);
          pb[qb][ch][3] = pack_bf16x2(s[qb][2 * ch + 1][2], s[qb][2 * ch + 1][3]);
        }
      }

      // ---- O^T += V^T P^T ----------------------------------------------------
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int dim = db * 16 + ln;
          const int gi = ch * 4 + lg;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&lds_v[b][dim * VTB + ((gi ^ swz_vt<kNK>(dim)) * 16)]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const u32x4 bw = u32x4{pb[qb][ch][0], pb[qb][ch][1], pb[qb][ch][2], pb[qb][ch][3]};
            o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bw), o[qb][db], 0, 0, 0);
          }
        }
      }

      if (t + 1 < t1) lstore(b ^ 1);
      __syncthreads();
    }
  }

  // ---- partial state of this split -------------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float lt = l[qb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int p = q0 + qb * 16 + ln;
    if (p < P) {
      const int64_t sh = ((int64_t)split * P + p) * H + h;
      if (lg == 0) part_ml[sh] = make_float2(m[qb], lt);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(part_o + sh * D + db * 16 + 4 * lg) = o[qb][db];
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs: the same split-K structure on the vector ALUs.  The K/V tile
// is staged in LDS once per workgroup and every thread (one query each)
// reads it by broadcast: the document is still read once for all streams.
constexpr int kF32NK = 32;

template <int D>
__global__ __launch_bounds__(kDocThreads) void doc_valu_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v, int P, int H, float c,
    const int32_t* __restrict__ doc_len_ptr, int n_splits, float* __restrict__ part_o, float2* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) float lk[kF32NK][D];
  __shared__ __attribute__((aligned(16))) float lv[kF32NK][D];
  const int split = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int p = blockIdx.z * kDocThreads + tid;
  const int L = *doc_len_ptr;
  const int n_tiles = (L + kF32NK - 1) / kF32NK;
  const int t0 = (int)((int64_t)split * n_tiles / n_splits);
  const int t1 = (int)((int64_t)(split + 1) * n_tiles / n_splits);
  const int key_end = min(t1 * kF32NK, L);
  const int64_t row = (int64_t)H * D;

  float qv[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = p < P ? q[((int64_t)p * H + h) * D + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int t = t0; t < t1; ++t) {
    const int kbase = t * kF32NK;
    for (int i = tid; i < kF32NK * D / 4; i += kDocThreads) {
      const int key = i / (D / 4), col = i % (D / 4);
      const int gk = kbase + key;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (gk < key_end) {
        kk = *reinterpret_cast<const float4*>(k + (int64_t)gk * row + (int64_t)h * D + col * 4);
        vv = *reinterpret_cast<const float4*>(v + (int64_t)gk * row + (int64_t)h * D + col * 4);
      }
      *reinterpret_cast<float4*>(&lk[key][col * 4]) = kk;
      *reinterpret_cast<float4*>(&lv[key][col * 4]) = vv;
    }
    __syncthreads();
    float x[kF32NK];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32NK; ++j) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) d = fmaf(qv[e], lk[j][e], d);
      x[j] = (kbase + j < key_end) ? d * c : -INFINITY;
      tmax = fmaxf(tmax, x[j]);
    }
    const float mn = fmaxf(m, tmax);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32NK; ++j) {
      const float pj = fast_exp2(x[j] - mn);
      l += pj;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(pj, lv[j][e], acc[e]);
    }
    __syncthreads();
  }
  if (p < P) {
    const int64_t sh = ((int64_t)split * P + p) * H + h;
    part_ml[sh] = make_float2(m, l);
#pragma unroll
    for (int e = 0; e < D; e += 4)
      *reinterpret_cast<float4*>(part_o + sh * D + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
}

}  // namespace

DocPlan choose_doc_plan(int64_t seq_len, int P, int H, int d, pp_dtype_t dtype, int num_cus) {
  DocPlan pl;
  int per_cu;  // workgroups resident per CU the launch is sized for
  if (dtype == PP_BF16) {
    pl.qb = P <= 64 ? 1 : (P <= 128 ? 2 : 4);
    pl.n_ptiles = (P + 64 * pl.qb - 1) / (64 * pl.qb);
    per_cu = pl.qb == 4 ? 1 : 2;
  } else {
    pl.qb = 0;
    pl.n_ptiles = (P + kDocThreads - 1) / kDocThreads;
    per_cu = 2;
  }
  const int64_t base = (int64_t)H * pl.n_ptiles;
  int64_t want = ((int64_t)num_cus * per_cu + base - 1) / base;
  const int64_t max_by_len = (seq_len + 255) / 256;  // at least ~256 slots of the upper bound per split
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  if (want > 256) want = 256;
  pl.n_splits = (int)want;
  return pl;
}

hipError_t launch_doc(const DocPlan& pl, const void* q, const void* k, const void* v, int P, int H, int d,
                      pp_dtype_t dtype, float c, const Workspace& ws, hipStream_t stream) {
  const dim3 grid(pl.n_splits, H, pl.n_ptiles);
  if (dtype == PP_BF16) {
    auto* qq = static_cast<const uint16_t*>(q);
    auto* kk = static_cast<const uint16_t*>(k);
    auto* vv = static_cast<const uint16_t*>(v);
#define PP_DOC_LAUNCH(DD, QQ) \
  doc_mfma_bf16_kernel<DD, QQ><<<grid, kDocThreads, 0, stream>>>(qq, kk, vv, P, H, c, ws.doc_len, pl.n_splits, ws.part_o, ws.part_ml)
    if (d == 128) {
      if (pl.qb == 1) PP_DOC_LAUNCH(128, 1);
      else if (pl.qb == 2) PP_DOC_LAUNCH(128, 2);
      else PP_DOC_LAUNCH(128, 4);
    } else {
      if (pl.qb == 1) PP_DOC_LAUNCH(64, 1);
      else if (pl.qb == 2) PP_DOC_LAUNCH(64, 2);
      else PP_DOC_LAUNCH(64, 4);
    }
#undef PP_DOC_LAUNCH
  } else {
    auto* qq = static_cast<const float*>(q);
    auto* kk = static_cast<const float*>(k);
    auto* vv = static_cast<const float*>(v);
    if (d == 128)
      doc_valu_f32_kernel<128><<<grid, kDocThreads, 0, stream>>>(qq, kk, vv, P, H, c, ws.doc_len, pl.n_splits, ws.part_o, ws.part_ml);
    else
      doc_valu_f32_kernel<64><<<grid, kDocThreads, 0, stream>>>(qq, kk, vv, P, H, c, ws.doc_len, pl.n_splits, ws.part_o, ws.part_ml);
  }
  return hipGetLastError();
}

}  // namespace pp
