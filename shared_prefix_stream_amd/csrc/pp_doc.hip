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
// here beyond the split's slot range: rows of a ragged last tile re-read the
// split's last row (finite data) and their scores are set to -inf.  Two
// further modes share the kernel: grouped key/value heads (the G query heads
// of a key/value head form one query tile, and several requests one grid)
// and a causal mode for the prefill (query tile pt against the document
// slots up to its own tile, masked above the diagonal).
#include <math.h>

#include <type_traits>

#include "pp_internal.h"

namespace pp {
namespace {

constexpr int kDocThreads = 256;  // workgroup of the fp32 vector-ALU kernel

// One direct global->LDS load of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): lane l's chunk lands at LDS byte lds_base + 16*l.
// Issued from asm so that the compiler, which cannot tell these LDS writes
// from the transposing LDS reads below, does not drain every outstanding load
// before each such read; the kernel waits on its own loads with explicit
// vmcnt waits instead.  The asm has no outputs, and it sets M0, which the
// compiler reserves and does not rely on in this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The LDS base (and below the global base) is wave-uniform; readfirstlane
// states it, since a call inside a branch on the wave's group may not be
// known uniform to the compiler.
// NT: the rows are read by this workgroup only, once per step, so they go
// through the caches with the non-temporal hint and do not evict what the
// step reads again (the split partials, the queries, the slot lists, the
// own-slot rows) or force write-backs of dirty lines.
template <bool NT>
__device__ __forceinline__ void lds_dma16(const void* gaddr, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(
                     __builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(gaddr)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(gaddr)
                 : "memory", "m0");
}
// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (no 64-bit address arithmetic on the vector ALUs).
template <bool NT>
__device__ __forceinline__ void lds_dma16_sv(const void* base, uint32_t voff, uint32_t lds_base) {
  const uint64_t b = (uint64_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const void* sbase = (const void*)(((uint64_t)hi << 32) | (uint64_t)lo);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(
                     __builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(voff), "s"(sbase)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int D, int QB, int NW>
struct DocTile {
  // Document slots per tile: 64, or more when needed for every wave to issue
  // at least one 1 KB direct load per tile (128 at d = 64 with 16 waves).
  static constexpr int NK = (1024 * NW) / (D * 2) > 64 ? (1024 * NW) / (D * 2) : 64;
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROWB = D * 2;                 // bytes of one K or V row (one head)
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int TILE_BYTES = NK * ROWB;       // K (or V) tile
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int NS = 4;                       // LDS ring stages (see the pipeline below)
  static constexpr int ROWS_PER_KB = 1024 / ROWB;    // rows one wave-wide 16-byte load fills
  static constexpr int NLD = TILE_BYTES / 1024 / NW;  // direct loads per thread per tile (K or V)
  static_assert(NLD >= 1 && TILE_BYTES % (1024 * NW) == 0, "tile shape");
};

// ---- LDS layouts -----------------------------------------------------------
// Tiles are filled by direct global->LDS loads: a wave-wide 16-byte load
// writes 1 KB of LDS contiguously (lane l at +16*l), and each lane may fetch
// any 16-byte chunk of the tile, so the layouts below are permutations of
// 16-byte chunks within each row (XOR swizzles that keep MFMA operand reads
// free of bank conflicts).
//
// K tile [NK][D]: the QK A operand of key block kb is read by lane (r, g) as
// 16 bytes of row key_of(kb, r); those 16 rows differ in key bits 0,1,3,4.

// 4-bit row pattern f(r) with: f bijective on even r, on odd r, on r<8 and
// on r>=8 (r = 0..15), for 128-byte rows where two rows share a bank line.
__device__ __forceinline__ int swz_rows128(int r) { return ((r >> 1) & 3) | (((r & 1) ^ ((r >> 3) & 1)) << 2); }

template <int D>
__device__ __forceinline__ int swz_k(int key) {
  const int r = (key & 3) | (((key >> 3) & 3) << 2);
  if constexpr (D == 128) {
    return r;  // 16 chunks per 256-byte row
  } else {
    return swz_rows128(r);  // 8 chunks per 128-byte row
  }
}

// V tile [NK][D], natural row order.  The P.V A operand (8 consecutive keys
// of one dim per lane) is read with the gfx950 transposing LDS load
// ds_read_b64_tr_b16: in each 16-lane group, lane 4r+j points at 4
// consecutive dims of row r, and lane m receives dim m of the 4 rows.  One
// such load touches rows 8g + r (g = lane/16, r = 0..3) in 32-byte pieces;
// the swizzle (even, so chunk pairs stay together) spreads them over banks.
template <int D>
__device__ __forceinline__ int swz_v(int key) {
  if constexpr (D == 128) {
    return 2 * ((key & 3) | (((key >> 3) & 1) << 2));
  } else {
    return 2 * (((key >> 1) & 1) | (((key >> 3) & 1) << 1));
  }
}

// Physical key (within a tile) of row r of 16-key MFMA block kb.  Chosen so
// that the QK accumulator rows a lane holds for key blocks 2c and 2c+1 are
// exactly the 8 consecutive keys 32c + 8g .. 32c + 8g + 7 that the same lane
// supplies as the P.V MFMA operand (g = lane / 16).
__device__ __forceinline__ int key_of(int kb, int r) { return 32 * (kb >> 1) + 8 * (r >> 2) + 4 * (kb & 1) + (r & 3); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup = NW waves; wave w owns queries [w*16*QB, (w+1)*16*QB) of the
// workgroup's query tile (16*QB*NW queries).  With 8 waves of 32 queries
// two waves share each SIMD, so one wave's softmax overlaps the other's
// matrix products.
//
// Queries of a workgroup: the P streams' queries of the G query heads that
// read key/value head h, query p = s * G + g for stream s and group member g
// (grouped key/value heads: one K/V tile serves G * P queries).  Several
// requests: grid.z = B * (query tiles per request), request-major; each
// request has its own document length (plan[b]), caches and queries.
//
// CAUSAL (prefill): query i is slot i of the sequence, and query tile pt
// attends to the document slots j < min((pt + 1) * tile, doc_len) with
// j <= i -- the part of every query's visible set that lies in the shared
// document prefix up to its own tile.  One split per tile; tiles are taken
// longest first.  A document slot's whole visible set lies in its tile's
// range, so with `out` given its output is final here and written directly
// (the per-slot kernel that follows skips those slots).
//
// NT (non-causal, one query tile per key/value head): no other workgroup
// reads this workgroup's key/value tiles, so they are loaded non-temporal.
template <int D, int QB, int NW, bool CAUSAL, bool NT = false>
__global__ __launch_bounds__(64 * NW) void doc_mfma_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int P,
    int H, float c, const int32_t* __restrict__ plan, int64_t seq_len, int n_splits,
    float* __restrict__ part_o, float2* __restrict__ part_ml, Batch bt, uint16_t* __restrict__ out) {
  using TL = DocTile<D, QB, NW>;
  constexpr int NK = TL::NK, NS = TL::NS, NLD = TL::NLD, ROWB = TL::ROWB, CPR = TL::CPR;
  constexpr int KC = D / 32;   // QK contraction steps (32 dims each)
  constexpr int DB = D / 16;   // 16-dim output blocks
  constexpr int KB = NK / 16;  // 16-key blocks per tile
  constexpr int CH = NK / 32;  // P.V contraction steps (32 keys each)

  __shared__ __attribute__((aligned(1024))) unsigned char ring[NS][TL::STAGE_BYTES];
  __shared__ int redo;

  const int split = blockIdx.x, h = blockIdx.y;
  const int nz = (int)gridDim.z / bt.B;  // query tiles per request
  const int b = (int)blockIdx.z / nz, zt = (int)blockIdx.z % nz;
  const int pt = CAUSAL ? nz - 1 - zt : zt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int q0 = pt * (16 * QB * NW) + wave * (16 * QB);
  // elements between consecutive slots (key/value heads), and this
  // workgroup's key/value head (grid.y runs over query heads when unfolded)
  const int64_t row = (int64_t)(H / bt.kv_group) * D;
  const int hk = h / bt.kv_group;
  const int G = bt.G, PQ = P * G, Hq = H * G;
  k += b * bt.kv_stride;
  v += b * bt.kv_stride;

  // Q fragments (B operand of S^T = K Q^T): lane (query ln, group lg) holds
  // dims kc*32 + 8*lg .. +8 of its query.  Padding queries are zero.  Their
  // loads are issued first, while the document length is still in flight.
  u32x4 qw[QB][KC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int p = q0 + qb * 16 + ln;
    const int pc = min(p, PQ - 1);  // in-bounds row for padding lanes (zeroed below)
    const int64_t qrow = (int64_t)(b * P + pc / G) * Hq + h * G + pc % G;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qw[qb][kc] = *reinterpret_cast<const u32x4*>(q + qrow * D + kc * 32 + lg * 8);
  }

  const int Ldoc = (int)min<int64_t>(load_doc_len(plan + b), seq_len);  // a plan never exceeds the slots given
  int L = Ldoc;
  if constexpr (CAUSAL) L = min(L, (pt + 1) * (16 * QB * NW));
  // floor(i * n_tiles / n_splits) as i * (n / k) + i * (n % k) / k: 32-bit
  // arithmetic only (i <= n_splits <= 256)
  const uint32_t n_tiles = ((uint32_t)L + NK - 1) / NK;
  const uint32_t tq = n_tiles / (uint32_t)n_splits, tr = n_tiles % (uint32_t)n_splits;
  const int t0 = (int)((uint32_t)split * tq + (uint32_t)split * tr / (uint32_t)n_splits);
  const int t1 = (int)((uint32_t)(split + 1) * tq + (uint32_t)(split + 1) * tr / (uint32_t)n_splits);
  const int key_end = min(t1 * NK, L);

  // Scores are taken as x = s * |c| with the sign of c folded into Q (a bf16
  // sign flip is exact), so the running maximum of x is that of s.
  // Two passes share the pipeline below.
  //  * Fast pass (always run): p = exp2(x) against the fixed reference 0 --
  //    no per-tile maximum and no rescaling.  The arithmetic is that of a
  //    running maximum of 0; it is accurate as long as the row sums stay
  //    within [2^-64, 2^64] (no overflow of p, no loss to underflow), which
  //    the pass checks at its end.
  //  * Exact pass (only if a row sum of the workgroup fell outside): running
  //    maximum with lazy rescaling, from the start of the split again.
  const uint32_t qsign = c < 0.f ? 0x80008000u : 0u;
  const float cabs = fabsf(c);

  bf16x8 qf[QB][KC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool pad = q0 + qb * 16 + ln >= PQ;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const u32x4 w = pad ? u32x4{0u, 0u, 0u, 0u} : (qw[qb][kc] ^ qsign);
      qf[qb][kc] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // O^T accumulators, and the softmax denominators: l is accumulated on the
  // matrix cores as an extra 16-row block whose A operand is all ones, so
  // every row (and lane) holds sum_k bf16(p_k) for its query -- the same
  // rounded weights the numerator uses.
  f32x4 o[QB][DB];
  f32x4 lsum[QB];
  float m[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    lsum[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  // Direct global->LDS loads of tile t into stage st.  Wave w's i-th load
  // fills 1 KB block (i*NW + w) of the K and of the V tile; rows past the
  // split's end re-read its last row (finite data, masked out of the scores).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ring_base = lds_addr(&ring[0][0]);
  // Per-lane byte offsets of its 16-byte pieces inside a tile (relative to
  // the tile's first row of head h), fixed for the whole split; the tile
  // base is a wave-uniform pointer.  Only the split's ragged last tile
  // clamps rows (to its last valid row, finite data masked out of the scores).
  // With two waves per SIMD the first wave of each pair issues the loads of
  // both (the second never waits on the vector-memory counter): the issue
  // stalls once per SIMD, in the first wave's slack before the barrier,
  // instead of on every wave right after it.
  constexpr int NIW = NW >= 8 ? 2 : 1;  // block sets a wave issues: its own (and its SIMD partner's)
  uint32_t koff[NIW][NLD], voff[NIW][NLD];
#pragma unroll
  for (int sset = 0; sset < NIW; ++sset)
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int blk = i * NW + wave_u + 4 * sset;
      const int r = blk * TL::ROWS_PER_KB + lane / CPR;
      const int slot = lane % CPR;
      koff[sset][i] = (uint32_t)(((int64_t)r * row + (int64_t)hk * D + (slot ^ swz_k<D>(r)) * 8) * 2);
      voff[sset][i] = (uint32_t)(((int64_t)r * row + (int64_t)hk * D + (slot ^ swz_v<D>(r)) * 8) * 2);
    }
  auto issue = [&](int t) __attribute__((always_inline)) {
    // (wave-uniform; stated so the value stays on the scalar unit for m0)
    const uint32_t ks = __builtin_amdgcn_readfirstlane(ring_base + ((t - t0) % NS) * TL::STAGE_BYTES);
    const uint32_t vs = ks + TL::TILE_BYTES;
    const int kbase = t * NK;
    const int64_t tile_elems = (int64_t)kbase * row;
    const uint16_t* kt = k + tile_elems;
    const uint16_t* vt = v + tile_elems;
    if (__builtin_expect(kbase + NK <= key_end, 1)) {
#pragma unroll
      for (int sset = 0; sset < NIW; ++sset)
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int blk = i * NW + wave_u + 4 * sset;
          lds_dma16_sv<NT>(kt, koff[sset][i], ks + blk * 1024);
          lds_dma16_sv<NT>(vt, voff[sset][i], vs + blk * 1024);
        }
    } else {
      asm volatile("" ::: "memory");  // (the ragged tile: a real branch)
#pragma unroll
      for (int sset = 0; sset < NIW; ++sset)
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int blk = i * NW + wave_u + 4 * sset;
          const int r = blk * TL::ROWS_PER_KB + lane / CPR;
          const int slot = lane % CPR;
          const int64_t g = (int64_t)min(kbase + r, key_end - 1) * row + (int64_t)hk * D;
          lds_dma16<NT>(k + g + (slot ^ swz_k<D>(r)) * 8, ks + blk * 1024);
          lds_dma16<NT>(v + g + (slot ^ swz_v<D>(r)) * 8, vs + blk * 1024);
        }
    }
  };

  // ---- S^T = K Q^T for tile t ------------------------------------------------
  // The K fragments of dim chunk kc+1 are read from LDS while the MFMAs of
  // chunk kc run (two register buffers), so LDS latency stays hidden.
  f32x4 s[QB][KB];
  auto qk = [&](int t) __attribute__((always_inline)) {
    const unsigned char* ks = ring[(t - t0) % NS];
    auto kfrag = [&](int kc, int kb) __attribute__((always_inline)) {
      const int key = key_of(kb, ln);
      const int col = kc * 4 + lg;
      return *reinterpret_cast<const bf16x8*>(ks + key * ROWB + ((col ^ swz_k<D>(key)) * 16));
    };
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 a[2][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) a[0][kb] = kfrag(0, kb);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (kc + 1 < KC) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) a[(kc + 1) & 1][kb] = kfrag(kc + 1, kb);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kc & 1][kb], qf[qb][kc], s[qb][kb], 0, 0, 0);
    }
    // the K fragments of chunk 0 first, then per fragment its QB MFMAs and
    // the read of a fragment one chunk later
    __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);
#pragma unroll
    for (int i = 0; i < KC * KB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // ---- online softmax of tile t (base 2, lazy rescale) -> packed P^T --------
  uint32_t pb[QB][CH][4];  // P^T as packed bf16 pairs: the P.V B operand
  // Scaled scores of keys outside the visible range set to -inf: the split's
  // ragged last tile, or (CAUSAL) keys past a query.  Taken only on tiles
  // that have such keys (wave-uniform test).
  auto mask_tile = [&](int t) __attribute__((always_inline)) {
    const int kbase = t * NK;
    if (__builtin_expect(kbase + NK > key_end || (CAUSAL && kbase + NK - 1 > q0), 0)) {
      // the empty asm keeps this rare block a branch: without it the compiler
      // turns the masking into compares and selects run on every tile
      asm volatile("" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 32 * (kb >> 1) + 8 * lg + 4 * (kb & 1) + i;
            if (kbase + key >= key_end || (CAUSAL && kbase + key > q0 + qb * 16 + ln)) s[qb][kb][i] = -INFINITY;
          }
    }
  };
  auto softmax = [&](int t) __attribute__((always_inline)) {
    // scaled scores x = s * |c| first, the mask after: a masked key is
    // x = -inf whatever the scale (scaling -inf by a zero scale would be NaN)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[qb][kb] *= cabs;
    mask_tile(t);
    // running maxima: lane (query ln, group lg) holds 4*KB keys of its query;
    // reduce over the 4 groups with lane swaps
    float tmax[QB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float smax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) smax = fmaxf(smax, s[qb][kb][i]);
      tmax[qb] = max_xor32(max_xor16(smax));
      grow |= tmax[qb] > m[qb] + kLazyTau;
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {  // wave-uniform, rare after the first tile
      asm volatile("" ::: "memory");  // (kept a branch: no rescale multiplies on other tiles)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mn = fmaxf(m[qb], tmax[qb]);
        const float alpha = fast_exp2(m[qb] - mn);
        m[qb] = mn;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mneg = -m[qb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[qb][kb][i] = fast_exp2(s[qb][kb][i] + mneg);
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        pb[qb][ch][0] = pack_bf16x2(s[qb][2 * ch][0], s[qb][2 * ch][1]);
        pb[qb][ch][1] = pack_bf16x2(s[qb][2 * ch][2], s[qb][2 * ch][3]);
        pb[qb][ch][2] = pack_bf16x2(s[qb][2 * ch + 1][0], s[qb][2 * ch + 1][1]);
        pb[qb][ch][3] = pack_bf16x2(s[qb][2 * ch + 1][2], s[qb][2 * ch + 1][3]);
      }
    }
  };

  // fast pass: p = exp2(x) with the fixed reference 0
  auto softmax_fast = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[qb][kb] *= cabs;  // scaled first, masked after (as in softmax)
    mask_tile(t);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        float pv_[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv_[i] = fast_exp2(s[qb][2 * ch][i]);
          pv_[4 + i] = fast_exp2(s[qb][2 * ch + 1][i]);
        }
        pb[qb][ch][0] = pack_bf16x2(pv_[0], pv_[1]);
        pb[qb][ch][1] = pack_bf16x2(pv_[2], pv_[3]);
        pb[qb][ch][2] = pack_bf16x2(pv_[4], pv_[5]);
        pb[qb][ch][3] = pack_bf16x2(pv_[6], pv_[7]);
      }
  };

  // ---- O^T += V^T P^T for tile t (and the row sums, on the matrix cores) ----
  // V operands are read with the transposing LDS load two (chunk, dim-block)
  // steps ahead of the MFMAs that use them.
  auto pv = [&](int t) __attribute__((always_inline)) {
    const unsigned char* vs = ring[(t - t0) % NS] + TL::TILE_BYTES;
    auto vfrag = [&](int ch, int db) __attribute__((always_inline)) {
      // lane (ln, lg) points at row 32ch + 8lg + 4half + ln/4, dims db*16 + 4(ln%4) .. +4
      bf16x4 half2[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key = 32 * ch + 8 * lg + 4 * half + (ln >> 2);
        const int dim = db * 16 + 4 * (ln & 3);
        const int chunk = dim >> 3;
        const unsigned char* src = vs + key * ROWB + ((chunk ^ swz_v<D>(key)) * 16) + (dim & 7) * 2;
        half2[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(src));
      }
      return __builtin_shufflevector(half2[0], half2[1], 0, 1, 2, 3, 4, 5, 6, 7);
    };
    constexpr int NSTEP = CH * DB;
    constexpr int AHEAD = 2;
    bf16x8 va[AHEAD + 1];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) va[i] = vfrag(i / DB, i % DB);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      const int ch = i / DB, db = i % DB;
      if (i + AHEAD < NSTEP) va[(i + AHEAD) % (AHEAD + 1)] = vfrag((i + AHEAD) / DB, (i + AHEAD) % DB);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const u32x4 bw = u32x4{pb[qb][ch][0], pb[qb][ch][1], pb[qb][ch][2], pb[qb][ch][3]};
        o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[i % (AHEAD + 1)], __builtin_bit_cast(bf16x8, bw),
                                                            o[qb][db], 0, 0, 0);
      }
      if (db == DB - 1) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const u32x4 bw = u32x4{pb[qb][ch][0], pb[qb][ch][1], pb[qb][ch][2], pb[qb][ch][3]};
          lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, bw), lsum[qb], 0, 0, 0);
        }
      }
    }
    // instruction order for the scheduler: the transposing reads of the
    // first PV_LEAD steps first, then per step its MFMAs and the reads of a
    // later step, so LDS latency hides behind PV_LEAD steps of MFMAs
    constexpr int PV_LEAD = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV_LEAD, 0);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i % DB == DB - 1) __builtin_amdgcn_sched_group_barrier(0x008, 2 * QB, 0);  // + the row-sum MFMAs
      else __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // ---- pipeline -----------------------------------------------------------------
  // The loads of tile t+NS-2 are issued in iteration t (tiles t-1 and t are
  // read in iteration t, t+1 .. t+NS-2 are in flight): right after the
  // barrier with one wave per SIMD, by group A at the end of its part with
  // two.  Waves of group A (all waves, or the first half when two waves
  // share a SIMD) run
  //     [P.V(t-1), QK(t)] (matrix cores) then softmax(t) (vector ALUs);
  // group B runs the same work shifted by half an iteration,
  //     softmax(t-1) then [P.V(t-1), QK(t)],
  // so after each barrier one wave of every SIMD is on the matrix cores while
  // the other is on the vector ALUs.
  static_assert(NS >= 3 && NS <= 6, "ring depth");
  constexpr int AHEAD_T = NS - 2;  // tiles in flight
  // wait until tile t has landed: at most n later tiles of this wave in flight
  auto wait_tiles = [&](int n) __attribute__((always_inline)) {
    if (n <= 0) wait_vmcnt<0>();
    else if (n == 1) wait_vmcnt<2 * NLD * NIW>();
    else if (n == 2) wait_vmcnt<4 * NLD * NIW>();
    else wait_vmcnt<6 * NLD * NIW>();
  };
  // waves w and w + 4 share a SIMD: alternate groups by (w / 4)
  const bool grp_b = NW >= 8 && ((wave >> 2) & 1);
  auto pipeline = [&](auto fast_tag) __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_tag)::value;
    auto smx = [&](int t) __attribute__((always_inline)) {
      if constexpr (FAST) softmax_fast(t);
      else softmax(t);
    };
    if (t0 < t1) {
      const bool issuer = !grp_b;  // loads are issued (and waited for) by group A only
#pragma unroll
      for (int i = 0; i < AHEAD_T; ++i)
        if (t0 + i < t1 && issuer) issue(t0 + i);
      for (int t = t0; t < t1; ++t) {
        if (issuer) wait_tiles(min(AHEAD_T - 1, t1 - 1 - t));  // tile t landed (group A's loads: all of it)
        __builtin_amdgcn_s_barrier();   // tile t is in LDS, and every wave is done with
        asm volatile("" ::: "memory");  // tile t-2 (its stage is refilled in this iteration)
        if (NW < 8 && t + AHEAD_T < t1) issue(t + AHEAD_T);
        // A wave on the matrix cores runs at raised priority, so that the
        // SIMD's arbiter feeds its MFMAs first and the other wave's vector
        // work fills the issue slots in between.
        if (!grp_b) {
          __builtin_amdgcn_s_setprio(1);
          if (t > t0) pv(t - 1);
          qk(t);
          __builtin_amdgcn_s_setprio(0);
          smx(t);
          if (NW >= 8 && t + AHEAD_T < t1) issue(t + AHEAD_T);  // into tile t-2's stage
        } else {
          if (t > t0) {
            smx(t - 1);
            __builtin_amdgcn_s_setprio(1);
            pv(t - 1);
          } else {
            __builtin_amdgcn_s_setprio(1);
          }
          qk(t);
          __builtin_amdgcn_s_setprio(0);
        }
      }
      if (grp_b) smx(t1 - 1);
      pv(t1 - 1);
    }
  };
  auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m[qb] = -INFINITY;
      lsum[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  pipeline(std::integral_constant<bool, true>{});
  // every row sum of the workgroup within [2^-64, 2^64] (NaN fails too)?
  bool bad = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lsum[qb][0];
    bad |= !(lt >= 0x1p-64f && lt <= 0x1p64f);
  }
  const bool wave_bad = t0 < t1 && __builtin_amdgcn_ballot_w64(bad) != 0;  // (all lanes vote)
  if (lane == 0) redo = 0;
  __syncthreads();
  if (wave_bad && lane == 0) atomicOr(&redo, 1);
  __syncthreads();  // also: every wave is done with the ring
  const bool exact = __builtin_amdgcn_readfirstlane(redo) != 0;
  if (exact) {  // workgroup-uniform, rare
    reset_state();
    pipeline(std::integral_constant<bool, false>{});
  }

  // ---- partial state of this split -------------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lsum[qb][0];
    const int p = q0 + qb * 16 + ln;
    if (CAUSAL && out && p < Ldoc) {  // (G = 1, B = 1 in the prefill: query p is slot p)
      const float inv = 1.f / lt;  // a document slot sees at least slot 0
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<uint2*>(out + ((int64_t)p * Hq + h) * D + db * 16 + 4 * lg) =
            make_uint2(pack_bf16x2(o[qb][db][0] * inv, o[qb][db][1] * inv),
                       pack_bf16x2(o[qb][db][2] * inv, o[qb][db][3] * inv));
    } else if (p < PQ) {
      const int64_t sh = ((int64_t)split * bt.B * P + b * P + p / G) * Hq + h * G + p % G;
      // reference of the split's state: 0 in the fast pass, the running
      // maximum in the exact pass; an empty split has none (-inf)
      const float mref = t0 >= t1 ? -INFINITY : (exact ? m[qb] : 0.f);
      if (lg == 0) part_ml[sh] = make_float2(mref, lt);
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDocThreads) void doc_valu_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v, int P, int H, float c,
    const int32_t* __restrict__ plan, int64_t seq_len, int n_splits, float* __restrict__ part_o,
    float2* __restrict__ part_ml, Batch bt, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float lk[kF32NK][D];
  __shared__ __attribute__((aligned(16))) float lv[kF32NK][D];
  const int split = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int nz = (int)gridDim.z / bt.B;  // query tiles per request (as in doc_mfma_bf16_kernel)
  const int b = (int)blockIdx.z / nz, zt = (int)blockIdx.z % nz;
  const int pt = CAUSAL ? nz - 1 - zt : zt;
  const int p = pt * kDocThreads + tid;  // query s * G + g of key/value head h
  const int G = bt.G, PQ = P * G, Hq = H * G;
  k += b * bt.kv_stride;
  v += b * bt.kv_stride;
  const int Ldoc = (int)min<int64_t>(load_doc_len(plan + b), seq_len);  // a plan never exceeds the slots given
  int L = Ldoc;
  if constexpr (CAUSAL) L = min(L, (pt + 1) * kDocThreads);  // see doc_mfma_bf16_kernel
  const int n_tiles = (L + kF32NK - 1) / kF32NK;
  const int t0 = (int)((int64_t)split * n_tiles / n_splits);
  const int t1 = (int)((int64_t)(split + 1) * n_tiles / n_splits);
  const int key_end = min(t1 * kF32NK, L);
  const int64_t row = (int64_t)(H / bt.kv_group) * D;  // key/value heads (see doc_mfma_bf16_kernel)

  float qv[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = p < PQ ? q[((int64_t)(b * P + p / G) * Hq + h * G + p % G) * D + e] : 0.f;
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
        kk = *reinterpret_cast<const float4*>(k + (int64_t)gk * row + (int64_t)(h / bt.kv_group) * D + col * 4);
        vv = *reinterpret_cast<const float4*>(v + (int64_t)gk * row + (int64_t)(h / bt.kv_group) * D + col * 4);
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
      x[j] = (kbase + j < key_end && (!CAUSAL || kbase + j <= p)) ? d * c : -INFINITY;
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
  if (CAUSAL && out && p < Ldoc) {  // a document slot's output is final (see doc_mfma_bf16_kernel)
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < D; e += 4)
      *reinterpret_cast<float4*>(out + ((int64_t)p * Hq + h) * D + e) =
          make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
  } else if (p < PQ) {
    const int64_t sh = ((int64_t)split * bt.B * P + b * P + p / G) * Hq + h * G + p % G;
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
    // 16-query blocks per wave and waves per workgroup: (1, 4) for P <= 64,
    // (2, 4) for P <= 128, else (2, 8): 256 queries of a head per workgroup
    // as 8 waves of 32 queries, two waves per SIMD
    pl.qb = P <= 64 ? 1 : 2;
    pl.nw = P <= 128 ? 4 : 8;
    const int per_wg = 16 * pl.qb * pl.nw;
    pl.n_ptiles = (P + per_wg - 1) / per_wg;
    per_cu = 1;
  } else {
    pl.qb = 0;
    pl.nw = 4;
    pl.n_ptiles = (P + kDocThreads - 1) / kDocThreads;
    per_cu = 2;
  }
  // As many splits as fill the resident slots in one round, never more:
  // with base workgroups per split, a count past floor(slots / base) starts a
  // second, partly idle round that costs as much as the first (e.g. 28
  // workgroups per split on 256 CUs: 9 splits, 252 workgroups, one round;
  // 10 splits would take two rounds of 1/10 of the work).  Monotone in the
  // CU count, so the workspace sized for 256 CUs covers every device.
  const int64_t base = (int64_t)H * pl.n_ptiles;
  int64_t want = ((int64_t)num_cus * per_cu) / base;
  const int64_t max_by_len = (seq_len + 255) / 256;  // at least ~256 slots of the upper bound per split
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  if (want > 256) want = 256;
  pl.n_splits = (int)want;
  return pl;
}

int doc_query_tile(const DocPlan& pl, pp_dtype_t dtype) {
  return dtype == PP_BF16 ? 16 * pl.qb * pl.nw : kDocThreads;
}

hipError_t launch_doc(const DocPlan& pl, const void* q, const void* k, const void* v, int64_t seq_len, int P, int H,
                      int d, pp_dtype_t dtype, float c, const Workspace& ws, hipStream_t stream, bool causal,
                      const Batch& bt, void* out, bool stream_nt) {
  const dim3 grid(pl.n_splits, H, pl.n_ptiles * bt.B);
  if (dtype == PP_BF16) {
    auto* qq = static_cast<const uint16_t*>(q);
    auto* kk = static_cast<const uint16_t*>(k);
    auto* vv = static_cast<const uint16_t*>(v);
    // one query tile per key/value head: each tile of keys and values is read
    // by one workgroup only
    const bool nt = stream_nt && !causal && pl.n_ptiles == 1 && bt.kv_group == 1;
#define PP_DOC_LAUNCH(DD, QQ, WW)                                                                                 \
  (causal ? launch_kernel(doc_mfma_bf16_kernel<DD, QQ, WW, true>, grid, dim3(64 * WW), stream, qq, kk, vv, P, H,       \
                          c, ws.plan, seq_len, pl.n_splits, ws.part_o, ws.part_ml, bt, static_cast<uint16_t*>(out))       \
   : nt   ? launch_kernel(doc_mfma_bf16_kernel<DD, QQ, WW, false, true>, grid, dim3(64 * WW), stream, qq, kk, vv, P, \
                          H, c, ws.plan, seq_len, pl.n_splits, ws.part_o, ws.part_ml, bt, nullptr)                        \
          : launch_kernel(doc_mfma_bf16_kernel<DD, QQ, WW, false>, grid, dim3(64 * WW), stream, qq, kk, vv, P, H, c,     \
                          ws.plan, seq_len, pl.n_splits, ws.part_o, ws.part_ml, bt, nullptr))
    // dispatch on the exact (d, 16-query blocks per wave, waves) triple
    const int cfg = d * 10000 + pl.qb * 100 + pl.nw;
    switch (cfg) {
      case 1280104: return PP_DOC_LAUNCH(128, 1, 4);
      case 1280204: return PP_DOC_LAUNCH(128, 2, 4);
      case 1280208: return PP_DOC_LAUNCH(128, 2, 8);
      case 640104: return PP_DOC_LAUNCH(64, 1, 4);
      case 640204: return PP_DOC_LAUNCH(64, 2, 4);
      case 640208: return PP_DOC_LAUNCH(64, 2, 8);
      default: return hipErrorInvalidConfiguration;
    }
#undef PP_DOC_LAUNCH
  } else {
    auto* qq = static_cast<const float*>(q);
    auto* kk = static_cast<const float*>(k);
    auto* vv = static_cast<const float*>(v);
#define PP_F32_LAUNCH(DD, CC)                                                                                \
  launch_kernel(doc_valu_f32_kernel<DD, CC>, grid, dim3(kDocThreads), stream, qq, kk, vv, P, H, c, ws.plan, seq_len, \
                pl.n_splits, ws.part_o, ws.part_ml, bt, static_cast<float*>(out))
    if (d == 128) return causal ? PP_F32_LAUNCH(128, true) : PP_F32_LAUNCH(128, false);
    return causal ? PP_F32_LAUNCH(64, true) : PP_F32_LAUNCH(64, false);
#undef PP_F32_LAUNCH
  }
}

}  // namespace pp
