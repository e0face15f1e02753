/*
 * ppattn.h -- C ABI of the Parallel Prompting decode-step attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (Parallel Prompting project page, "How it works", item 1, the
 * stream mask; arXiv abstract of "Read Once, Answer Many"): P answer streams
 * of one request are packed after a shared document in one KV cache.  Every
 * KV slot carries a stream id.  At one decode step each stream has one query
 * token, and stream s attends only to the document and to its own slots.
 * The page states that each answer is then the same as decoding its question
 * alone; this library computes exactly that result, reading the document's
 * K/V once for all P streams (the page's "one matrix x matrix product"
 * instead of one vector x matrix product per question).
 *
 * Definition of out, for every stream s in [0,P) and head h in [0,H):
 *   V_s = { j < seq_len : stream_id[j] == 0 || stream_id[j] == s + 1 }
 *   x_j = scale * dot(q[s,h,:], k_cache[j,h,:])
 *   out[s,h,:] = sum_{j in V_s} softmax_j(x) * v_cache[j,h,:]
 *   out[s,h,:] = 0 when V_s is empty.
 * Id encoding: 0 = document, s+1 = stream s (the page's document id -1 and
 * streams 0..P-1, shifted by one).  Ids outside {0..P} are visible to no
 * stream (they are not an error).  No position test is made: every cached
 * slot precedes the decode query; whether the query's own K/V is already in
 * the cache is the caller's choice.  The leading run of id-0 slots is the
 * document fast path; id-0 slots after that run are still visible to every
 * stream (handled with the streams' own slots).
 *
 * Layouts (all row-major, contiguous, caller-owned DEVICE memory, 16-byte
 * aligned):
 *   q         [P, H, d]         element type `dtype`
 *   k_cache   [T >= seq_len, H, d]  element type `dtype`; only the first
 *   v_cache   [T >= seq_len, H, d]  seq_len slots are ever read
 *   stream_id [T >= seq_len]    int32
 *   out       [P, H, d]         element type `dtype` (bf16 results are rounded
 *                               to nearest even); every element is written
 * Arithmetic: bf16 or fp32 inputs, fp32 accumulation and softmax.
 *
 * Ownership and asynchrony: the library allocates no memory.  Scratch space
 * is the caller's `workspace` (device memory of at least
 * pp_attn_workspace_bytes(...) bytes, 16-byte aligned).  Work is enqueued on
 * `hip_stream` (a hipStream_t of the current device; NULL = the null
 * stream) and the call returns
 * without waiting and without reading device data on the host.  Inputs,
 * `out` and `workspace` must stay valid until the stream has passed the
 * call.  Two calls that run at the same time must not share a workspace.
 * The library keeps no mutable global state besides a once-per-device cache
 * of device properties; it is safe to call from several host threads.
 *
 * Errors: every entry point returns a pp_status_t and never throws or
 * aborts.  Arguments are checked on the host before any HIP call:
 *   PP_ERR_INVALID_ARG  null pointer, P/H/seq_len < 1, seq_len or P too
 *                       large, non-finite scale, misaligned pointer, `out`
 *                       overlapping an input or the workspace
 *   PP_ERR_UNSUPPORTED  d not in {64, 128}, unknown dtype
 *   PP_ERR_WORKSPACE    workspace null or smaller than required
 *   PP_ERR_HIP          a HIP launch or device query failed
 * Device data is not validated: NaN/Inf in K/V slots a stream does not see
 * never reach that stream's output.  pp_last_error_message() gives a
 * human-readable reason for the calling thread's last failure.
 */
#ifndef PPATTN_H
#define PPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PP_ABI_VERSION 2

typedef enum {
  PP_OK = 0,
  PP_ERR_INVALID_ARG = 1,
  PP_ERR_UNSUPPORTED = 2,
  PP_ERR_WORKSPACE = 3,
  PP_ERR_HIP = 4
} pp_status_t;

typedef enum { PP_BF16 = 0, PP_F32 = 1 } pp_dtype_t;

/* Largest accepted seq_len and P. */
#define PP_MAX_SEQ_LEN ((int64_t)1 << 30)
#define PP_MAX_STREAMS 65535
#define PP_MAX_HEADS 65535
#define PP_MAX_REQUESTS 65535

/* ABI version of the loaded library (PP_ABI_VERSION at build time). */
int pp_abi_version(void);

/* Static description of a status code. */
const char* pp_status_string(pp_status_t status);

/* Reason for the calling thread's most recent non-OK status ("" if none). */
const char* pp_last_error_message(void);

/* Bytes of workspace that pp_attn_decode, pp_attn_decode_batched,
 * pp_attn_decode_planned and pp_attn_decode_append need for this shape (one
 * size serves all of them).  Returns 0 for arguments that either
 * entry point would reject. */
size_t pp_attn_workspace_bytes(int64_t seq_len, int32_t P, int32_t H, int32_t d, pp_dtype_t dtype);

/* One decode step of multi-stream shared-document attention (definition
 * above).  The document prefix is read once for all streams: its K/V tiles
 * are staged in LDS and contracted against all P queries of a head with
 * matrix-core (MFMA) products, split over the document into partial softmax
 * states; each stream's own slots are gathered by that stream only; partial
 * states are merged in a fixed order, so results are bitwise reproducible
 * run to run.  [Parallel Prompting project page, "How it works": stream mask,
 * document read once per step for all streams.] */
pp_status_t pp_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* stream_id, int64_t seq_len, int32_t P, int32_t H,
                           int32_t d, float scale, void* out, pp_dtype_t dtype, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc:
 * pp_attn_decode without a workspace argument.  Its workspace is a fixed
 * scratch array of the library in each GPU's memory,
 * PP_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load until the
 * process ends; the call itself allocates nothing.  Shapes whose
 * pp_attn_workspace_bytes exceeds that size are rejected with
 * PP_ERR_WORKSPACE.  Every call on one GPU uses the same array: calls that
 * overlap on a GPU (other streams, other host threads) race and must be
 * serialized by the caller.  The array used is the current device's:
 * a non-null hip_stream of another device is rejected with
 * PP_ERR_INVALID_ARG.  Arguments, results and the other errors as
 * pp_attn_decode (PP_ERR_HIP also if the array's device address cannot be
 * obtained). */
#define PP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pp_status_t pp_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* stream_id, int64_t seq_len, int32_t P, int32_t H,
                                   int32_t d, float scale, void* out, pp_dtype_t dtype, void* hip_stream);

/* The same result computed as P independent requests ("batched requests",
 * one request per question, as a stock serving engine runs them): every
 * stream reads the whole document's K/V for itself with a per-query
 * split-K GEMV, then its own slots.  [Parallel Prompting project page,
 * illustration "Inside decode step" and "How it works": a per-question
 * request reads the document once per question per step.]  Provided as the
 * comparison baseline; same arguments and contract as pp_attn_decode. */
pp_status_t pp_attn_decode_batched(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* stream_id, int64_t seq_len, int32_t P, int32_t H,
                                   int32_t d, float scale, void* out, pp_dtype_t dtype,
                                   void* workspace, size_t workspace_bytes, void* hip_stream);

/* pp_attn_decode with a visibility plan computed earlier by pp_attn_plan for
 * the same stream_id and seq_len, instead of computing it again: a decode
 * step applies the same stream rule in every layer (Parallel Prompting
 * project page, "How it works", item 1: the stream id of a KV slot decides
 * its visibility; the ids do not change between the layers of a step), so
 * one plan per step serves all of them.
 *   plan_doc_len   device int32[1], as written by pp_attn_plan
 *   plan_counts    device int32[P]
 *   plan_slots     device int32[P * plan_capacity] (NULL if plan_capacity is
 *                  0); lists longer than plan_capacity are completed on the
 *                  device from stream_id
 * The plan buffers are read only and caller-owned; they must not overlap
 * `out` or the workspace (PP_ERR_INVALID_ARG), and must hold the plan of
 * this stream_id (a stale plan gives wrong results, it is not detected).
 * Other arguments, results and errors as pp_attn_decode. */
pp_status_t pp_attn_decode_planned(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* stream_id, int64_t seq_len, int32_t P, int32_t H,
                                   int32_t d, float scale, void* out, pp_dtype_t dtype,
                                   const int32_t* plan_doc_len, const int32_t* plan_counts,
                                   const int32_t* plan_slots, int64_t plan_capacity,
                                   void* workspace, size_t workspace_bytes, void* hip_stream);

/* Several Parallel Prompting requests in one launch, with grouped key/value
 * heads (Parallel Prompting project page: the best number of streams per
 * request is 16-64, so a server batches requests; its real-benchmark model
 * shares each key/value head between several query heads).  Request b has
 * its own document, P streams, stream ids and caches; within a request the
 * definition of pp_attn_decode holds, with query head hq of a stream reading
 * key/value head hq / (Hq / Hkv):
 *   q          [B, P, Hq, d]               out [B, P, Hq, d]
 *   k_cache,   [B, max_seq_len, Hkv, d]    (request b's slot j at row
 *   v_cache                                 b * max_seq_len + j)
 *   stream_id  [B, max_seq_len] int32      (per request: 0 = its document,
 *                                           s + 1 = its stream s)
 *   seq_lens   device int32[B]: request b's seq_len, clamped on the device to
 *              [0, max_seq_len] (0: its streams see nothing, out is zero)
 *   active     device int32[B * P] or NULL (all active): 0 retires stream
 *              b * P + s -- it sees nothing, its output is zero and its
 *              per-stream work is skipped.
 * A server batching continuously (project page, "Continuous batching":
 * the batch is refilled as requests finish) keeps B request slots: a slot
 * whose request finished gets length 0 (idle, no document work) until the
 * next request's ids and caches are written there and its length set;
 * streams that finished early are retired with `active`.
 * Hq must be a multiple of Hkv.  The document kernel contracts each K/V tile
 * of a request against all P * Hq / Hkv queries of its key/value head.
 * Workspace: pp_attn_multi_workspace_bytes(max_seq_len, B, P, Hq, Hkv, d,
 * dtype).  Other contract and errors as pp_attn_decode (PP_ERR_INVALID_ARG
 * also for B out of [1, PP_MAX_REQUESTS], Hq % Hkv != 0, a null seq_lens, or
 * too many query tiles for the grid).  pp_attn_decode_multi_batched is the
 * per-question baseline of the same launch. */
size_t pp_attn_multi_workspace_bytes(int64_t max_seq_len, int32_t B, int32_t P, int32_t Hq, int32_t Hkv,
                                     int32_t d, pp_dtype_t dtype);
pp_status_t pp_attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* stream_id, const int32_t* seq_lens, const int32_t* active,
                                 int64_t max_seq_len, int32_t B, int32_t P, int32_t Hq, int32_t Hkv,
                                 int32_t d, float scale, void* out, pp_dtype_t dtype, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);
pp_status_t pp_attn_decode_multi_batched(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* stream_id, const int32_t* seq_lens,
                                         const int32_t* active, int64_t max_seq_len, int32_t B, int32_t P,
                                         int32_t Hq, int32_t Hkv, int32_t d, float scale, void* out,
                                         pp_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                         void* hip_stream);

/* Starts a decode step in which every stream appends one slot (Parallel
 * Prompting project page, "How it works": each decode step appends one token
 * per stream and has a fixed shape, so a whole step can be captured once as
 * a HIP graph and replayed).  The step's start lives in device memory, so
 * the same launches serve every step:
 *   base_len       device int32[1]: slots already in the cache; the step's
 *                  new slots are base_len[0] + s for s in [0, P), and the
 *                  step's length is seq_len = base_len[0] + P
 *   stream_id      device int32[max_seq_len]; this call writes
 *                  stream_id[base_len[0] + s] = s + 1
 *   plan_head      device int32[2], written: {doc_len, seq_len}
 *   plan_counts    device int32[P], written: slots past doc_len that stream
 *                  s sees (including its new one)
 *   plan_slots     device int32[P * plan_capacity], written: the first
 *                  plan_capacity of them per stream, ascending (NULL when
 *                  plan_capacity is 0)
 * That is pp_attn_plan over the ids with the new slots written.  The
 * caller advances base_len[0] by P between steps (on the stream, e.g. inside
 * the captured graph).  A base_len[0] outside [0, max_seq_len - P] writes an
 * empty plan ({0, 0}, counts 0) and no id; the layers of such a step write
 * nothing to the caches and zeros to out.  One plan serves every layer of
 * the step (pp_attn_decode_append).  Buffers are caller-owned device memory
 * and must not overlap each other, stream_id or base_len
 * (PP_ERR_INVALID_ARG); stream_id 16-byte aligned.  Errors as above. */
pp_status_t pp_step_plan(int32_t* stream_id, const int32_t* base_len, int64_t max_seq_len, int32_t P,
                         int32_t* plan_head, int32_t* plan_counts, int32_t* plan_slots,
                         int64_t plan_capacity, void* hip_stream);

/* One layer of a decode step started by pp_step_plan: append, then attend.
 * For every stream s, with seq_len = plan_head[1] and its new slot
 * j_s = seq_len - P + s:
 *   pos_s  = plan_head[0] + plan_counts[s] - 1, the shared position of the
 *            new token: the number of slots stream s sees before it (Parallel
 *            Prompting project page, "How it works", item 2: every stream's
 *            positions start right after the document, as if its question
 *            were the only one)
 *   rotary embedding at pos_s of q[s] and k_new[s], rotate-half pairs
 *   (i, i + d/2) turned by pos_s * rope_base^(-2i/d) (rope_base <= 0: no
 *   rotation), angles formed and reduced modulo 2*pi in double precision,
 *   their sine and cosine and the rotation in fp32, one rounding to `dtype`
 *   k_cache[j_s] = rotated k_new[s];  v_cache[j_s] = v_new[s]
 *   out = pp_attn_decode_planned(rotated q, k_cache, v_cache, stream_id,
 *                                seq_len, ...)  with the step's plan, query
 *         head h reading key/value head h / (Hq / Hkv).
 *   q                [P, Hq, d] element type `dtype`, device, read only
 *   k_new, v_new     [P, Hkv, d], device, read only
 *   k_cache, v_cache [max_seq_len, Hkv, d], device, rows j_s written
 *   out              [P, Hq, d]
 *   max_seq_len      host bound of every step's seq_len (sizes the caches,
 *                    stream_id and the workspace: pp_attn_multi_workspace_bytes(
 *                    max_seq_len, 1, P, Hq, Hkv, d, dtype), which is
 *                    pp_attn_workspace_bytes(max_seq_len, P, Hq, d, dtype)
 *                    when Hq == Hkv)
 * Hq must be a multiple of Hkv.  The caches must not overlap each other or
 * any other argument; k_new and v_new must not overlap out or the workspace
 * (PP_ERR_INVALID_ARG); rope_base must be finite.  Other arguments, results
 * and errors as pp_attn_decode_planned. */
pp_status_t pp_attn_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                  void* v_cache, const int32_t* stream_id, int64_t max_seq_len, int32_t P,
                                  int32_t Hq, int32_t Hkv, int32_t d, float scale, double rope_base,
                                  const int32_t* plan_head, const int32_t* plan_counts,
                                  const int32_t* plan_slots, int64_t plan_capacity, void* out,
                                  pp_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                  void* hip_stream);

/* The appending step for B requests at once (request slots of a server:
 * Parallel Prompting project page, "Continuous batching", where a finished
 * request's slot takes the next one).  Request b is what pp_step_plan and
 * pp_attn_decode_append do for one request, on its own rows:
 *   stream_id        device int32[B][max_seq_len]
 *   base_len         device int32[B]: request b's step starts at
 *                    base_len[b]; a value outside [0, max_seq_len - P]
 *                    marks an idle slot (empty plan, no id, cache row or
 *                    output written by the layers except zeros in out)
 *   active           device int32[B][P] or NULL: 0 retires stream s of
 *                    request b (it lists nothing and its output is zero;
 *                    its new slot gets its id, but no key or value is
 *                    written there: no stream sees that slot); give the
 *                    step's plan and its layers the same mask
 *   plan_head        device int32[2 * B], written: doc_len of requests
 *                    0..B-1, then their seq_len (for B = 1 the layout of
 *                    pp_step_plan)
 *   plan_counts      device int32[B][P];  plan_slots int32[B][P][plan_capacity]
 *   q, out           [B][P][Hq][d];  k_new, v_new [B][P][Hkv][d]
 *   k_cache, v_cache [B][max_seq_len][Hkv][d]
 * Workspace: pp_attn_multi_workspace_bytes(max_seq_len, B, P, Hq, Hkv, d,
 * dtype).  Buffers are caller-owned device memory; the overlap rules and
 * errors are those of the one-request calls, with PP_ERR_INVALID_ARG also for
 * B out of [1, PP_MAX_REQUESTS]. */
pp_status_t pp_step_plan_multi(int32_t* stream_id, const int32_t* base_len, const int32_t* active,
                               int64_t max_seq_len, int32_t B, int32_t P, int32_t* plan_head,
                               int32_t* plan_counts, int32_t* plan_slots, int64_t plan_capacity,
                               void* hip_stream);
pp_status_t pp_attn_decode_append_multi(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                        void* v_cache, const int32_t* stream_id, const int32_t* active,
                                        int64_t max_seq_len, int32_t B, int32_t P, int32_t Hq, int32_t Hkv,
                                        int32_t d, float scale, double rope_base, const int32_t* plan_head,
                                        const int32_t* plan_counts, const int32_t* plan_slots,
                                        int64_t plan_capacity, void* out, pp_dtype_t dtype, void* workspace,
                                        size_t workspace_bytes, void* hip_stream);

/* Prefill of the whole packed request -- the document and every stream's
 * question tokens as one sequence, attended once (Parallel Prompting project
 * page, "How it works" and its illustration: the document and all questions
 * go into one request, prefilled together).  Every slot i < seq_len is a
 * query, and it attends under the same stream rule, causally:
 *   V(i) = { j <= i : stream_id[j] == 0 || stream_id[j] == stream_id[i] }
 *   out[i,h,:] = sum_{j in V(i)} softmax_j(scale * dot(q[i,h,:], k[j,h,:])) * v[j,h,:]
 * A document slot sees the document up to itself; a stream's slot sees the
 * whole document before it and its own stream's slots up to itself (never
 * another stream's).  Layouts: q, out [seq_len, Hq, d] and k, v
 * [seq_len, Hkv, d] of `dtype` (Hq a multiple of Hkv: query head h reads
 * key/value head h / (Hq / Hkv); Hkv = Hq without grouping), stream_id
 * [seq_len] int32, contiguous, 16-byte aligned, device memory;
 * seq_len <= 65535 * 256.  The leading run of id-0 slots is contracted on
 * the matrix cores in query tiles (causal inside the run); each slot's
 * remaining visible slots past that run are compacted from stream_id and
 * gathered.  Workspace: pp_attn_prefill_workspace_bytes(seq_len, H, d,
 * dtype) bytes.  Contract, asynchrony and errors as pp_attn_decode. */
size_t pp_attn_prefill_workspace_bytes(int64_t seq_len, int32_t Hq, int32_t d, pp_dtype_t dtype);
pp_status_t pp_attn_prefill(const void* q, const void* k, const void* v, const int32_t* stream_id,
                            int64_t seq_len, int32_t Hq, int32_t Hkv, int32_t d, float scale, void* out,
                            pp_dtype_t dtype, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Profiling variant of pp_attn_decode (batched == 0) or pp_attn_decode_batched
 * (batched != 0): identical arguments, contract and results, and it also
 * binds caller-created hipEvent_t events to the start and the end of each of
 * its kernels (hipExtLaunchKernel), so that hipEventElapsedTime(events[2i],
 * events[2i + 1]) is the execution time of stage i's kernel alone, on the
 * stream the kernels run on.  The stages, in launch order, are: visibility
 * plan, document part, own-slot gather + merge.  Needs n_events >=
 * PP_PROFILE_EVENTS (else PP_ERR_INVALID_ARG); a failed launch is
 * PP_ERR_HIP. */
#define PP_PROFILE_EVENTS 6
pp_status_t pp_attn_decode_profiled(int32_t batched, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* stream_id, int64_t seq_len, int32_t P, int32_t H, int32_t d,
                                    float scale, void* out, pp_dtype_t dtype, void* workspace,
                                    size_t workspace_bytes, void* hip_stream, void* const* events,
                                    int32_t n_events);

/* The integer visibility plan that both entry points evaluate on the device
 * (their first kernels), exposed for inspection: the same device code.
 * Writes, on `hip_stream`:
 *   doc_len_out[0]      length of the leading run of id-0 slots (<= seq_len)
 *   tail_count_out[s]   number of slots j >= doc_len visible to stream s
 *                       (its own slots and later id-0 slots)
 *   tail_slots_out[s*tail_capacity + i]  the first min(count, tail_capacity)
 *                       of those slots, ascending
 * All three are caller-owned device buffers (int32; tail_slots_out may be
 * NULL when tail_capacity is 0).  `workspace` is caller-owned device
 * scratch of at least pp_attn_plan_workspace_bytes(seq_len, P) bytes (never
 * less than PP_PLAN_WORKSPACE_BYTES); it must not overlap stream_id or the
 * outputs (PP_ERR_INVALID_ARG).  For P <= 1024 the plan is built in two
 * passes over chunks of the ids (per-chunk counts of every stream's id, then
 * each visible slot placed at its rank in slot order), O(seq_len) work in
 * all; larger P take one pass per stream over all ids.  [Project page, "How
 * it works", item 1.]  Errors as above. */
#define PP_PLAN_WORKSPACE_BYTES 512
size_t pp_attn_plan_workspace_bytes(int64_t seq_len, int32_t P);
pp_status_t pp_attn_plan(const int32_t* stream_id, int64_t seq_len, int32_t P,
                         int32_t* doc_len_out, int32_t* tail_count_out, int32_t* tail_slots_out,
                         int64_t tail_capacity, void* workspace, size_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PPATTN_H */
