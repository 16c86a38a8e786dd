/*
 * attn_fwd.h - C ABI of libattn_fwd.so: causal grouped-query attention
 * forward (and its backward, attn_bwd) on AMD Instinct MI355X (gfx950).
 *
 * The operation is the attention fixture of the LuisaCompute "Attention
 * execution mapping" review, section 1: bottom-right causal GQA in which
 * query head h reads kv-head h / (Hq/Hkv) and key k is legal for query row q
 * when k <= q + K - Q, with the online-softmax state (row max, row sum,
 * accumulator) carried across KV blocks so one program covers prefill and
 * decode.  Int32 per-sequence lengths, unequal lengths, empty sequences,
 * sliding windows and finite padded rows come from the attention feature
 * list of the Laya "Fast backends" page (sections "TileLang portability" and
 * "Numerics").  Readings taken where the pages are silent:
 *   - with lengths, K_b = seqlens_k[b] replaces K in the offset:
 *     p(q) = q + K_b - Q, and keys k >= K_b do not exist;
 *   - window W > 0 keeps the W keys p(q)-W < k <= p(q); W <= 0 disables it;
 *   - a row with no legal key gets O = 0 and LSE = -inf;
 *   - LSE = ln(sum over legal k of exp(scale * q.k)), stored as float.
 *
 * Layouts: contiguous row-major [B, H, T, width] for every tensor:
 *   q [B, Hq, Q, D], k [B, Hkv, K, D], v [B, Hkv, K, Dv],
 *   o [B, Hq, Q, Dv], lse [B, Hq, Q] (float).
 * K is the padded key length; seqlens_k (int32[B], device memory) may be
 * NULL, meaning every K_b = K.  Base pointers must be 16-byte aligned.
 *
 * Every pointer argument is a DEVICE pointer.  `stream` is a hipStream_t
 * passed as void* (NULL = the null stream).  Calls are asynchronous: they
 * return after enqueueing kernels on `stream`, with no host synchronisation;
 * a device fault surfaces at the caller's next synchronisation.
 *
 * Ownership: the caller owns every buffer.  The library keeps no pointer to
 * a caller's buffer past the call's stream-ordered completion and frees
 * nothing it did not allocate.  Inputs are only read.  o and lse must not
 * alias the inputs.  Scratch for the split-KV passes (decode, and prefill
 * when its tiles are few) and for the backward is a library-owned device
 * buffer per (device, stream) the library has been called on: calls on one
 * stream share it in stream order, calls on different streams never share
 * one.  Each call makes its stream wait (on the GPU) for the buffer's
 * previous call, so a new stream that reuses a destroyed stream's handle
 * cannot overtake the old stream's work on it.  A call that needs more than
 * the buffer holds waits on the host for the buffer's previous call, then
 * frees and reallocates it (at least 1.5x, rounded to 2 MiB); no other call
 * synchronises with the host, so calls can be queued ahead of the GPU.  The
 * buffers are kept until attn_fwd_release_scratch or process exit.  Under
 * HIP graph capture a call uses the capturing stream's buffer as it stands:
 * make one call of the same or larger plan on that stream before capturing
 * (a capture that would need a larger buffer returns ATTN_ERR_HIP), and do
 * not run replays concurrently with other calls on that stream; or use
 * attn_fwd_noalloc.
 *
 * Head widths: D and Dv up to 128 run on kernels sized for them; wider
 * heads run on 8-wave forms of the prefill kernel (decode with more than 16
 * packed rows g*Q included; up to 16 such rows of heads up to 256 take the
 * split-KV decode kernel padded to 256): up to 256 with two 64-key K/V
 * blocks resident, up to 512 with
 * 32-key blocks and the output channels in parts of 256 on separate
 * workgroups that each recompute the scores (the FlyDSL post, "FMHA through
 * AOTriton", gives 512 a body of its own for the same LDS reason: two
 * resident 512-wide blocks do not fit).  The fp32 path stops at 128.
 *
 * seqlens_k is never read on the host.  Values outside [0, K] are a caller
 * error; the kernels clamp them to [0, K] so memory outside the tensors is
 * never touched.
 *
 * Environment (read at each call; for tests and tuning, not needed in use):
 *   ATTN_FWD_SPLIT_WORKERS=n   workers of the split-KV decode pass (n >= 1);
 *   ATTN_FWD_PREFILL_SPLITS=n  key-range pieces per prefill tile (n >= 1,
 *                              at most 32; rounded to whole pieces);
 *   ATTN_FWD_FAIL_ALLOC=1      every scratch allocation fails (the calls
 *                              that need scratch return ATTN_ERR_OOM);
 *   ATTN_FWD_CUS=n, ATTN_FWD_XCDS=n  compute units / XCDs the launch plans
 *                              assume (otherwise queried once per device).
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* nothing launched */
  ATTN_ERR_UNSUPPORTED = 2, /* nothing launched */
  ATTN_ERR_OOM = 3,         /* scratch allocation failed; nothing launched */
  ATTN_ERR_HIP = 4,         /* a HIP call or launch failed */
  ATTN_ERR_SCRATCH_LIMIT = 5 /* attn_fwd_noalloc: more scratch than it holds; nothing launched */
};

/*
 * bf16 inputs (q, k, v as bfloat16), bf16 output o, float lse.
 * Scores, softmax state and accumulators are float; the weights P are
 * rounded to bf16 before the P.V product (GPU intermediates keep the input
 * type, Laya "Fast backends", "TileLang portability").
 *
 * Returns:
 *   ATTN_ERR_INVALID_ARG  a negative size; Hq > 0 with Hkv == 0 or
 *                         Hq % Hkv != 0; a non-finite scale; q/o/lse NULL
 *                         while B*Hq*Q > 0; k/v NULL while B*Hkv*K > 0;
 *   ATTN_ERR_UNSUPPORTED  D or Dv not a multiple of 16 in [16, 512]
 *                         ([16, 128] for the fp32 path); or one
 *                         (batch, head) slice of 2 GiB or more in bf16
 *                         (Q*D, Q*Dv, K*D or K*Dv >= 2^30 elements);
 *   ATTN_ERR_OOM, ATTN_ERR_HIP as above;
 *   ATTN_OK               also when B*Hq*Q == 0 (nothing launched).
 * K == 0, or every K_b == 0, writes O = 0 and LSE = -inf for all rows.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Q, int K,
             int D, int Dv, const int32_t* seqlens_k, int window, float scale, void* stream);

/* Same contract with float q, k, v and float o; all arithmetic in float. */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq, int Hkv, int Q,
                 int K, int D, int Dv, const int32_t* seqlens_k, int window, float scale, void* stream);

/*
 * Options of attn_fwd_ex (bit flags; 0 gives attn_fwd).
 *   ATTN_FWD_FP16       q, k, v and o are IEEE binary16 instead of bfloat16,
 *                       and the weights P are rounded to binary16 before
 *                       the P.V product (the Laya "Fast backends" page,
 *                       "Numerics", compares GPU results on inputs rounded to
 *                       bf16 or fp16);
 *   ATTN_FWD_FP32       q, k, v and o are float: the attn_fwd_f32 path;
 *   ATTN_FWD_NONCAUSAL  no causal limit: every key k < K_b is legal for every
 *                       row (LuisaCompute "Attention execution mapping"
 *                       review, section 7, lists non-causal masks as the next
 *                       semantics to add).  Rows have no legal key only when
 *                       K_b == 0.  A window is measured back from the
 *                       diagonal, so window > 0 with this flag is rejected.
 * Everything else (layout, seqlens_k, ownership, scratch, status codes) is
 * as for attn_fwd.  Unknown flag bits, FP16 together with FP32, or
 * NONCAUSAL with window > 0 return ATTN_ERR_INVALID_ARG (nothing launched).
 */
enum attn_fwd_flags { ATTN_FWD_FP16 = 1, ATTN_FWD_FP32 = 2, ATTN_FWD_NONCAUSAL = 4 };

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Q,
                int K, int D, int Dv, const int32_t* seqlens_k, int window, float scale, int flags, void* stream);

/*
 * attn_fwd_ex for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, kernels, launch plan and results (bitwise those of
 * attn_fwd_ex), but the scratch of the split-KV passes is a 64 MiB array
 * held by the library on every GPU it runs on until the process ends, so
 * the call allocates and frees nothing.  The caller still passes every
 * input and output.  A plan whose scratch (attn_fwd_plan's workspace_bytes)
 * exceeds 64 MiB returns ATTN_ERR_SCRATCH_LIMIT with nothing launched; every
 * other status is as for attn_fwd_ex.  The first call on a device looks up
 * that device's copy of the array.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (on different streams, or queued
 * ahead of one another's completion on different streams) race; calls on
 * one stream are ordered and safe.
 */
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Q, int K, int D, int Dv, const int32_t* seqlens_k, int window, float scale, int flags,
                     void* stream);

/*
 * Paged K/V cache (block-table indirection, as a serving engine keeps it;
 * the LuisaCompute review, section 7, names paged KV among the cases its
 * validation matrix does not cover yet).  k_pages [num_pages, Hkv, page_size, D] and v_pages [num_pages, Hkv,
 * page_size, Dv] (contiguous; a page holds page_size consecutive keys of
 * every kv-head); block_table int32 [B, pages_per_seq] on the device: keys
 * j*page_size .. (j+1)*page_size - 1 of sequence b are in page
 * block_table[b*pages_per_seq + j].  The padded length is K = pages_per_seq *
 * page_size; seqlens_k, window, scale, flags (ATTN_FWD_FP16,
 * ATTN_FWD_NONCAUSAL) and everything else are as for attn_fwd_ex, computed
 * exactly as attn_fwd_ex on the cache gathered into [B, Hkv, K, width].
 * Pages may be shared between sequences.  page_size must be a power of two in
 * [64, 65536] and the 16-bit types are required: otherwise
 * ATTN_ERR_UNSUPPORTED.  A table entry outside [0, num_pages) is a caller
 * error; the kernels clamp it so no load leaves the cache.  Table entries of
 * pages past a sequence's K_b are never read.
 */
int attn_fwd_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse, int B, int Hq,
                   int Hkv, int Q, int D, int Dv, const int32_t* block_table, int pages_per_seq, int page_size,
                   int num_pages, const int32_t* seqlens_k, int window, float scale, int flags, void* stream);

/*
 * Backward of attn_fwd_ex: the gradients of sum(dO * O) with respect to q, k
 * and v (no gradient flows into the LSE output), for the same attention
 * (causal unless ATTN_FWD_NONCAUSAL, window, seqlens_k, scale).  The FlyDSL
 * post, "FMHA through AOTriton", describes this pass as separate dQ and dK/dV
 * kernels that reuse the forward's layouts; a kv-head's dK and dV sum over
 * its Hq/Hkv query heads.
 *
 * Inputs: q, k, v as given to the forward; o [B,Hq,Q,Dv] and lse [B,Hq,Q]
 * (float) as the forward returned them for those inputs; dout [B,Hq,Q,Dv].
 * Outputs: dq [B,Hq,Q,D], dk [B,Hkv,K,D], dv [B,Hkv,K,Dv], all in the
 * storage type (bf16, or IEEE binary16 with ATTN_FWD_FP16); every element is
 * written, keys at or past K_b get 0.  Sums are fp32; the weights and dS are
 * rounded to the storage type for the matrix products.  Deterministic (no
 * atomics).  Scratch (two floats per query row) is the stream's buffer, as
 * for the forward.
 *
 * Returns as attn_fwd_ex, and ATTN_ERR_UNSUPPORTED for ATTN_FWD_FP32 or D, Dv
 * outside multiples of 16 in [16, 256] (above 128, dK and dV are computed by
 * separate launches, each recomputing the weights).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
             void* dk, void* dv, int B, int Hq, int Hkv, int Q, int K, int D, int Dv, const int32_t* seqlens_k,
             int window, float scale, int flags, void* stream);

/*
 * Frees every scratch buffer the allocating entry points hold (one per
 * device and stream they were called on), after waiting for each of those
 * devices to finish its work.  Calls made afterwards allocate again.  Not
 * to be called while another host thread is inside a call of this library.
 * Returns ATTN_OK, or ATTN_ERR_HIP if a wait or free failed (the buffers
 * are forgotten either way).  This is the library's own memory management;
 * it computes nothing, so no passage of the attention write-ups defines it.
 */
int attn_fwd_release_scratch(void);

/* Static description of a status code; never NULL. */
const char* attn_fwd_strerror(int status);

/*
 * The launch plan attn_fwd would use for these sizes, without launching
 * anything (host only).  path: 0 = no launch, 1 = prefill kernel,
 * 2 = split-KV decode + combine.  On the decode path the keys of all
 * (batch, kv-head) groups, in 32-key sub-blocks laid end to end, are cut
 * into split_workers equal contiguous shares (0 when K == 0), each giving
 * one partial softmax state per group piece; partial_slots bounds the
 * pieces (B*Hkv + split_workers) and workspace_bytes is the scratch the
 * decode path needs for them (partial_slots * g*Q rows *
 * (Dv + 2) floats).  On the prefill path split_workers is the number of
 * pieces each 128-row tile's key range is cut into (1: none; more when the
 * tiles alone would leave most of the GPU idle), partial_slots the
 * (tile, piece) pairs and workspace_bytes their partial states
 * (partial_slots * 128 rows * (Dv + 2) floats); the fp32 path never
 * splits.  Returns the status attn_fwd would return for an argument
 * check.
 */
typedef struct attn_fwd_plan_t {
  int path;
  int split_workers;
  int partial_slots;
  int64_t workspace_bytes;
} attn_fwd_plan_t;

int attn_fwd_plan(int B, int Hq, int Hkv, int Q, int K, int D, int Dv, int window, attn_fwd_plan_t* plan);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
