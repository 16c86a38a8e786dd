// Internal declarations of libattn_fwd.so: kernel parameter block, launch
// helpers and the device-side building blocks shared by the gfx950 kernels.
// Nothing here is part of the public ABI (include/attn_fwd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn {

// Workgroup geometry of the bf16 prefill kernel: kPrefillWaves waves of 64
// lanes, each wave owning 32 query rows (two 16-column MFMA tiles), 64 keys
// per KV block.
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRowsPerWave = 32;
constexpr int kPrefillBM = kPrefillWaves * kPrefillRowsPerWave;  // query rows per workgroup
constexpr int kPrefillBN = 64;                                   // keys per block

// Prefill tiles: each covers 128 rows of the row list of one (batch, kv-head)
// group.  Row r of the list is query row r % Q of query head h_base + r / Q.
// Per-head tiles (the list is one head's Q rows) are used when Q >= 128 or
// the group has one head; packed tiles (the list is the g*Q rows of the
// group's heads, head-major) when a head has fewer rows than a tile, so one
// tile holds the rows of several heads, which share every K/V block (the
// short query runs of chunked prefill and speculative decoding).
__host__ __device__ inline bool prefill_packed(int Q, int group) { return group > 1 && Q < kPrefillBM; }
// Tiles of one (batch, kv-head) group.
__host__ __device__ inline int prefill_group_tiles(int Q, int group) {
  const int n_qt = (Q + kPrefillBM - 1) / kPrefillBM;
  return prefill_packed(Q, group) ? (group * Q + kPrefillBM - 1) / kPrefillBM : group * n_qt;
}
// Split-KV prefill: when the tiles alone leave most workgroup slots of the
// chip idle (few long sequences), or hold so few rows that one long sequence
// would keep a single workgroup busy long after the rest (decode-like tiles
// over lengths that vary), each tile's key range is cut into pieces of a
// fixed number of blocks, processed by separate workgroups that write fp32
// partial states; a combine pass merges them.  A tile whose range is short
// leaves its later pieces empty.  At most kPrefillMaxSplits pieces, each at
// least kPrefillMinSplitBlocks blocks (kPrefillMinSplitBlocksIdle while the
// pieces would not give every CU a workgroup).
constexpr int kPrefillMaxSplits = 32;
constexpr int kPrefillMinSplitBlocks = 32;
constexpr int kPrefillMinSplitBlocksIdle = 16;

// Split-KV decode: single-wave workers streaming 32-key sub-blocks, each an
// equal share of all (batch, kv-head) groups' sub-blocks.
constexpr int kDecodeSub = 32;
constexpr int kDecodeMaxRows = 32;  // g*Q rows packed per (batch, kv-head)
// Any Q whose g*Q rows fit the two 16-row MFMA tiles takes the split-KV path
// (decode Q = 1..4, and the short query runs of speculative decoding or
// chunked prefill): the packed rows share each K/V read.
constexpr int kDecodeMaxQ = kDecodeMaxRows;
// Heads wider than 128 (up to 256) take the split-KV path only up to this many
// packed rows (one 16-row MFMA tile).
constexpr int kDecodeMaxRowsWide = 16;
// Each worker of the split pass takes at least kDecodeMinShare sub-blocks.
constexpr int kDecodeMinShare = 4;

// fp32 path: one workgroup of 256 threads per (batch, head, 16 query rows).
constexpr int kF32Rows = 16;
constexpr int kF32Keys = 32;

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seqlens;  // may be null: every K_b = K
  int B, Hq, Hkv, Q, K, D, Dv;
  int window;              // <= 0: none
  int causal_shift;        // 0, or kNonCausalShift: no causal limit (see row_delta)
  int f16;                 // bf16 kernels: 1 when q, k, v, o are IEEE binary16 instead of bf16
  int group;               // Hq / Hkv
  int q_sign;              // 0x8000 when the scale is negative (q is negated), else 0
  float scale_log2;        // |scale| * log2(e)
  float scale;             // raw scale (fp32 path)
  // Split-KV scratch.  Decode: one partial per (slot, row), slot = group +
  // worker.  Prefill: one per (part, tile row), part = (group * n_split +
  // piece) * tiles per group + tile, tile row in [0, 128).
  float* ws_m;             // [slots][rows]  running max, log2 units
  float* ws_l;             // [slots][rows]  sum of 2^(s*c - m)
  float* ws_acc;           // [slots][rows][Dv] unnormalised P.V
  int n_workers;           // workgroups of the split pass (0: no keys at all)
  int rows;                // group * Q
  int n_split;             // prefill: key-range pieces per tile (1: no split)
  int split_blocks;        // prefill: 64-key blocks per piece (piece s starts s * split_blocks into the tile's range)
  int dv_parts;            // prefill, heads over 256: output-channel parts of 256 (1 otherwise)
  int n_xcd;               // XCDs of the device: workgroup i of a launch runs on XCD i % n_xcd
  // Paged K/V cache (block_table null: contiguous k [B,Hkv,K,D], v [B,Hkv,K,Dv]).
  // Otherwise k [num_pages,Hkv,2^page_shift,D], v [num_pages,Hkv,2^page_shift,Dv]
  // and keys [j << page_shift, (j + 1) << page_shift) of sequence b are in page
  // block_table[b * pages_per_seq + j]; K = pages_per_seq << page_shift.
  const int32_t* block_table;
  int pages_per_seq;
  int page_shift;
  int num_pages;
};

// Backward pass (gradients of sum(dO * O) w.r.t. q, k, v).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;           // forward output
  const void* dout;        // dO [B,Hq,Q,Dv]
  const float* lse;        // forward LSE [B,Hq,Q]
  float* delta;            // scratch [B,Hq,Q]: rowsum(dO * O)
  float* lse2;             // scratch [B,Hq,Q]: LSE * log2(e), +inf for rows without a key
  void* dq;                // [B,Hq,Q,D]
  void* dk;                // [B,Hkv,K,D]
  void* dv;                // [B,Hkv,K,Dv]
  const int32_t* seqlens;
  int B, Hq, Hkv, Q, K, D, Dv;
  int window, causal_shift, f16, group, q_sign;
  float scale_log2;        // |scale| * log2(e), kept positive as in the forward
  float scale;             // signed scale: dQ = scale * dS K
  float abs_scale;         // dK = |scale| * dS^T (sign-adjusted q)
};
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);

// Launchers (each returns hipGetLastError() after the launch).
hipError_t launch_prefill_bf16(const Params& p, hipStream_t stream);
hipError_t launch_prefill_combine(const Params& p, hipStream_t stream);   // merge of a split prefill
hipError_t launch_decode_bf16(const Params& p, hipStream_t stream);
hipError_t launch_fwd_f32(const Params& p, hipStream_t stream);

// Smallest page of a paged cache: a 64-key prefill block or an aligned 32-key
// decode sub-block never straddles two pages.
constexpr int kMinPageShift = 6;

// Padded widths the kernels are instantiated for.
inline int pad_width(int d) { return d <= 64 ? 64 : (d <= 128 ? 128 : (d <= 256 ? 256 : 512)); }

// Row q of sequence b sits at absolute position q + row_delta: K_b - Q
// (bottom-right alignment), or, without the causal limit, far enough past
// every key that the causal test k <= position never excludes one.  With the
// shift, positions stay below 2^31 for every size the library accepts
// (Q, K < 2^27).
constexpr int kNonCausalShift = 1 << 30;
__host__ __device__ inline int row_delta(int Kb, int Q, int causal_shift) { return Kb - Q + causal_shift; }

// ---------------------------------------------------------------------------
// Device building blocks
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16-byte stores (non-temporal builtin)
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

#define ATTN_LDS __attribute__((address_space(3)))

__device__ __forceinline__ int clamp_len(const int32_t* seqlens, int b, int K) {
  if (!seqlens) return K;
  int s = seqlens[b];
  return s < 0 ? 0 : (s > K ? K : s);
}

// Page of a paged cache that holds key kb of sequence b (0 for a contiguous
// cache).  A table entry outside [0, num_pages) is a caller error; it is
// clamped so no load leaves the cache.
__device__ __forceinline__ int kv_page(const Params& p, int b, int kb) {
  if (!p.block_table) return 0;
  const int pg = p.block_table[(int64_t)b * p.pages_per_seq + (kb >> p.page_shift)];
  return pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
}

// K and V rows of keys kb, kb + 1, ... of (sequence b, kv-head kh), with `page`
// from kv_page(p, b, kb), and how many rows follow contiguously: to the end
// of the slice, or of the page.
struct KvSpan {
  const uint16_t* k;
  const uint16_t* v;
  int rows;
};
template <bool PAGED>
__device__ __forceinline__ KvSpan kv_span_t(const Params& p, int b, int kh, int kb, int page) {
  const uint16_t* k = static_cast<const uint16_t*>(p.k);
  const uint16_t* v = static_cast<const uint16_t*>(p.v);
  if constexpr (!PAGED) {
    (void)page;
    const int64_t r = ((int64_t)b * p.Hkv + kh) * p.K + kb;
    return KvSpan{k + r * p.D, v + r * p.Dv, p.K - kb};
  } else {
    (void)b;
    const int off = kb & ((1 << p.page_shift) - 1);
    const int64_t r = (((int64_t)page * p.Hkv + kh) << p.page_shift) + off;
    return KvSpan{k + r * p.D, v + r * p.Dv, (1 << p.page_shift) - off};
  }
}
__device__ __forceinline__ KvSpan kv_span(const Params& p, int b, int kh, int kb, int page) {
  return p.block_table ? kv_span_t<true>(p, b, kh, kb, page) : kv_span_t<false>(p, b, kh, kb, page);
}

// v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16]
// (e = 0..7) and receives C[4(l/16)+r][l%16] (r = 0..3).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, output
// lane c element r is element c%4 of the 8 bytes addressed by lane 4r + c/4.
// With lane i of the group addressing row (base + i/4), columns 4(i%4)..+3 of
// a row-major 16-bit tile, lane c receives column c of rows base..base+3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}
// The same at a raw LDS byte address.
__device__ __forceinline__ bf16x4 lds_read_tr16(uint32_t addr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(uintptr_t)(addr));
  return __builtin_bit_cast(bf16x4, r);
}

// 16-byte LDS read at a raw LDS byte address.
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  return *(const ATTN_LDS bf16x8*)(uintptr_t)(addr);
}

// max(a, b) and max(a, b, c) as single v_max_f32 / v_max3_f32.  Written as
// asm because the compiler, to honour IEEE NaN quieting, otherwise
// canonicalises each input (MFMA results, permlane results) with an extra
// v_max first; the inputs here are finite or -inf.
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Butterfly over lanes l, l^16, l^32, l^48 using the gfx950 permlane swaps.
__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float group4_max(float x) { return xor32_max(xor16_max(x)); }
__device__ __forceinline__ float group4_sum(float x) { return xor32_sum(xor16_sum(x)); }

// Reductions over the whole wave (butterfly with DPP-free shuffles).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = max2f(x, __shfl_xor(x, o));
  return group4_max(x);
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o);
  return group4_sum(x);
}


__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online softmax with a lazy reference: a row keeps its reference max m (log2
// units) until a block's max exceeds it by more than kLazyRescale, so the
// weights 2^(s*c - m) stay <= 2^kLazyRescale and the row sum and accumulators
// are rescaled only when some lane of the wave needs it.  The result is the
// same softmax: numerator and denominator share the reference.
constexpr float kLazyRescale = 8.f;

// Updates m_run from the block max mb (log2 units, -inf if the block has no
// legal key for this row).  Returns true (wave-uniform) when the caller must
// multiply its row sum and accumulators by alpha.
__device__ __forceinline__ bool softmax_rebase(float& m_run, float mb, float& alpha) {
  alpha = 1.f;
  if (!__builtin_amdgcn_ballot_w64(mb > m_run + kLazyRescale)) return false;
  const float mnew = fmaxf(m_run, mb);
  alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m_run - mnew);
  m_run = mnew;
  return true;
}

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1, so the body can
// branch on i at compile time.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Pack eight floats into bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16x8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

// The 16-bit element type of the matrix kernels: bf16 (F16 = false) or IEEE
// binary16 (F16 = true).  Fragments travel as bf16x8 bit patterns (loads and
// LDS reads only move bits); the MFMA, the packing of the softmax weights and
// the output conversion are the type's own.
template <bool F16>
struct Elem;
template <>
struct Elem<false> {
  __device__ static f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) { return mfma16x16x32(a, b, c); }
  // v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8(l/32)+e], B[8(l/32)+e][l%32]
  // (e = 0..7) and receives C[8(r/4) + 4(l/32) + r%4][l%32] in register r.
  __device__ static f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static bf16x8 pack(f32x4 lo, f32x4 hi) { return pack_bf16x8(lo, hi); }
  __device__ static uint16_t cvt(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
};
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <>
struct Elem<true> {
  __device__ static f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  }
  __device__ static f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  }
  __device__ static bf16x8 pack(f32x4 lo, f32x4 hi) {
    f16x8 r;
    r[0] = (_Float16)lo[0]; r[1] = (_Float16)lo[1]; r[2] = (_Float16)lo[2]; r[3] = (_Float16)lo[3];
    r[4] = (_Float16)hi[0]; r[5] = (_Float16)hi[1]; r[6] = (_Float16)hi[2]; r[7] = (_Float16)hi[3];
    return __builtin_bit_cast(bf16x8, r);
  }
  __device__ static uint16_t cvt(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
};

__device__ __forceinline__ bf16x8 concat_bf16x4(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ uint4 load_u4(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// ---------------------------------------------------------------------------
// Direct HBM -> LDS tile loads
// ---------------------------------------------------------------------------
// Raw buffer resource over one (batch, head) slice of `bytes` bytes.  Offsets
// at or beyond `bytes` read as zero, which is how key rows past K_b and
// channel chunks past D are zero-filled without branches.  Word 3 selects a
// 32-bit data format, as raw buffer loads on gfx9-class parts require.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;

typedef int rsrc_t __attribute__((ext_vector_type(4)));

// Descriptor words: 48-bit base, stride 0 (raw), num_records = bytes.
__device__ __forceinline__ rsrc_t slice_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return rsrc_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, kRsrcWord3};
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const ATTN_LDS void*)(p);
}

// One wave-wide 16-byte-per-lane load straight into LDS: lane l's 16 bytes
// land at LDS offset lds_wave_base + 16*l (lds_wave_base is wave-uniform).
// Issued as inline asm on purpose: the compiler then inserts no waits of its
// own for these loads (it cannot tell ring stages apart and would wait for
// every load in flight before any LDS read); the kernels wait explicitly with
// wait_vmcnt, counting only these loads, which are the only vector-memory
// operations inside their loops.  m0 is set right before the load; the
// compiler never keeps a value of its own in m0 across code on this target.
__device__ __forceinline__ void load_lds16(rsrc_t rs, uint32_t lds_wave_base, uint32_t voffset) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_wave_base), "v"(voffset), "s"(rs)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// The same load with the non-temporal hint, for data read once (the decode
// pass's K/V stream): it keeps the stream from displacing what the caches
// hold (measured on MI355X: the batched long-context decode streams
// 6.5 TB/s with it, 5.8 without; the prefill, whose tiles share K/V blocks
// through L2, loses 7% with it).
__device__ __forceinline__ void load_lds16_nt(rsrc_t rs, uint32_t lds_wave_base, uint32_t voffset) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(lds_wave_base), "v"(voffset), "s"(rs)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// The 4-byte form: lane l's 4 bytes land at lds_wave_base + 4*l.
__device__ __forceinline__ void load_lds4(rsrc_t rs, uint32_t lds_wave_base, uint32_t voffset) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_wave_base), "v"(voffset), "s"(rs)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// Makes the compiler treat `x` as produced here, after an explicit wait, so it
// inserts no further waits for the load that produced it.
template <typename T>
__device__ __forceinline__ void launder(T& x) {
  asm volatile("" : "+v"(x));
}

// Waits until at most N vector-memory operations of this wave are in flight
// (direct-to-LDS loads count until their data is in LDS).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS tiles of rows of NCH 16-byte chunks are stored XOR-swizzled: chunk c of
// row r sits at chunk position c ^ swz(r).  K tiles use swz(r) = r % min(NCH,
// 16) so the 16 rows of a 16-byte MFMA-fragment read hit distinct banks; V
// tiles use swz(r) = 2r % NCH so the 4-row, 32-byte pieces of a transposed
// read do.
template <int NCH>
__device__ __forceinline__ int swz_k(int row) { return row & ((NCH < 16 ? NCH : 16) - 1); }
template <int NCH>
__device__ __forceinline__ int swz_v(int row) { return (2 * row) & (NCH - 1); }

}  // namespace attn
