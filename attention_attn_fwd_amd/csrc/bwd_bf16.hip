// Backward pass on gfx950: the gradients of sum(dO * O) with respect to q, k
// and v for the same causal / windowed / variable-length GQA attention as the
// forward (LuisaCompute "Attention execution mapping" review, section 1; the
// FlyDSL post, "FMHA through AOTriton", describes the backward as separate dQ
// and dK/dV kernels built from the forward's pieces, the dK/dV loop being the
// forward loop transposed: K and V held in registers, Q and dO streamed).
//
// Per row, with the forward's LSE: P = exp(S - LSE), dP = dO V^T,
// delta = rowsum(dO * O) (= sum_k P dP), dS = P (dP - delta); then
// dV = P^T dO, dK = scale dS^T q, dQ = scale dS K.  A kv-head's dK and dV sum
// over its query heads.  Two passes, no atomics (bitwise reproducible):
//   * bwd_dq_kernel: one workgroup per 128 query rows of one head, 8 waves of
//     16 rows, streaming 64-key K and V blocks through a two-stage LDS ring
//     by direct loads.  Per block: S^T = K q^T and dP^T = V dO^T with q and dO
//     in registers (the forward's layout: a lane holds 4 keys of one row),
//     dS^T in registers, then dQ^T += K^T dS^T with K^T read transposed
//     (ds_read_b64_tr_b16) in the key order of the dS^T registers.  It also
//     forms each row's delta (from the O and dO rows it loads) and LSE in
//     log2 units (+inf for a row with no legal key, so its weights are 0),
//     and stores both for the second pass;
//   * bwd_dkdv_kernel: one workgroup per 128 keys of one kv-head, 8 waves of
//     16 keys, K and V in registers, streaming 64-row blocks of q and dO (and
//     the rows' LSE and delta) of every query head of the group.  Per block:
//     S = q K^T, dP = dO V^T (a lane holds 4 rows of one key), P and dS, then
//     dV^T += dO^T P and dK^T += q^T dS with q and dO read transposed.
// Masks are the forward's: initial accumulators 0 / -inf on blocks that
// straddle the diagonal, a window edge or K_b; blocks a wave cannot see are
// skipped by that wave.  The weights and dS are rounded to the storage type
// for the products (as P is in the forward); accumulators are fp32.
#include <type_traits>

#include "attn_internal.h"

namespace attn {

constexpr int kBwdRows = 128;  // rows (dQ) or keys (dK/dV) per workgroup
constexpr int kBwdBlock = 64;  // streamed keys (dQ) or rows (dK/dV) per block
constexpr int kBwdWaves = 8;

template <int DP, int DVP, int NW = kBwdWaves>
struct BwdShape {
  static constexpr int KS = DP / 32;    // k-steps over the q/k channels
  static constexpr int KSV = DVP / 32;  // k-steps over the v channels
  static constexpr int KA = KS < 4 ? KS : 4;
  static constexpr int KB = KSV < 4 ? KSV : 4;
  static constexpr int JD = DP / 16;    // 16-wide channel tiles of dQ^T / dK^T
  static constexpr int JV = DVP / 16;   // of dV^T
  static constexpr int ACH = DP / 8;    // 16-byte chunks per row of the A tile (width DP)
  static constexpr int BCH = DVP / 8;   // of the B tile (width DVP)
  static constexpr int AROWB = DP * 2;
  static constexpr int BROWB = DVP * 2;
  static constexpr int A_TILE = kBwdBlock * AROWB;
  static constexpr int B_TILE = kBwdBlock * BROWB;
  static constexpr int B_BASE = 2 * A_TILE;
  static constexpr int X_BASE = 2 * A_TILE + 2 * B_TILE;  // per-row LSE and delta of the dK/dV stream
  static constexpr int X_STAGE = 2 * kBwdBlock * 4;
  static constexpr int LDS = X_BASE + 2 * X_STAGE;
  static constexpr int ROUND = NW * 1024;  // bytes one wave-wide 16-byte load round of the workgroup covers
  static constexpr int A_LOADS = A_TILE / ROUND;
  static constexpr int B_LOADS = B_TILE / ROUND;
  static constexpr int A_ROWS_PER_LOAD = ROUND / AROWB;
  static constexpr int B_ROWS_PER_LOAD = ROUND / BROWB;
  static_assert(A_TILE % ROUND == 0 && B_TILE % ROUND == 0, "load split");
  static_assert(A_ROWS_PER_LOAD % (ACH < 16 ? ACH : 16) == 0 && B_ROWS_PER_LOAD % (BCH < 16 ? BCH : 16) == 0,
                "a load round covers whole swizzle periods");
  static_assert(A_TILE + 48 * AROWB + 1024 < 65536 && B_TILE + 48 * BROWB + 1024 < 65536, "ds_read immediates");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Direct loads of two row tiles (A: width DP, B: width DVP) of kBwdBlock rows
// into a two-stage ring, and the per-lane LDS addresses of their 16-byte
// fragment reads and transposed reads.  Rows hold 16-byte chunks XOR-swizzled
// with swz_k; the chunk index of k-step s is 4s + g4, whose bits above the
// fourth are untouched by the swizzle, so k-step s reads at frag[s % 4] +
// 256 * (s / 4).  A load round of the workgroup (8 KiB) covers whole swizzle
// periods, so each lane fetches the same chunk of every round.
template <int DP, int DVP, bool EXACT, int NW = kBwdWaves>
struct BwdTiles {
  using S = BwdShape<DP, DVP, NW>;
  uint32_t lds0, aoff, boff, astep, bstep, abase_w, bbase_w;
  uint32_t afrag[S::KA], bfrag[S::KB];
  uint32_t atr[S::JD], btr[S::JV];

  __device__ __forceinline__ void init(uint32_t lds, int wave, int lane, int D, int Dv) {
    lds0 = lds;
    const int l16 = lane & 15, g4 = lane >> 4;
    auto lane_off = [&](int rowb, int nch, int width) -> uint32_t {
      const int off = wave * 1024 + 16 * lane;
      const int row = off / rowb, pos = (off % rowb) >> 4;
      const int ch = pos ^ (row & ((nch < 16 ? nch : 16) - 1));
      if (EXACT) return (uint32_t)(row * width + ch * 8) * 2;
      return ch < width / 8 ? (uint32_t)(row * width + ch * 8) * 2 : kOutOfRange;
    };
    aoff = lane_off(S::AROWB, S::ACH, D);
    boff = lane_off(S::BROWB, S::BCH, Dv);
    astep = (uint32_t)(S::A_ROWS_PER_LOAD * D * 2);
    bstep = (uint32_t)(S::B_ROWS_PER_LOAD * Dv * 2);
    abase_w = lds0 + wave * 1024;
    bbase_w = lds0 + S::B_BASE + wave * 1024;
#pragma unroll
    for (int s = 0; s < S::KA; ++s) afrag[s] = lds0 + l16 * S::AROWB + (((4 * s + g4) ^ swz_k<S::ACH>(l16)) << 4);
#pragma unroll
    for (int s = 0; s < S::KB; ++s)
      bfrag[s] = lds0 + S::B_BASE + l16 * S::BROWB + (((4 * s + g4) ^ swz_k<S::BCH>(l16)) << 4);
    const int vrow = 4 * g4 + (l16 >> 2);
#pragma unroll
    for (int j = 0; j < S::JD; ++j)
      atr[j] = lds0 + vrow * S::AROWB + (((2 * j + ((l16 & 3) >> 1)) ^ swz_k<S::ACH>(vrow)) << 4) + (l16 & 1) * 8;
#pragma unroll
    for (int j = 0; j < S::JV; ++j)
      btr[j] = lds0 + S::B_BASE + vrow * S::BROWB + (((2 * j + ((l16 & 3) >> 1)) ^ swz_k<S::BCH>(vrow)) << 4) +
               (l16 & 1) * 8;
  }
  // Rows [0, rows) of A (row stride D elements) and B (row stride Dv) into stage stg.
  __device__ __forceinline__ void issue(const void* a, const void* b, uint32_t rows, int D, int Dv, int stg) const {
    const rsrc_t ra = slice_rsrc(a, rows * D * 2);
    const rsrc_t rb = slice_rsrc(b, rows * Dv * 2);
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i) load_lds16(ra, abase_w + stg * S::A_TILE + i * S::ROUND, aoff + i * astep);
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i) load_lds16(rb, bbase_w + stg * S::B_TILE + i * S::ROUND, boff + i * bstep);
  }
  // 16-byte fragments: rows 16i + l16, channels 32s + 8*g4 .. + 7.
  template <int STG>
  __device__ __forceinline__ bf16x8 a_frag(int i, int s) const {
    return lds_read_b128(afrag[s % 4] + STG * S::A_TILE + 16 * i * S::AROWB + 256 * (s / 4));
  }
  template <int STG>
  __device__ __forceinline__ bf16x8 b_frag(int i, int s) const {
    return lds_read_b128(bfrag[s % 4] + STG * S::B_TILE + 16 * i * S::BROWB + 256 * (s / 4));
  }
  // Transposed fragments of channel tile j over rows 32kk + 4*g4 + e (e < 4)
  // and 32kk + 16 + 4*g4 + e - 4 (the register order of a 16x16 result).
  template <int STG>
  __device__ __forceinline__ bf16x8 a_tr(int kk, int j) const {
    const uint32_t lo = atr[j] + STG * S::A_TILE + 32 * kk * S::AROWB;
    return concat_bf16x4(lds_read_tr16(lo), lds_read_tr16(lo + 16 * S::AROWB));
  }
  template <int STG>
  __device__ __forceinline__ bf16x8 b_tr(int kk, int j) const {
    const uint32_t lo = btr[j] + STG * S::B_TILE + 32 * kk * S::BROWB;
    return concat_bf16x4(lds_read_tr16(lo), lds_read_tr16(lo + 16 * S::BROWB));
  }
};

__device__ __forceinline__ bf16x8 neg_bf16x8(bf16x8 x, uint32_t sign) {
  uint4 u = __builtin_bit_cast(uint4, x);
  u.x ^= sign; u.y ^= sign; u.z ^= sign; u.w ^= sign;
  return __builtin_bit_cast(bf16x8, u);
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 128 query rows of head h of sequence b; wave w owns rows
// 16w .. 16w + 15 (lane column l16).
// ---------------------------------------------------------------------------
// Heads of exactly 64 or 128 channels: two workgroups per CU (4 waves per
// SIMD, at most 128 VGPRs), 8% faster than one on the dense prefill shape's
// backward.  Padded widths (their channel bounds take registers) and wider
// heads (q, dO fragments and accumulators): one, without spills.
template <int DP, int DVP, bool EXACT, bool F16>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(EXACT && DP <= 128 && DVP <= 128 ? 4 : 2,
                                                                      EXACT && DP <= 128 && DVP <= 128 ? 4 : 2))) void
bwd_dq_kernel(BwdParams p) {
  using S = BwdShape<DP, DVP>;
  using E = Elem<F16>;
  constexpr int BN = kBwdBlock;
  const int D = EXACT ? DP : p.D;
  const int Dv = EXACT ? DVP : p.Dv;
  __shared__ __attribute__((aligned(16))) unsigned char ring[S::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  // Tile order: heaviest causal tile first, heads fastest.
  const int n_qt = (p.Q + kBwdRows - 1) / kBwdRows;
  const int x = blockIdx.x;
  const int h = x % p.Hq;
  const int rest = x / p.Hq;
  const int b = rest % p.B;
  const int qt = n_qt - 1 - rest / p.B;
  const int kh = h / p.group;

  const int Kb = clamp_len(p.seqlens, b, p.K);
  const int delta = row_delta(Kb, p.Q, p.causal_shift);
  const int W = p.window;
  const int q0 = qt * kBwdRows;
  const int q_last = min(q0 + kBwdRows, p.Q) - 1;
  const int kv_hi = min(Kb, q_last + delta + 1);
  const int kv_lo = W > 0 ? max(0, q0 + delta - W + 1) : 0;
  const int jb0 = kv_lo / BN;
  const int jb1 = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : jb0;

  const int qw0 = q0 + wave * 16;
  const bool wave_has_rows = qw0 < p.Q;
  const int qw_last = min(qw0 + 16, p.Q) - 1;
  const int pw_first = qw0 + delta, pw_last = qw_last + delta;
  const int row = qw0 + l16;
  const bool row_ok = row < p.Q;
  const int64_t rowi = ((int64_t)b * p.Hq + h) * p.Q + row;
  const float c = p.scale_log2;
  const uint32_t qx = p.q_sign ? 0x80008000u : 0u;

  // q (sign-adjusted) and dO fragments: B operands of S^T = K q^T and dP^T = V dO^T.
  // The row's O chunks at the dO chunks' channels give delta = rowsum(dO * O).
  bf16x8 qf[S::KS], gf[S::KSV];
  float dlt = 0.f;
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + rowi * D;
    const uint16_t* grow = static_cast<const uint16_t*>(p.dout) + rowi * Dv;
    const uint16_t* orow = static_cast<const uint16_t*>(p.o) + rowi * Dv;
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
      const int col = 32 * s + 8 * g4;
      qf[s] = neg_bf16x8(__builtin_bit_cast(bf16x8, (row_ok && col < D) ? load_u4(qrow + col) : zero_u4()), qx);
    }
    auto widen = [](uint32_t h) -> float {
      if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
      else return __builtin_bit_cast(float, h << 16);
    };
#pragma unroll
    for (int s = 0; s < S::KSV; ++s) {
      const int col = 32 * s + 8 * g4;
      const bool in = row_ok && col < Dv;
      const uint4 gu = in ? load_u4(grow + col) : zero_u4();
      const uint4 ou = in ? load_u4(orow + col) : zero_u4();
      gf[s] = __builtin_bit_cast(bf16x8, gu);
      const uint32_t ga[4] = {gu.x, gu.y, gu.z, gu.w}, oa[4] = {ou.x, ou.y, ou.z, ou.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dlt = fmaf(widen(ga[e] & 0xFFFFu), widen(oa[e] & 0xFFFFu), dlt);
        dlt = fmaf(widen(ga[e] >> 16), widen(oa[e] >> 16), dlt);
      }
    }
  }
  const float lse_in = row_ok ? p.lse[rowi] : -INFINITY;
  wait_vmcnt<0>();
  dlt = group4_sum(dlt);
  const float lse2 = lse_in == -INFINITY ? INFINITY : lse_in * 1.44269504088896340736f;
  if (row_ok && g4 == 0) {  // for the dK/dV pass
    p.delta[rowi] = dlt;
    p.lse2[rowi] = lse2;
  }
#pragma unroll
  for (int s = 0; s < S::KS; ++s) launder(qf[s]);
#pragma unroll
  for (int s = 0; s < S::KSV; ++s) launder(gf[s]);
  float lse2v = lse2, dltv = dlt;
  launder(lse2v);
  launder(dltv);

  BwdTiles<DP, DVP, EXACT> tl;
  tl.init(lds_offset(ring), wave, lane, D, Dv);
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.Hkv + kh) * p.K * D;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.Hkv + kh) * p.K * Dv;
  auto issue = [&](int jb, int stg) {
    const int kb0 = jb * BN;
    tl.issue(kg + (int64_t)kb0 * D, vg + (int64_t)kb0 * Dv, (uint32_t)min(Kb - kb0, BN), D, Dv, stg);
  };

  auto wave_sees = [&](int jb) {
    const int kb0 = jb * BN;
    return wave_has_rows && kb0 <= pw_last && kb0 < Kb && !(W > 0 && kb0 + BN - 1 < pw_first - W + 1);
  };
  auto wave_full = [&](int jb) {
    const int kb0 = jb * BN;
    return (kb0 + BN - 1 <= pw_first) && (kb0 + BN <= Kb) && (W <= 0 || kb0 >= pw_last - W + 1);
  };

  f32x4 acc[S::JD];
#pragma unroll
  for (int j = 0; j < S::JD; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto body = [&](int jb, auto stg_tag, bool full) {
    constexpr int STG = decltype(stg_tag)::value;
    const int kb0 = jb * BN;
    f32x4 s[4], dp[4];
    if (full) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      // Key kb0 + 16i + 4*g4 + r of row `row` (position row + delta).
      const int rel = row + delta - kb0 - 4 * g4;
      const int hi = min(rel, Kb - kb0 - 4 * g4 - 1);
      const int lo = W > 0 ? max(rel - W + 1, 0) : 0;
      const uint32_t span = (uint32_t)(hi - lo);
      const bool none = hi < lo;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s[i][r] = (!none & ((uint32_t)(16 * i + r - lo) <= span)) ? 0.f : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < S::KS; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = E::mfma(tl.template a_frag<STG>(i, st), qf[st], s[i]);
#pragma unroll
    for (int st = 0; st < S::KSV; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[i] = E::mfma(tl.template b_frag<STG>(i, st), gf[st], dp[i]);
    // dS^T = P^T (dP^T - delta), P^T = 2^(s c - lse2).
    f32x4 ds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pw = fast_exp2(fmaf(s[i][r], c, -lse2v));
        ds[i][r] = pw * (dp[i][r] - dltv);
      }
    const bf16x8 dsp0 = E::pack(ds[0], ds[1]);
    const bf16x8 dsp1 = E::pack(ds[2], ds[3]);
    // dQ^T += K^T dS^T over the block's two 32-key halves.
#pragma unroll
    for (int j = 0; j < S::JD; ++j) {
      acc[j] = E::mfma(tl.template a_tr<STG>(0, j), dsp0, acc[j]);
      acc[j] = E::mfma(tl.template a_tr<STG>(1, j), dsp1, acc[j]);
    }
  };

  auto block = [&](int jb, auto stg_tag) {
    if (jb + 1 < jb1) issue(jb + 1, decltype(stg_tag)::value ^ 1);
    if (wave_sees(jb)) body(jb, stg_tag, wave_full(jb));
    wait_vmcnt<0>();
    __syncthreads();
  };
  if (jb0 < jb1) {
    issue(jb0, 0);
    wait_vmcnt<0>();
    __syncthreads();
  }
  for (int jb = jb0; jb < jb1; jb += 2) {
    block(jb, std::integral_constant<int, 0>{});
    if (jb + 1 < jb1) block(jb + 1, std::integral_constant<int, 1>{});
  }

  if (!row_ok) return;
  uint16_t* out = static_cast<uint16_t*>(p.dq) + rowi * D;
#pragma unroll
  for (int j = 0; j < S::JD; ++j) {
    const int d = 16 * j + 4 * g4;
    if (d < D) {
      ushort4 v4;
      v4.x = E::cvt(acc[j][0] * p.scale);
      v4.y = E::cvt(acc[j][1] * p.scale);
      v4.z = E::cvt(acc[j][2] * p.scale);
      v4.w = E::cvt(acc[j][3] * p.scale);
      *reinterpret_cast<ushort4*>(out + d) = v4;
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 128 keys of kv-head kh of sequence b; wave w owns keys
// 16w .. 16w + 15 (lane column l16).  Streams 64-row blocks of q and dO of
// the group's query heads, with the rows' lse2 and delta.
// ---------------------------------------------------------------------------
// DK / DV select the outputs: both for heads up to 128; for wider heads one
// launch each (dV needs only S and P; dK needs S, dP and dS), so a wave holds
// one accumulator set.  NW waves of 16 keys: heads up to 128 take 4 (tiles of
// 64 keys, two workgroups per CU, so the two waves on a SIMD come from
// different workgroups and do not meet at the same barriers; 1-2% faster
// than one 8-wave workgroup per CU on the dense and the windowed varlen
// prefill shapes), wider heads 8 (one workgroup per CU).
template <int DP, int DVP, bool EXACT, bool F16, bool DK, bool DV, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void bwd_dkdv_kernel(BwdParams p) {
  static_assert(DK || DV, "an output");
  using S = BwdShape<DP, DVP, NW>;
  constexpr int KEYS = 16 * NW;  // keys per workgroup
  using E = Elem<F16>;
  constexpr int BR = kBwdBlock;
  const int D = EXACT ? DP : p.D;
  const int Dv = EXACT ? DVP : p.Dv;
  __shared__ __attribute__((aligned(16))) unsigned char ring[S::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  // Tile order: key tiles from the start of the sequence (they see the most
  // rows under the causal limit), kv-heads fastest.
  const int n_kt = (p.K + KEYS - 1) / KEYS;
  const int x = blockIdx.x;
  const int kh = x % p.Hkv;
  const int rest = x / p.Hkv;
  const int b = rest % p.B;
  const int kt = rest / p.B;
  (void)n_kt;

  const int Kb = clamp_len(p.seqlens, b, p.K);
  const int delta = row_delta(Kb, p.Q, p.causal_shift);
  const int W = p.window;
  const int k0 = kt * KEYS;
  const int kw0 = k0 + wave * 16;
  const int key = kw0 + l16;
  const bool key_ok = key < Kb;
  const int64_t keyi = ((int64_t)b * p.Hkv + kh) * p.K + key;

  // K and V fragments: B operands of S = q K^T and dP = dO V^T.
  bf16x8 kf[S::KS], vf[S::KSV];
  {
    const uint16_t* krow = static_cast<const uint16_t*>(p.k) + keyi * D;
    const uint16_t* vrow = static_cast<const uint16_t*>(p.v) + keyi * Dv;
    // The scale's sign goes on K here (S = (sign q) K^T = q (sign K)^T), so the
    // streamed q fragments are used as they are.
    const uint32_t kx = p.q_sign ? 0x80008000u : 0u;
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
      const int col = 32 * s + 8 * g4;
      kf[s] = neg_bf16x8(__builtin_bit_cast(bf16x8, (key_ok && col < D) ? load_u4(krow + col) : zero_u4()), kx);
    }
#pragma unroll
    for (int s = 0; s < S::KSV; ++s) {
      const int col = 32 * s + 8 * g4;
      vf[s] = (DK && key_ok && col < Dv) ? __builtin_bit_cast(bf16x8, load_u4(vrow + col))
                                         : __builtin_bit_cast(bf16x8, zero_u4());
    }
  }
  wait_vmcnt<0>();
#pragma unroll
  for (int s = 0; s < S::KS; ++s) launder(kf[s]);
  if constexpr (DK) {
#pragma unroll
    for (int s = 0; s < S::KSV; ++s) launder(vf[s]);
  }

  // Rows that can see a key of this workgroup: position q + delta >= k0
  // (causal) and q + delta < k0 + KEYS - 1 + W (window).
  int q_lo = 0, q_hi = 0;
  if (k0 < Kb) {
    q_lo = max(0, k0 - delta);
    q_hi = p.Q;
    if (W > 0) q_hi = (int)min((int64_t)p.Q, (int64_t)k0 + KEYS - 1 + W - delta);
  }
  const int rb0 = q_lo / BR;
  const int rb1 = q_hi > q_lo ? (q_hi + BR - 1) / BR : rb0;
  const int nrb = rb1 - rb0;
  const int steps = nrb * p.group;  // (head, row block) pairs, head-major

  BwdTiles<DP, DVP, EXACT, NW> tl;
  tl.init(lds_offset(ring), wave, lane, D, Dv);
  const uint32_t xbase = lds_offset(ring) + S::X_BASE;
  auto issue = [&](int step, int stg) {
    const int hh = step / nrb, rb = rb0 + step % nrb;
    const int h = kh * p.group + hh;
    const int r0 = rb * BR;
    const int64_t ri = ((int64_t)b * p.Hq + h) * p.Q + r0;
    const uint32_t rows = (uint32_t)min(p.Q - r0, BR);
    tl.issue(static_cast<const uint16_t*>(p.q) + ri * D, static_cast<const uint16_t*>(p.dout) + ri * Dv, rows, D,
             Dv, stg);
    if (wave == 0) {  // lse2 and delta of the 64 rows: one 4-byte load per lane each
      load_lds4(slice_rsrc(p.lse2 + ri, rows * 4), xbase + stg * S::X_STAGE, 4 * lane);
      load_lds4(slice_rsrc(p.delta + ri, rows * 4), xbase + stg * S::X_STAGE + BR * 4, 4 * lane);
    }
  };

  // Wave-level view of step `step`: rows [r0, r0 + 64) against keys
  // [kw0, kw0 + 16).
  auto step_rows = [&](int step) { return (rb0 + step % nrb) * BR; };
  auto wave_sees = [&](int r0) {
    const int r_last = min(r0 + BR, p.Q) - 1;
    return kw0 < Kb && kw0 <= r_last + delta && !(W > 0 && kw0 + 15 <= r0 + delta - W);
  };
  auto wave_full = [&](int r0) {
    return kw0 + 15 < Kb && kw0 + 15 <= r0 + delta && (W <= 0 || kw0 > r0 + BR - 1 + delta - W);
  };

  f32x4 acck[S::JD], accv[S::JV];
#pragma unroll
  for (int j = 0; j < S::JD; ++j) acck[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < S::JV; ++j) accv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c = p.scale_log2;

  auto body = [&](int r0, auto stg_tag, bool full) {
    constexpr int STG = decltype(stg_tag)::value;
    f32x4 s[4], dp[4];
    if (full) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      // Row r0 + 16i + 4*g4 + r at position (that) + delta against key `key`:
      // legal iff 0 <= t < W (or t >= 0 without a window), t = position - key.
      const int t0 = r0 + 4 * g4 + delta - key;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 16 * i + r;
          s[i][r] = (key_ok && t >= 0 && (W <= 0 || t < W)) ? 0.f : -INFINITY;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < S::KS; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = E::mfma(tl.template a_frag<STG>(i, st), kf[st], s[i]);
    if constexpr (DK) {
#pragma unroll
      for (int st = 0; st < S::KSV; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) dp[i] = E::mfma(tl.template b_frag<STG>(i, st), vf[st], dp[i]);
    }
    // Rows 16i + 4*g4 + r: their lse2 and delta from LDS.
    f32x4 pw[4], ds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t xa = xbase + STG * S::X_STAGE + (16 * i + 4 * g4) * 4;
      const f32x4 l2 = __builtin_bit_cast(f32x4, lds_read_b128(xa));
#pragma unroll
      for (int r = 0; r < 4; ++r) pw[i][r] = fast_exp2(fmaf(s[i][r], c, -l2[r]));
      if constexpr (DK) {
        const f32x4 dl = __builtin_bit_cast(f32x4, lds_read_b128(xa + BR * 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[i][r] = pw[i][r] * (dp[i][r] - dl[r]);
      }
    }
    // dV^T += dO^T P and dK^T += q^T dS over the block's two 32-row halves.
    if constexpr (DV) {
      const bf16x8 pp0 = E::pack(pw[0], pw[1]), pp1 = E::pack(pw[2], pw[3]);
#pragma unroll
      for (int j = 0; j < S::JV; ++j) {
        accv[j] = E::mfma(tl.template b_tr<STG>(0, j), pp0, accv[j]);
        accv[j] = E::mfma(tl.template b_tr<STG>(1, j), pp1, accv[j]);
      }
    }
    if constexpr (DK) {
      const bf16x8 dsp0 = E::pack(ds[0], ds[1]), dsp1 = E::pack(ds[2], ds[3]);
#pragma unroll
      for (int j = 0; j < S::JD; ++j) {
        acck[j] = E::mfma(tl.template a_tr<STG>(0, j), dsp0, acck[j]);
        acck[j] = E::mfma(tl.template a_tr<STG>(1, j), dsp1, acck[j]);
      }
    }
  };

  auto block = [&](int step, auto stg_tag) {
    if (step + 1 < steps) issue(step + 1, decltype(stg_tag)::value ^ 1);
    const int r0 = step_rows(step);
    if (wave_sees(r0)) body(r0, stg_tag, wave_full(r0));
    wait_vmcnt<0>();
    __syncthreads();
  };
  if (steps > 0) {
    issue(0, 0);
    wait_vmcnt<0>();
    __syncthreads();
  }
  for (int step = 0; step < steps; step += 2) {
    block(step, std::integral_constant<int, 0>{});
    if (step + 1 < steps) block(step + 1, std::integral_constant<int, 1>{});
  }

  // Keys past K_b (and whole tiles past it) get zero gradients.
  if (key >= p.K) return;
  uint16_t* ko = static_cast<uint16_t*>(p.dk) + keyi * D;
  uint16_t* vo = static_cast<uint16_t*>(p.dv) + keyi * Dv;
#pragma unroll
  for (int j = 0; j < (DK ? S::JD : 0); ++j) {
    const int d = 16 * j + 4 * g4;
    if (d < D) {
      ushort4 v4;
      v4.x = E::cvt(acck[j][0] * p.scale);
      v4.y = E::cvt(acck[j][1] * p.scale);
      v4.z = E::cvt(acck[j][2] * p.scale);
      v4.w = E::cvt(acck[j][3] * p.scale);
      *reinterpret_cast<ushort4*>(ko + d) = v4;
    }
  }
#pragma unroll
  for (int j = 0; j < (DV ? S::JV : 0); ++j) {
    const int d = 16 * j + 4 * g4;
    if (d < Dv) {
      ushort4 v4;
      v4.x = E::cvt(accv[j][0]);
      v4.y = E::cvt(accv[j][1]);
      v4.z = E::cvt(accv[j][2]);
      v4.w = E::cvt(accv[j][3]);
      *reinterpret_cast<ushort4*>(vo + d) = v4;
    }
  }
}

template <int DP, int DVP>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  BwdParams arg = p;
  void* args[] = {&arg};
  const int64_t rows = (int64_t)p.B * p.Hq * p.Q;
  hipError_t e = hipSuccess;
  const bool exact = p.D == DP && p.Dv == DVP;
  const int sel = (exact ? 1 : 0) | (p.f16 ? 2 : 0);
  const void* const dq[4] = {
      reinterpret_cast<const void*>(&bwd_dq_kernel<DP, DVP, false, false>),
      reinterpret_cast<const void*>(&bwd_dq_kernel<DP, DVP, true, false>),
      reinterpret_cast<const void*>(&bwd_dq_kernel<DP, DVP, false, true>),
      reinterpret_cast<const void*>(&bwd_dq_kernel<DP, DVP, true, true>),
  };
  if (rows > 0) {
    const int64_t n_qt = (p.Q + kBwdRows - 1) / kBwdRows;
    e = hipLaunchKernel(dq[sel], dim3((unsigned)(n_qt * p.Hq * p.B)), dim3(64 * kBwdWaves), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  constexpr bool kSplit = DP > 128 || DVP > 128;  // dK and dV in separate launches
  constexpr int NW = kSplit ? kBwdWaves : 4;       // waves (of 16 keys) per dK/dV workgroup
  const int64_t n_kt = (p.K + 16 * NW - 1) / (16 * NW);
  if (n_kt == 0 || p.B == 0 || p.Hkv == 0) return hipSuccess;
  const dim3 kgrid((unsigned)(n_kt * p.Hkv * p.B));
  if constexpr (!kSplit) {
    const void* const both[4] = {
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, false, false, true, true, NW>),
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, true, false, true, true, NW>),
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, false, true, true, true, NW>),
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, true, true, true, true, NW>),
    };
    return hipLaunchKernel(both[sel], kgrid, dim3(64 * NW), args, 0, stream);
  } else {
    const void* const dk[4] = {
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, false, false, true, false, NW>),
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, true, false, true, false, NW>),
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, false, true, true, false, NW>),
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, true, true, true, false, NW>),
    };
    const void* const dv[4] = {
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, false, false, false, true, NW>),
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, true, false, false, true, NW>),
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, false, true, false, true, NW>),
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<DP, DVP, true, true, false, true, NW>),
    };
    e = hipLaunchKernel(dk[sel], kgrid, dim3(64 * NW), args, 0, stream);
    if (e != hipSuccess) return e;
    return hipLaunchKernel(dv[sel], kgrid, dim3(64 * NW), args, 0, stream);
  }
}

// Heads up to 128 wide on kernels sized for them; wider (up to 256) padded to
// 256 on both sides.
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  const int dp = pad_width(p.D), dvp = pad_width(p.Dv);
  if (dp > 128 || dvp > 128) return launch_bwd_t<256, 256>(p, stream);
  if (dp == 64 && dvp == 64) return launch_bwd_t<64, 64>(p, stream);
  if (dp == 64 && dvp == 128) return launch_bwd_t<64, 128>(p, stream);
  if (dp == 128 && dvp == 64) return launch_bwd_t<128, 64>(p, stream);
  return launch_bwd_t<128, 128>(p, stream);
}

}  // namespace attn
