// bf16 prefill kernel for gfx950: causal GQA attention forward with online
// softmax (LuisaCompute "Attention execution mapping" review, section 1: the
// fixture's bottom-right causal GQA and the (row_max, row_sum, acc) state
// carried across KV blocks; section 2: the phase graph load Q -> per KV block
// load K/V -> QK -> mask -> max/exp/sum -> rescale -> PV -> update).
//
// Mapping on CDNA4:
//   * one workgroup = 4 waves = a tile of 128 query rows of one (batch,
//     kv-head) group: rows of one query head, or, when a head has fewer than
//     128 rows, the rows of several heads of the group (they read the same
//     K/V, section 5 of the review); each wave owns 32 rows as two 16-column
//     MFMA tiles, Q held in registers; two workgroups share a CU, so each
//     SIMD runs one wave of each and the softmax of one overlaps the matrix
//     products of the other;
//   * when the tiles are too few to fill the GPU (few long sequences), each
//     tile's key range is cut into pieces run by separate workgroups, which
//     write their (row_max, row_sum, acc) state in fp32; a combine pass merges
//     the pieces of a row in order (the legal merge of section 5);
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16, so each lane holds 16 keys of
//     one query column and the row max/sum is in-lane plus two permlane swaps;
//     P^T stays in that register layout and feeds O^T = V^T P^T directly, V^T
//     fragments read from row-major LDS through ds_read_b64_tr_b16;
//   * K/V blocks of 64 keys go HBM -> LDS by direct buffer loads into a
//     two-stage ring: block j+1 is in flight while block j is computed, one
//     barrier per block; rows past K_b and channels past D read as zero from
//     the buffer range check;
//   * tiles are XOR-swizzled in LDS so the 16-byte K fragment reads and the
//     transposed V reads are free of bank conflicts; the swizzle of a lane's
//     fragment does not depend on the key tile, so every LDS address is one of
//     a few per-lane registers plus an immediate (the loop is unrolled over
//     the two ring stages so the stage offset is an immediate too);
//   * the VALU work per block is kept to the softmax itself: wave-level
//     control is scalar; masks are evaluated only on blocks that straddle the
//     causal diagonal, a window edge or the sequence end, as the initial S^T
//     accumulator (0 for a legal key, -inf otherwise); blocks no row of a wave
//     can see are skipped by that wave; and the running max is lazy: weights
//     are formed against the current reference and the block max is computed
//     only when a partial row sum shows a weight may exceed 2^kLazyRescale;
//   * tiles are ordered heaviest causal tile first within a (batch, kv-head)
//     group, and the groups are dealt to the 8 XCDs so an XCD streams one
//     group's K/V through its L2 at a time.
#include <type_traits>

#include "attn_internal.h"
#include "prefill_common.h"

namespace attn {

// Padded widths DP, DVP; NW waves per workgroup, each owning NT 16-row MFMA
// tiles of the 128-row tile (NW * NT * 16 = 128).  Heads up to 128 wide use
// 4 waves of 32 rows, two workgroups per CU; wider heads use 8 waves of 16
// rows (half the per-wave registers: the Q fragments and accumulators of a
// 256-wide head), one workgroup per CU, so the two waves on a SIMD still
// overlap one's softmax with the other's products.
// LDS ring: K of stage 0, K of stage 1, V of stage 0, V of stage 1, so every
// read offset that depends on the stage or the key tile fits the 16-bit
// immediate of a ds_read.
template <int DP, int DVP, int NW, int BN_ = kPrefillBN>
struct PrefillShape {
  static constexpr int BN = BN_;            // keys per block
  static constexpr int KT = BN / 16;        // 16-key MFMA tiles per block
  static constexpr int NT = kPrefillBM / (16 * NW);  // 16-row MFMA tiles per wave
  static constexpr int KS = DP / 32;        // 32-deep k-steps of Q.K
  static constexpr int JV = DVP / 16;       // 16-wide dv tiles of O^T
  static constexpr int KCH = DP / 8;        // 16-byte chunks per K row
  static constexpr int VCH = DVP / 8;
  static constexpr int KROWB = DP * 2;      // LDS bytes per K row
  static constexpr int VROWB = DVP * 2;
  static constexpr int K_TILE = BN * KROWB;
  static constexpr int V_TILE = BN * VROWB;
  static constexpr int V_BASE = 2 * K_TILE;
  static constexpr int LDS = 2 * (K_TILE + V_TILE);
  static constexpr int ROUND = NW * 1024;   // bytes one wave-wide 16-byte load round of the workgroup covers
  static constexpr int K_LOADS = K_TILE / ROUND;  // 16-byte loads per thread per block
  static constexpr int V_LOADS = V_TILE / ROUND;
  static constexpr int K_ROWS_PER_LOAD = ROUND / KROWB;  // tile rows one load round covers
  static constexpr int V_ROWS_PER_LOAD = ROUND / VROWB;
  static_assert(NT * 16 * NW == kPrefillBM && (NT == 1 || NT == 2), "tile geometry");
  static_assert((BN == 32 || BN == 64) && kPrefillBN % BN == 0, "block size");
  static_assert(K_TILE % ROUND == 0 && V_TILE % ROUND == 0, "load split");
  // Swizzle periods in rows: 16 or fewer for K, VCH / 2 for V.  A load round
  // covers whole periods (a lane fetches the same chunk in every round), or
  // a period spans K_VAR rounds that cycle through K_VAR lane offsets.
  static constexpr int K_PERIOD = KCH < 16 ? KCH : 16;
  static constexpr int K_VAR = K_ROWS_PER_LOAD % K_PERIOD == 0 ? 1 : K_PERIOD / K_ROWS_PER_LOAD;
  static_assert(K_VAR == 1 || (K_PERIOD % K_ROWS_PER_LOAD == 0 && K_LOADS % K_VAR == 0), "K swizzle");
  static_assert(V_ROWS_PER_LOAD % (VCH / 2) == 0, "V swizzle");
  static_assert(K_TILE + (KT - 1) * 16 * KROWB < 65536 && V_TILE + (32 * (KT / 2 - 1) + 16) * VROWB < 65536,
                "ds_read immediates");
  static_assert(LDS <= 160 * 1024, "LDS of a CU");
};

// EXACT: D == DP and Dv == DVP, so row strides are compile-time constants and
// no channel is padding (the common case); otherwise padded channels read zero.
// F16: the 16-bit inputs and output are IEEE binary16 instead of bf16.
// PAGED: K and V live in a paged cache (Params::block_table).
template <int DP, int DVP, int NW, int BN_, bool DVSPLIT, bool EXACT, bool F16, bool PAGED>
__global__ __launch_bounds__(64 * NW, 8 / NW) void prefill_bf16_kernel(Params p) {
  using S = PrefillShape<DP, DVP, NW, BN_>;
  constexpr int NT = S::NT, KT = S::KT;
  constexpr int ROWS_W = 16 * NT;  // rows per wave
  using E = Elem<F16>;
  constexpr int BN = S::BN;
  const int D = EXACT ? DP : p.D;
  // DVSPLIT: this workgroup computes channels [dv0, dv0 + DVP) of the Dv_all
  // output channels (part dv0 / DVP of p.dv_parts); the scores are the same
  // for every part.  Dv is the width of this part.
  const int Dv_all = DVSPLIT ? p.Dv : (EXACT ? DVP : p.Dv);
  __shared__ __attribute__((aligned(16))) unsigned char ring[S::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  const PrefillTile tile = prefill_tile(p);
  const int b = tile.b, kh = tile.kh, Q = p.Q;
  const int dv0 = DVSPLIT ? tile.dv_part * DVP : 0;
  const int Dv = DVSPLIT ? min(DVP, Dv_all - dv0) : Dv_all;
  const bool lead = !DVSPLIT || tile.dv_part == 0;  // writes the row statistics (m, l, LSE)

  const int Kb = clamp_len(p.seqlens, b, p.K);
  const int delta = row_delta(Kb, Q, p.causal_shift);  // absolute position of query row q is q + delta
  const int W = p.window;

  // The tile's rows and their query positions bound its KV range.
  const int t_last = min(tile.r0 + kPrefillBM, tile.n_rows) - 1;
  int tq_lo, tq_hi;
  row_q_range(tile.r0, t_last, Q, &tq_lo, &tq_hi);
  const int kv_hi = min(Kb, tq_hi + delta + 1);
  const int kv_lo = W > 0 ? max(0, tq_lo + delta - W + 1) : 0;
  int jb0 = kv_lo / BN;
  int jb1 = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : jb0;
  if (p.n_split > 1) {  // this workgroup's piece: split_blocks 64-key blocks, or what is left of them
    const int64_t pb = (int64_t)p.split_blocks * (kPrefillBN / BN);
    const int64_t s0 = (int64_t)jb0 + (int64_t)tile.split * pb;
    jb0 = (int)min((int64_t)jb1, s0);
    jb1 = (int)min((int64_t)jb1, s0 + pb);
  }

  // Wave-level (scalar) row range and the positions its rows span.
  const int rw0 = tile.r0 + wave * ROWS_W;
  const bool wave_has_rows = rw0 < tile.n_rows;
  int qw_lo = 0, qw_hi = 0;
  if (wave_has_rows) row_q_range(rw0, min(rw0 + ROWS_W, tile.n_rows) - 1, Q, &qw_lo, &qw_hi);
  const int pw_first = qw_lo + delta, pw_last = qw_hi + delta;
  const float c = p.scale_log2;
  const uint32_t qx = p.q_sign ? 0x80008000u : 0u;

  // This lane's rows (one per 16-row MFMA tile): query row q_row[t] of head
  // h_base + hh_row[t]; row_ok[t] false past the row list.
  int q_row[NT], hh_row[NT];
  bool row_ok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = rw0 + 16 * t + l16;
    row_ok[t] = r < tile.n_rows;
    hh_row[t] = r / Q;
    q_row[t] = r - hh_row[t] * Q;
  }
  auto row_index = [&](int t) {  // flat (b, head, q) row of O and LSE
    return ((int64_t)b * p.Hq + tile.h_base + hh_row[t]) * Q + q_row[t];
  };
  // Partial-state slot of this lane's row t in a split pass.
  auto part_slot = [&](int t) { return (int64_t)tile.part * kPrefillBM + (rw0 - tile.r0) + 16 * t + l16; };

  // A tile or piece with no key (an empty sequence, rows above a short
  // sequence's first key, a piece past the end of the tile's range): its rows
  // get O = 0 and LSE = -inf, or an empty partial state, without loading Q.
  // The condition is uniform over the workgroup.
  if (jb0 >= jb1) {
    if (!wave_has_rows) return;
    if (p.n_split > 1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (row_ok[t] && lead && g4 == 0) {
          p.ws_m[part_slot(t)] = -INFINITY;
          p.ws_l[part_slot(t)] = 0.f;
        }
      }
      return;
    }
    // Zero rows written whole, 16 bytes per lane, non-temporal (O is not
    // read again here).
    const int nrows = min(ROWS_W, tile.n_rows - rw0), chunks = Dv / 8;
    for (int i = lane; i < nrows * chunks; i += 64) {
      const int rr = i / chunks, r = rw0 + rr;
      const int hh = r / Q;
      const int64_t row = ((int64_t)b * p.Hq + tile.h_base + hh) * Q + (r - hh * Q);
      __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                  reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.o) + row * Dv_all + dv0 +
                                                           8 * (i - rr * chunks)));
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (row_ok[t] && lead && g4 == 0) p.lse[row_index(t)] = -INFINITY;
    return;
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds row l16 of the tile,
  // channels 32s + 8*g4 .. +7.
  bf16x8 qf[NT][S::KS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + row_index(t) * D;
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
      const int col = 32 * s + 8 * g4;
      uint4 u = (row_ok[t] && col < D) ? load_u4(qrow + col) : zero_u4();
      u.x ^= qx; u.y ^= qx; u.z ^= qx; u.w ^= qx;
      qf[t][s] = __builtin_bit_cast(bf16x8, u);
    }
  }
  // Q is in registers before any direct load is issued (issuing the first
  // K/V block ahead of the Q loads measured no different, on the dense and
  // on the windowed variable-length prefill).
  wait_vmcnt<0>();
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int s = 0; s < S::KS; ++s) launder(qf[t][s]);

  // Direct loads.  Load round i of wave w fills tile bytes [(NW*i + w) KiB,
  // +1 KiB); lane l's 16 bytes land at position l of that KiB, so the lane
  // fetches the global chunk the swizzle puts there.  A round covers a whole
  // number of swizzle periods of rows, so the chunk a lane fetches is the same
  // in every round and its global offset advances by a fixed step.
  // Round r of a tile covers rows r * ROWS_PER_LOAD onward; `first_row`
  // shifts the lane's row for the K_VAR offsets of a K swizzle period.
  auto lane_off = [&](int rowb, bool is_v, int stride, int col0, int width, int first_row) -> uint32_t {
    const int off = wave * 1024 + 16 * lane;
    const int row = off / rowb + first_row, pos = (off % rowb) >> 4;
    const int ch = pos ^ (is_v ? swz_v<S::VCH>(row) : swz_k<S::KCH>(row));
    if (EXACT) return (uint32_t)(row * stride + col0 + ch * 8) * 2;
    return ch < width / 8 ? (uint32_t)(row * stride + col0 + ch * 8) * 2 : kOutOfRange;
  };
  uint32_t koff[S::K_VAR];
#pragma unroll
  for (int v = 0; v < S::K_VAR; ++v) koff[v] = lane_off(S::KROWB, false, D, 0, D, v * S::K_ROWS_PER_LOAD);
  const uint32_t voff = lane_off(S::VROWB, true, Dv_all, dv0, Dv, 0);
  const uint32_t kstep = (uint32_t)(S::K_VAR * S::K_ROWS_PER_LOAD * D * 2);
  const uint32_t vstep = (uint32_t)(S::V_ROWS_PER_LOAD * Dv_all * 2);
  const uint32_t lds0 = lds_offset(ring);
  // Block jb's loads; `page` holds its keys when the cache is paged (blocks
  // never straddle a page), read from the table a block ahead of its use.
  // Contiguous cache: the (batch, kv-head) slices' addresses once per tile;
  // a block's K/V start at a 32-bit byte offset into them.
  const uint16_t* kslice = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.Hkv + kh) * p.K * D;
  const uint16_t* vslice = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.Hkv + kh) * p.K * Dv_all;
  auto issue = [&](int jb, int stg, int page) {
    const int kb0 = jb * BN;
    rsrc_t rk, rv;
    if constexpr (PAGED) {
      const KvSpan sp = kv_span_t<PAGED>(p, b, kh, kb0, page);
      const uint32_t rows_left = (uint32_t)min(Kb - kb0, sp.rows);
      rk = slice_rsrc(sp.k, rows_left * D * 2);
      rv = slice_rsrc(sp.v, rows_left * Dv_all * 2);
    } else {
      (void)page;
      const uint32_t rows_left = (uint32_t)(Kb - kb0);
      rk = slice_rsrc(reinterpret_cast<const char*>(kslice) + (uint32_t)kb0 * (uint32_t)(D * 2), rows_left * D * 2);
      rv = slice_rsrc(reinterpret_cast<const char*>(vslice) + (uint32_t)kb0 * (uint32_t)(Dv_all * 2),
                      rows_left * Dv_all * 2);
    }
    const uint32_t kbase = lds0 + stg * S::K_TILE + wave * 1024;
    const uint32_t vbase = lds0 + S::V_BASE + stg * S::V_TILE + wave * 1024;
#pragma unroll
    for (int i = 0; i < S::K_LOADS; ++i)
      load_lds16(rk, kbase + i * S::ROUND, koff[i % S::K_VAR] + (i / S::K_VAR) * kstep);
#pragma unroll
    for (int i = 0; i < S::V_LOADS; ++i) load_lds16(rv, vbase + i * S::ROUND, voff + i * vstep);
  };

  // Per-lane LDS read offsets (stage 0).  K fragment of k-step s, key tile i:
  // row 16i + l16, chunk (4s + g4) ^ swz_k(row); swz_k(row) = swz_k(l16) for
  // every i, below 16, so k-step s reads at ka[s % 4] + 256 * (s / 4).  V^T
  // fragment of dv tile j: rows 32kk + 4*g4 + l16/4 (+16), chunk
  // (2j + (l16 & 3)/2) ^ swz_v(row), half (l16 & 1); swz_v is the same for
  // every kk and for the +16 row.
  constexpr int KA = S::KS < 4 ? S::KS : 4;
  uint32_t ka[KA], va[S::JV];
#pragma unroll
  for (int s = 0; s < KA; ++s)
    ka[s] = lds0 + l16 * S::KROWB + ((((4 * s + g4) ^ swz_k<S::KCH>(l16))) << 4);
  auto k_addr = [&](int st) { return ka[st % 4] + 256 * (st / 4); };
  {
    const int vrow = 4 * g4 + (l16 >> 2);
#pragma unroll
    for (int j = 0; j < S::JV; ++j)
      va[j] = lds0 + S::V_BASE + vrow * S::VROWB + (((2 * j + ((l16 & 3) >> 1)) ^ swz_v<S::VCH>(vrow)) << 4) +
              (l16 & 1) * 8;
  }

  // The blocks in which some row of this wave has a legal key, [see_lo,
  // see_hi], and those in which every key is legal for every row of the
  // wave, [full_lo, full_hi] (scalar, once per tile): a block is seen iff
  // kb0 <= pw_last, kb0 < K_b and (no window or kb0 + BN - 1 >= pw_first -
  // W + 1); full iff kb0 + BN - 1 <= pw_first, kb0 + BN <= K_b and (no
  // window or kb0 >= pw_last - W + 1).  BN is a power of two, so the
  // floor / ceiling divisions are arithmetic shifts for either sign.
  constexpr int LG = BN == 64 ? 6 : 5;
  static_assert((1 << LG) == BN, "block size");
  auto fdiv = [](int a) { return a >> LG; };
  auto cdiv = [](int a) { return (a + BN - 1) >> LG; };
  const int see_hi = wave_has_rows ? min(fdiv(pw_last), fdiv(Kb - 1)) : -1;
  const int see_lo = W > 0 ? cdiv(pw_first - W + 2 - BN) : 0;
  const int full_hi = min(fdiv(pw_first - BN + 1), fdiv(Kb - BN));
  const int full_lo = W > 0 ? cdiv(pw_last - W + 1) : 0;

  float m_run[NT], l_run[NT];
  f32x4 acc[S::JV][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int j = 0; j < S::JV; ++j) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Initial S^T accumulator of a block that straddles the causal diagonal, a
  // window edge or the sequence end: 0 for a legal key, -inf otherwise, so the
  // products leave -inf at every illegal key.  Key kb0 + 4*g4 + x (x = 16i +
  // r) is legal for query position pq iff lo <= x <= hi, with hi from
  // causality and K_b and lo from the window.  Which bound can bite anywhere
  // in the wave is known per block (scalar): the upper one on the diagonal or
  // at K_b, the lower one at a window edge; with one of them, one signed
  // compare against an immediate x per element, with both one unsigned range
  // compare (an empty range moves lo out of reach).
  auto mask_bias = [&](int kb0, f32x4 (&s)[KT][NT]) {
    const bool need_lo = W > 0 && kb0 < pw_last - W + 1;
    const bool need_hi = !(kb0 + BN - 1 <= pw_first && kb0 + BN <= Kb);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int rel = q_row[t] + delta - kb0 - 4 * g4;  // pq - (kb0 + 4*g4)
      const int hi = min(rel, Kb - kb0 - 4 * g4 - 1);
      const int lo = W > 0 ? max(rel - W + 1, 0) : 0;
      if (need_lo && need_hi) {
        const bool none = hi < lo;
        const uint32_t span = none ? 0u : (uint32_t)(hi - lo);
        const int lo2 = none ? (1 << 30) : lo;
#pragma unroll
        for (int i = 0; i < KT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[i][t][r] = (uint32_t)(16 * i + r - lo2) <= span ? 0.f : -INFINITY;
      } else if (need_hi) {
#pragma unroll
        for (int i = 0; i < KT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[i][t][r] = 16 * i + r <= hi ? 0.f : -INFINITY;
      } else {
#pragma unroll
        for (int i = 0; i < KT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[i][t][r] = 16 * i + r >= lo ? 0.f : -INFINITY;
      }
    }
  };

  // Block row max in log2 units (-inf: no legal key in the block; the scale
  // factor c is positive, so -inf * c stays -inf).
  // Column max over the block in log2 units (-inf: no legal key; c > 0 keeps
  // -inf * c at -inf): per-lane v_max3 chain, then the four lane groups.
  auto block_max = [&](const f32x4 (&s)[KT][NT], int t) {
    float mx = max3f(s[0][t][0], s[0][t][1], s[0][t][2]);
    mx = max3f(mx, s[0][t][3], s[1][t][0]);
    mx = max3f(mx, s[1][t][1], s[1][t][2]);
    if constexpr (KT == 4) {
      mx = max3f(mx, s[1][t][3], s[2][t][0]);
      mx = max3f(mx, s[2][t][1], s[2][t][2]);
      mx = max3f(mx, s[2][t][3], s[3][t][0]);
      mx = max3f(mx, s[3][t][1], s[3][t][2]);
      mx = max2f(mx, s[3][t][3]);
    } else {
      static_assert(KT == 2, "block of 32 or 64 keys");
      mx = max2f(mx, s[1][t][3]);
    }
    return group4_max(mx) * c;
  };

  // Online softmax of one block (scores s -> bf16 weights pf).  The weights
  // are first formed against the current reference m (lazy: it moves only
  // when needed).  If every lane's partial row sum over its 16 keys is at
  // most 2^kLazyRescale, no weight exceeds that bound and the reference
  // stays; no block max is computed.  Otherwise, or while a row has no
  // reference yet, the column max moves the reference, the accumulators are
  // rescaled and the weights recomputed (rare: a few blocks per row).
  auto softmax = [&](const f32x4 (&s)[KT][NT], bf16x8 (&pf)[NT][KT / 2]) {
    f32x4 e[KT][NT];
    float rs[NT];
    auto weights = [&](int t) {
      const float mneg = m_run[t] == -INFINITY ? 0.f : -m_run[t];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < KT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[i][t][r] = fast_exp2(fmaf(s[i][t][r], c, mneg));
          sum += e[i][t][r];
        }
      }
      rs[t] = sum;
    };
#pragma unroll
    for (int t = 0; t < NT; ++t) weights(t);
    constexpr float kBound = 256.f;  // 2^kLazyRescale
    static_assert(kLazyRescale == 8.f, "kBound is 2^kLazyRescale");
    bool need = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) need = need | !(rs[t] <= kBound) | (m_run[t] == -INFINITY);
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float mnew = fmaxf(m_run[t], block_max(s, t));
        const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m_run[t] - mnew);
        m_run[t] = mnew;
        l_run[t] *= alpha;
#pragma unroll
        for (int j = 0; j < S::JV; ++j) acc[j][t] *= alpha;
        weights(t);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      l_run[t] += rs[t];
#pragma unroll
      for (int kk = 0; kk < KT / 2; ++kk) pf[t][kk] = E::pack(e[2 * kk][t], e[2 * kk + 1][t]);
    }
  };

  // One KV block in ring stage STG (a compile-time constant, so every LDS
  // address below is a per-lane register plus an immediate).  Only the
  // initial accumulator of S^T differs between blocks whose keys are all
  // legal for every row of the wave (FULL: zero, an inline constant) and the
  // rest (mask_bias).
  auto body = [&](int jb, auto stg_tag, bool full) {
    constexpr int STG = decltype(stg_tag)::value;
    constexpr uint32_t KOFF = STG * S::K_TILE, VOFF = STG * S::V_TILE;
    {
      const int kb0 = jb * BN;
      f32x4 s[KT][NT];
      // S^T = K Q^T.  The K fragments of k-step st + 1 are read while the
      // MFMAs of k-step st run; the fences keep the compiler from hoisting
      // every read of the block (64 registers) ahead of the products.
      auto qk = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        bf16x8 ak[2][KT];
        if constexpr (!FULL) mask_bias(kb0, s);
#pragma unroll
        for (int i = 0; i < KT; ++i) ak[0][i] = lds_read_b128(k_addr(0) + KOFF + 16 * i * S::KROWB);
#pragma unroll
        for (int st = 0; st < S::KS; ++st) {
          if (st + 1 < S::KS) {
#pragma unroll
            for (int i = 0; i < KT; ++i)
              ak[(st + 1) & 1][i] = lds_read_b128(k_addr(st + 1) + KOFF + 16 * i * S::KROWB);
          }
#pragma unroll
          for (int i = 0; i < KT; ++i) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const f32x4 c0 = (FULL && st == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : s[i][t];
              s[i][t] = E::mfma(ak[st & 1][i], qf[t][st], c0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (full) qk(std::true_type{});
      else qk(std::false_type{});
      // V^T fragment of (kk, j): rows 32kk + 4*g4 + l16/4 and 16 below.
      auto read_v = [&](int kk, int j) {
        const uint32_t lo = va[j] + VOFF + 32 * kk * S::VROWB;
        return concat_bf16x4(lds_read_tr16(lo), lds_read_tr16(lo + 16 * S::VROWB));
      };
      // The first two V fragments are in flight during the softmax.
      bf16x8 av[2][2];
      av[0][0] = read_v(0, 0);
      av[0][1] = read_v(0, 1);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 pf[NT][KT / 2];
      softmax(s, pf);
      __builtin_amdgcn_sched_barrier(0);
      // O^T += V^T P^T over the block's 32-key halves, two dv tiles per step
      // with the next step's fragments in flight.  The contraction index e of
      // the B operand maps to key 32kk + 4*g4 + e (e < 4) or 32kk + 16 + 4*g4 +
      // e - 4, the S^T register layout; the V^T fragment is read in the same
      // order.
      constexpr int NP = (KT / 2) * (S::JV / 2);  // steps of two dv tiles over the halves
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        const int kk = n / (S::JV / 2), j = 2 * (n % (S::JV / 2));
        if (n + 1 < NP) {
          const int kk1 = (n + 1) / (S::JV / 2), j1 = 2 * ((n + 1) % (S::JV / 2));
          av[(n + 1) & 1][0] = read_v(kk1, j1);
          av[(n + 1) & 1][1] = read_v(kk1, j1 + 1);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[j + u][t] = E::mfma(av[n & 1][u], pf[t][kk], acc[j + u][t]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // Paged cache: the page of block jb + 1 is loaded during block jb - 1 by a
  // buffer load of this sequence's table row and settled after that block's
  // closing wait, so no wait for it ever covers the next block's K/V loads.
  // Without a table nothing is loaded (and the register the loads target is
  // never written otherwise, so no wait is ever placed for it).
  constexpr bool paged = PAGED;
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(p.block_table ? p.block_table + (int64_t)b * p.pages_per_seq : nullptr), (short)0,
      p.block_table ? p.pages_per_seq * 4 : 0, kRsrcWord3);
  auto page_fetch = [&](int jb) -> int {
    return __builtin_amdgcn_raw_buffer_load_b32(trs, ((min(jb, jb1 - 1) * BN) >> p.page_shift) * 4, 0, 0);
  };
  auto page_settle = [&](int x) -> int {
    launder(x);
    const int pg = __builtin_amdgcn_readfirstlane(x);
    return pg < 0 ? 0 : (pg >= p.num_pages ? max(p.num_pages - 1, 0) : pg);
  };
  int pg_next = 0;  // loaded, not yet settled
  auto block = [&](int jb, auto stg_tag) {
    const int pg = paged ? page_settle(pg_next) : 0;
    if (jb + 1 < jb1) issue(jb + 1, decltype(stg_tag)::value ^ 1, pg);
    if (paged) pg_next = page_fetch(jb + 2);
    if (jb >= see_lo && jb <= see_hi) body(jb, stg_tag, jb >= full_lo && jb <= full_hi);
    // Block jb + 1 has landed for every wave, and every wave is done with
    // the stage of block jb, which the next block's loads overwrite.
    wait_vmcnt<0>();
    __syncthreads();
  };

  // Prologue (jb0 < jb1 here): the first block (its table entry first when
  // the cache is paged).
  if (paged) {
    pg_next = page_fetch(jb0);
    wait_vmcnt<0>();
  }
  issue(jb0, 0, paged ? page_settle(pg_next) : 0);
  if (paged) pg_next = page_fetch(jb0 + 1);
  wait_vmcnt<0>();
  __syncthreads();
  for (int jb = jb0; jb < jb1; jb += 2) {
    block(jb, std::integral_constant<int, 0>{});
    if (jb + 1 < jb1) block(jb + 1, std::integral_constant<int, 1>{});
  }

  if (!wave_has_rows) return;
  if (p.n_split > 1) {
    // Partial state of this piece: (m, l) and the unnormalised acc; a row
    // that saw no legal key gets m = -inf, l = 0 and no acc.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float lt = group4_sum(l_run[t]);
      if (row_ok[t]) {
        const int64_t slot = part_slot(t);
        if (lead && g4 == 0) {
          p.ws_m[slot] = lt > 0.f ? m_run[t] : -INFINITY;
          p.ws_l[slot] = lt;
        }
        if (lt > 0.f) {
          float* arow = p.ws_acc + slot * Dv_all + dv0;
#pragma unroll
          for (int j = 0; j < S::JV; ++j) {
            const int dv = 16 * j + 4 * g4;
            if (dv < Dv) *reinterpret_cast<f32x4*>(arow + dv) = acc[j][t];
          }
        }
      }
    }
    return;
  }
  // O = acc / l in the storage type, staged row-major in this wave's slice
  // of the ring (every wave passed the last block's barrier and no load is
  // in flight, so the ring is free; rows padded by 16 bytes so the 8-byte
  // writes of 16 rows fall on distinct banks), then stored as whole rows,
  // 16 bytes per lane, non-temporal (windowed varlen prefill 504.6 -> 493.4
  // us, dense 518.5 -> 512.0 us, against cached stores).
  constexpr int OSTRIDE = DVP + 8;  // elements per staged row
  static_assert(NW * ROWS_W * OSTRIDE * 2 <= S::LDS, "O staging fits the ring");
  uint16_t* ostage = reinterpret_cast<uint16_t*>(ring) + wave * ROWS_W * OSTRIDE;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = group4_sum(l_run[t]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int j = 0; j < S::JV; ++j) {
      ushort4 ov;
      ov.x = E::cvt(acc[j][t][0] * inv);
      ov.y = E::cvt(acc[j][t][1] * inv);
      ov.z = E::cvt(acc[j][t][2] * inv);
      ov.w = E::cvt(acc[j][t][3] * inv);
      *reinterpret_cast<ushort4*>(ostage + (16 * t + l16) * OSTRIDE + 16 * j + 4 * g4) = ov;
    }
    if (row_ok[t] && lead && g4 == 0)
      p.lse[row_index(t)] = lt > 0.f ? (m_run[t] + __log2f(lt)) * 0.69314718055994530942f : -INFINITY;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int nrows = min(ROWS_W, tile.n_rows - rw0), chunks = Dv / 8;
  for (int i = lane; i < nrows * chunks; i += 64) {
    const int rr = i / chunks, c8 = 8 * (i - rr * chunks), r = rw0 + rr;
    const int hh = r / Q;
    const int64_t row = ((int64_t)b * p.Hq + tile.h_base + hh) * Q + (r - hh * Q);
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(ostage + rr * OSTRIDE + c8),
                                reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.o) + row * Dv_all + dv0 + c8));
  }
}

// Combine pass of split-KV prefill: one wave per output row merges the row's
// n_split partial states in split order (the merge of two online-softmax
// states: rescale both to the larger max, add sums and accumulators), then
// normalises and writes O and the LSE.  Lane l owns channels CPL*l ..
// CPL*l + CPL - 1 (CPL = 2 up to 128 channels, 4 up to 256, 8 up to 512).
// The pieces are taken eight at a time, all their loads issued together, and
// folded into a running (M, L, o); a piece with m = -inf has no acc (never
// written) and is skipped.
struct alignas(32) float8_t {
  float4 lo, hi;
};
template <bool F16, int CPL>
__global__ __launch_bounds__(256) void prefill_combine_kernel(Params p) {
  using V = std::conditional_t<CPL == 2, float2, std::conditional_t<CPL == 4, float4, float8_t>>;
  static_assert(sizeof(V) == CPL * sizeof(float), "channels per lane");
  using E = Elem<F16>;
  constexpr int U = 8;
  const int lane = threadIdx.x & 63;
  // Output row (b, h, q), then the tile that holds it (the inverse of
  // prefill_tile_of): its rank rem in the group and the row within it.
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)p.B * p.Hq * p.Q) return;
  const int q = (int)(row % p.Q);
  const int bh = (int)(row / p.Q);
  const int b = bh / p.Hq, h = bh - b * p.Hq;
  const int kh = h / p.group, hg = h - kh * p.group;
  const int grp = b * p.Hkv + kh;
  const int per_grp = prefill_group_tiles(p.Q, p.group);
  int rem, r_local;
  if (prefill_packed(p.Q, p.group)) {
    const int r = hg * p.Q + q;  // row of the group's list
    rem = per_grp - 1 - r / kPrefillBM;
    r_local = r % kPrefillBM;
  } else {
    const int n_qt = (p.Q + kPrefillBM - 1) / kPrefillBM;
    rem = (n_qt - 1 - q / kPrefillBM) * p.group + hg;
    r_local = q % kPrefillBM;
  }
  // Slot of piece s: ((grp * n_split + s) * per_grp + rem) * 128 + r_local.
  const int64_t slot0 = ((int64_t)grp * p.n_split * per_grp + rem) * kPrefillBM + r_local;
  const int64_t slot_step = (int64_t)per_grp * kPrefillBM;
  const int dv = CPL * lane;
  const bool has_dv = dv < p.Dv;  // Dv is a multiple of 16: all CPL channels or none

  float mx = -INFINITY, l = 0.f, o[CPL] = {};
  for (int s0 = 0; s0 < p.n_split; s0 += U) {
    float ms[U], ls[U];
    V a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t slot = slot0 + (int64_t)(s0 + u) * slot_step;
      const bool in = s0 + u < p.n_split;
      ms[u] = in ? p.ws_m[slot] : -INFINITY;
      ls[u] = in ? p.ws_l[slot] : 0.f;
      a[u] = (in && has_dv) ? *reinterpret_cast<const V*>(p.ws_acc + slot * p.Dv + dv) : V{};
    }
    float mn = mx;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, ms[u]);
    if (mn == -INFINITY) continue;
    const float alpha = exp2f(mx - mn);  // 0 while nothing is merged yet (mx = -inf)
    l *= alpha;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ms[u] == -INFINITY) continue;
      const float w = exp2f(ms[u] - mn);
      l += ls[u] * w;
      const float* av = reinterpret_cast<const float*>(&a[u]);
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] += av[c] * w;
    }
    mx = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (has_dv) {
    uint16_t* orow = static_cast<uint16_t*>(p.o) + row * p.Dv + dv;
    if constexpr (CPL == 2) {
      ushort2 ov;
      ov.x = E::cvt(o[0] * inv);
      ov.y = E::cvt(o[1] * inv);
      *reinterpret_cast<ushort2*>(orow) = ov;
    } else {
#pragma unroll
      for (int c4 = 0; c4 < CPL; c4 += 4) {
        ushort4 ov;
        ov.x = E::cvt(o[c4] * inv);
        ov.y = E::cvt(o[c4 + 1] * inv);
        ov.z = E::cvt(o[c4 + 2] * inv);
        ov.w = E::cvt(o[c4 + 3] * inv);
        *reinterpret_cast<ushort4*>(orow + c4) = ov;
      }
    }
  }
  if (lane == 0) p.lse[row] = l > 0.f ? (mx + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

// The combine pass of a split prefill: one wave per output row, four rows to a
// workgroup; CPL channels per lane cover Dv.
hipError_t launch_prefill_combine(const Params& p, hipStream_t stream) {
  Params arg = p;
  void* args[] = {&arg};
  const dim3 cgrid((unsigned)(((int64_t)p.B * p.Hq * p.Q + 3) / 4));
  const int cpl = p.Dv <= 128 ? 2 : (p.Dv <= 256 ? 4 : 8);
  const void* cfn;
  if (cpl == 2) cfn = p.f16 ? reinterpret_cast<const void*>(&prefill_combine_kernel<true, 2>)
                            : reinterpret_cast<const void*>(&prefill_combine_kernel<false, 2>);
  else if (cpl == 4) cfn = p.f16 ? reinterpret_cast<const void*>(&prefill_combine_kernel<true, 4>)
                                 : reinterpret_cast<const void*>(&prefill_combine_kernel<false, 4>);
  else cfn = p.f16 ? reinterpret_cast<const void*>(&prefill_combine_kernel<true, 8>)
                   : reinterpret_cast<const void*>(&prefill_combine_kernel<false, 8>);
  return hipLaunchKernel(cfn, cgrid, dim3(256), args, 0, stream);
}

template <int DP, int DVP, int NW, int BN, bool DVSPLIT>
static hipError_t launch_prefill_t(const Params& p, hipStream_t stream) {
  const int64_t tiles = (int64_t)prefill_group_tiles(p.Q, p.group) * p.Hkv * p.B;
  const dim3 grid((unsigned)(tiles * p.n_split * p.dv_parts));
  Params arg = p;
  void* args[] = {&arg};
  const void* const kernels[8] = {
      reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, NW, BN, DVSPLIT, false, false, false>),
      reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, NW, BN, DVSPLIT, true, false, false>),
      reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, NW, BN, DVSPLIT, false, true, false>),
      reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, NW, BN, DVSPLIT, true, true, false>),
      reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, NW, BN, DVSPLIT, false, false, true>),
      reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, NW, BN, DVSPLIT, true, false, true>),
      reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, NW, BN, DVSPLIT, false, true, true>),
      reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, NW, BN, DVSPLIT, true, true, true>),
  };
  const int exact = p.D == DP && p.Dv == DVP * p.dv_parts;
  const void* fn = kernels[exact | (p.f16 ? 2 : 0) | (p.block_table ? 4 : 0)];
  hipError_t e = hipLaunchKernel(fn, grid, dim3(64 * NW), args, 0, stream);
  if (e != hipSuccess || p.n_split <= 1) return e;
  return launch_prefill_combine(p, stream);
}

// Heads up to 128 wide: 4 waves of 32 rows, 64-key blocks.  Up to 256 (padded
// to 256 on both sides): 8 waves of 16 rows.  Up to 512: 8 waves of 16 rows
// over 32-key blocks of 512 channels, and the output channels in parts of 256
// computed by separate workgroups that each recompute the scores (the
// accumulators of 512 channels would not fit a wave's registers).
hipError_t launch_prefill_bf16(const Params& p, hipStream_t stream) {
  const int dp = pad_width(p.D), dvp = pad_width(p.Dv);
  if (dp > 256 || dvp > 256) return launch_prefill_t<512, 256, 8, 32, true>(p, stream);
  if (dp > 128 || dvp > 128) return launch_prefill_t<256, 256, 8, 64, false>(p, stream);
  if (dp == 64 && dvp == 64) return launch_prefill_t<64, 64, 4, 64, false>(p, stream);
  if (dp == 64 && dvp == 128) return launch_prefill_t<64, 128, 4, 64, false>(p, stream);
  if (dp == 128 && dvp == 64) return launch_prefill_t<128, 64, 4, 64, false>(p, stream);
  return launch_prefill_t<128, 128, 4, 64, false>(p, stream);
}

}  // namespace attn
