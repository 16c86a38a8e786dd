// bf16 prefill kernel for gfx950: causal GQA attention forward with online
// softmax (LuisaCompute "Attention execution mapping" review, section 1: the
// fixture's bottom-right causal GQA and the (row_max, row_sum, acc) state
// carried across KV blocks; section 2: the phase graph load Q -> per KV block
// load K/V -> QK -> mask -> max/exp/sum -> rescale -> PV -> update).
//
// Mapping on CDNA4:
//   * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//     owns 32 rows as two 16-column MFMA tiles, Q held in registers; two
//     workgroups share a CU, so each SIMD runs one wave of each;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16, so each lane holds 16 keys of
//     one query column and the row max/sum is in-lane plus two permlane swaps;
//     P^T stays in that register layout and feeds O^T = V^T P^T directly, V^T
//     fragments read from row-major LDS through ds_read_b64_tr_b16;
//   * software pipeline over KV blocks of 64 keys: while a wave runs the
//     softmax of block j on the VALU, the MFMA unit computes S^T of block j+1
//     (the FlyDSL FMHA post describes the same overlap of one tile's softmax
//     with another tile's matrix products), then P.V of block j; so K runs
//     one block ahead of V, in a three-stage LDS ring against V's two stages
//     (80 KiB at D = Dv = 128, two workgroups per CU);
//   * K/V blocks go HBM -> LDS by direct buffer loads issued a step ahead, one
//     barrier per block; rows past K_b and channels past D read as zero from
//     the buffer range check;
//   * tiles are XOR-swizzled in LDS so the 16-byte K fragment reads and the
//     transposed V reads are free of bank conflicts; a lane's fragment
//     addresses are one register XOR a k-step or dv-tile constant, plus an
//     immediate for the key tile and the V stage (the loop is unrolled over
//     the two V stages);
//   * the VALU work per block is kept to the softmax itself: wave-level
//     control is scalar; masks are evaluated only on blocks that straddle the
//     causal diagonal, a window edge or the sequence end, as the initial S^T
//     accumulator (0 for a legal key, -inf otherwise); blocks no row of a wave
//     can see are skipped by that wave; row maxima are v_max3 chains; and the
//     running max moves only when a row's block max exceeds it by more than
//     kLazyRescale (the accumulators are rescaled in a branch after the
//     interleaved section);
//   * tiles are ordered heaviest causal tile first within a (batch, kv-head)
//     group, and the groups are dealt to the 8 XCDs so an XCD streams one
//     group's K/V through its L2 at a time.
#include <type_traits>

#include "attn_internal.h"

namespace attn {

template <int DP, int DVP>
struct PrefillShape {
  static constexpr int KS = DP / 32;        // 32-deep k-steps of Q.K
  static constexpr int JV = DVP / 16;       // 16-wide dv tiles of O^T
  static constexpr int KCH = DP / 8;        // 16-byte chunks per K row
  static constexpr int VCH = DVP / 8;
  static constexpr int KROWB = DP * 2;      // LDS bytes per K row
  static constexpr int VROWB = DVP * 2;
  static constexpr int K_TILE = kPrefillBN * KROWB;
  static constexpr int V_TILE = kPrefillBN * VROWB;
  static constexpr int K_STAGES = 3;        // K runs one block ahead of V
  static constexpr int V_BASE = K_STAGES * K_TILE;
  static constexpr int LDS = V_BASE + 2 * V_TILE;
  static constexpr int K_LOADS = K_TILE / 4096;  // 16-byte loads per thread per block
  static constexpr int V_LOADS = V_TILE / 4096;
  static constexpr int K_ROWS_PER_LOAD = 4096 / KROWB;  // tile rows one 4 KiB load round covers
  static constexpr int V_ROWS_PER_LOAD = 4096 / VROWB;
  static_assert(K_TILE % 4096 == 0 && V_TILE % 4096 == 0, "load split");
};

// Block index -> (query tile, batch, head).  When the (batch, kv-head) groups
// divide evenly over the 8 XCDs (workgroup i runs on XCD i % 8), each XCD gets
// whole groups and finishes one group (all its query heads and tiles,
// heaviest tile first) before the next, so the workgroups resident on an XCD
// stream the same K/V slice through its L2; otherwise the order is heaviest
// tile first with heads fastest.
__device__ __forceinline__ void prefill_tile(const Params& p, int n_qt, int* qt, int* b, int* h) {
  const int x = blockIdx.x;
  const int groups = p.B * p.Hkv;
  if ((groups & 7) == 0) {
    const int xcd = x & 7, slot = x >> 3;
    const int per_grp = p.group * n_qt;
    const int gi = slot / per_grp, rem = slot - gi * per_grp;
    const int qrank = rem / p.group;
    const int grp = gi * 8 + xcd;
    *b = grp / p.Hkv;
    *h = (grp - *b * p.Hkv) * p.group + rem % p.group;
    *qt = n_qt - 1 - qrank;
  } else {
    *h = x % p.Hq;
    const int y = x / p.Hq;
    *b = y % p.B;
    *qt = n_qt - 1 - y / p.B;
  }
}

// EXACT: D == DP and Dv == DVP, so row strides are compile-time constants and
// no channel is padding (the common case); otherwise padded channels read zero.
template <int DP, int DVP, bool EXACT>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(Params p) {
  using S = PrefillShape<DP, DVP>;
  constexpr int BN = kPrefillBN;
  const int D = EXACT ? DP : p.D;
  const int Dv = EXACT ? DVP : p.Dv;
  __shared__ __attribute__((aligned(16))) unsigned char ring[S::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  const int n_qt = (p.Q + kPrefillBM - 1) / kPrefillBM;
  int qt, b, h;
  prefill_tile(p, n_qt, &qt, &b, &h);
  const int kh = h / p.group;

  const int Kb = clamp_len(p.seqlens, b, p.K);
  const int delta = Kb - p.Q;  // absolute position of row q is q + delta
  const int W = p.window;
  const int q0 = qt * kPrefillBM;
  const int q_end = min(q0 + kPrefillBM, p.Q);

  const int kv_hi = min(Kb, q_end - 1 + delta + 1);
  const int kv_lo = W > 0 ? max(0, q0 + delta - W + 1) : 0;
  const int jb0 = kv_lo / BN;
  const int jb1 = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : jb0;

  const int64_t kv_slice = (int64_t)b * p.Hkv + kh;
  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.Hq + h) * p.Q * D;
  const uint16_t* kslice = static_cast<const uint16_t*>(p.k) + kv_slice * p.K * D;
  const uint16_t* vslice = static_cast<const uint16_t*>(p.v) + kv_slice * p.K * Dv;
  uint16_t* og = static_cast<uint16_t*>(p.o) + ((int64_t)b * p.Hq + h) * p.Q * Dv;
  float* lg = p.lse + ((int64_t)b * p.Hq + h) * p.Q;

  // Wave-level (scalar) row range and absolute positions.
  const int qw0 = q0 + wave * kPrefillRowsPerWave;
  const bool wave_has_rows = qw0 < p.Q;
  const int qw_last = min(qw0 + kPrefillRowsPerWave, p.Q) - 1;
  const int pw_first = qw0 + delta, pw_last = qw_last + delta;
  const float c = p.scale_log2;
  const uint32_t qx = p.q_sign ? 0x80008000u : 0u;

  // Q fragments (B operand of S^T = K Q^T): lane holds row l16 of the tile,
  // channels 32s + 8*g4 .. +7.
  bf16x8 qf[2][S::KS];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = qw0 + 16 * t + l16;
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
      const int col = 32 * s + 8 * g4;
      uint4 u = (row < p.Q && col < D) ? load_u4(qg + (int64_t)row * D + col) : zero_u4();
      u.x ^= qx; u.y ^= qx; u.z ^= qx; u.w ^= qx;
      qf[t][s] = __builtin_bit_cast(bf16x8, u);
    }
  }
  // Q is in registers before any direct load is issued.
  wait_vmcnt<0>();
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < S::KS; ++s) launder(qf[t][s]);

  // Direct loads.  Load round i of wave w fills tile bytes [(4i + w) KiB,
  // +1 KiB); lane l's 16 bytes land at position l of that KiB, so the lane
  // fetches the global chunk the swizzle puts there.  A round covers a whole
  // number of swizzle periods of rows, so the chunk a lane fetches is the same
  // in every round and its global offset advances by a fixed step.
  auto lane_off = [&](int rowb, int nch, bool is_v, int width) -> uint32_t {
    const int off = wave * 1024 + 16 * lane;
    const int row = off / rowb, pos = (off % rowb) >> 4;
    const int ch = pos ^ (is_v ? ((2 * row) & (nch - 1)) : (row & (nch - 1)));
    if (EXACT) return (uint32_t)(row * width + ch * 8) * 2;
    return ch < width / 8 ? (uint32_t)(row * width + ch * 8) * 2 : kOutOfRange;
  };
  const uint32_t koff = lane_off(S::KROWB, S::KCH, false, D);
  const uint32_t voff = lane_off(S::VROWB, S::VCH, true, Dv);
  const uint32_t kstep = (uint32_t)(S::K_ROWS_PER_LOAD * D * 2);
  const uint32_t vstep = (uint32_t)(S::V_ROWS_PER_LOAD * Dv * 2);
  const uint32_t lds0 = lds_offset(ring);
  // K of block jb lives in K stage (jb - jb0) % 3, V in V stage (jb - jb0) % 2.
  auto kstage_off = [&](int jb) -> uint32_t { return (uint32_t)((jb - jb0) % S::K_STAGES) * S::K_TILE; };
  // The per-round offsets are formed at each issue (the base is laundered so
  // the compiler does not keep all of them live across the loop).
  auto issue_k = [&](int jb) {
    const int kb0 = jb * BN;
    const rsrc_t rk = slice_rsrc(kslice + (int64_t)kb0 * D, (uint32_t)(Kb - kb0) * D * 2);
    const uint32_t base = lds0 + kstage_off(jb) + wave * 1024;
    uint32_t o = koff;
    launder(o);
#pragma unroll
    for (int i = 0; i < S::K_LOADS; ++i) load_lds16(rk, base + i * 4096, o + i * kstep);
  };
  auto issue_v = [&](int jb, int vst) {
    const int kb0 = jb * BN;
    const rsrc_t rv = slice_rsrc(vslice + (int64_t)kb0 * Dv, (uint32_t)(Kb - kb0) * Dv * 2);
    const uint32_t base = lds0 + S::V_BASE + vst * S::V_TILE + wave * 1024;
    uint32_t o = voff;
    launder(o);
#pragma unroll
    for (int i = 0; i < S::V_LOADS; ++i) load_lds16(rv, base + i * 4096, o + i * vstep);
  };

  // Per-lane LDS read offsets (stage 0).  K fragment of k-step s, key tile i:
  // row 16i + l16, chunk (4s + g4) ^ swz_k(row); swz_k(row) = l16 % KCH for
  // every i.  V^T fragment of dv tile j: rows 32kk + 4*g4 + l16/4 (+16), chunk
  // (2j + (l16 & 3)/2) ^ swz_v(row), half (l16 & 1); swz_v is the same for
  // every kk and for the +16 row.
  // With the K row stride a multiple of 128 bytes the chunk bits of the
  // offset start at bit 4, so the address for k-step s is ka0 ^ (s << 6)
  // ((4s + g4) ^ swz = 4s ^ (g4 ^ swz)): one register instead of KS.
  static_assert(S::KROWB % 128 == 0 && S::K_TILE % 256 == 0, "K address bits");
  const uint32_t ka0 = lds0 + l16 * S::KROWB + (((g4 ^ swz_k<S::KCH>(l16))) << 4);
  // Likewise the V^T fragment of dv tile j is at va0 ^ (j << 5): swz_v is
  // even, so (2j + b) ^ swz = 2j ^ (b + swz) and the chunk bits start at 4.
  static_assert(S::VROWB % 128 == 0 && S::V_BASE % 256 == 0, "V address bits");
  const int vrow = 4 * g4 + (l16 >> 2);
  const uint32_t va0 =
      lds0 + S::V_BASE + vrow * S::VROWB + ((((l16 & 3) >> 1) ^ swz_v<S::VCH>(vrow)) << 4) + (l16 & 1) * 8;

  // Whether any row of this wave has a legal key in block jb / every key of
  // block jb is legal for every row of this wave (scalar).
  auto wave_sees = [&](int jb) {
    const int kb0 = jb * BN;
    return wave_has_rows && kb0 <= pw_last && kb0 < Kb && !(W > 0 && kb0 + BN - 1 < pw_first - W + 1);
  };
  auto wave_full = [&](int jb) {
    const int kb0 = jb * BN;
    return (kb0 + BN - 1 <= pw_first) && (kb0 + BN <= Kb) && (W <= 0 || kb0 >= pw_last - W + 1);
  };

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4 acc[S::JV][2];
#pragma unroll
  for (int j = 0; j < S::JV; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Initial S^T accumulator of a block that straddles the causal diagonal, a
  // window edge or the sequence end: 0 for a legal key, -inf otherwise, so the
  // products leave -inf at every illegal key.  Key kb0 + 4*g4 + x (x = 16i +
  // r) is legal for query position pq iff lo <= x <= hi, with hi from
  // causality and K_b and lo from the window: one unsigned compare against an
  // immediate x per element.
  auto mask_bias = [&](int kb0, f32x4 (&s)[4][2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int rel = qw0 + 16 * t + l16 + delta - kb0 - 4 * g4;  // pq - (kb0 + 4*g4)
      const int hi = min(rel, Kb - kb0 - 4 * g4 - 1);
      const int lo = W > 0 ? max(rel - W + 1, 0) : 0;
      const uint32_t span = (uint32_t)(hi - lo);
      const bool none = hi < lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool legal = !none & ((uint32_t)(16 * i + r - lo) <= span);
          s[i][t][r] = legal ? 0.f : -INFINITY;
        }
      }
    }
  };

  // Online softmax of one block's scores, in parts that can be spread over
  // the MFMAs of the next block's K Q^T.  sm_max: block row max (v_max3 chain
  // + two permlane swaps; -inf: no legal key, and c > 0 keeps -inf * c at
  // -inf), lazy reference update (it moves only when some lane of the wave
  // needs it; the wave-uniform result tells the caller to multiply its
  // accumulators by alpha).  sm_exp(t, ih): weights 2^(s*c - m) of key tiles
  // 2ih, 2ih+1 of query tile t, rounded to bf16 in pf, summed into the row
  // sum.  A row whose reference is still -inf has only -inf scores (a legal
  // key would have moved it), so its offset is taken as 0 to give 2^-inf = 0.
  struct SoftmaxState {
    float alpha[2], mneg[2], rs[2];
    bool rebase;
  };
  auto sm_max = [&](const f32x4 (&s)[4][2], SoftmaxState& st) {
    float mb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float mx = max3f(s[0][t][0], s[0][t][1], s[0][t][2]);
      mx = max3f(mx, s[0][t][3], s[1][t][0]);
      mx = max3f(mx, s[1][t][1], s[1][t][2]);
      mx = max3f(mx, s[1][t][3], s[2][t][0]);
      mx = max3f(mx, s[2][t][1], s[2][t][2]);
      mx = max3f(mx, s[2][t][3], s[3][t][0]);
      mx = max3f(mx, s[3][t][1], s[3][t][2]);
      mx = max2f(mx, s[3][t][3]);
      mb[t] = group4_max(mx) * c;
    }
    const bool need = (mb[0] > m_run[0] + kLazyRescale) || (mb[1] > m_run[1] + kLazyRescale);
    st.rebase = __builtin_amdgcn_ballot_w64(need) != 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float mnew = st.rebase ? fmaxf(m_run[t], mb[t]) : m_run[t];
      st.alpha[t] = (mnew == -INFINITY) ? 1.f : fast_exp2(m_run[t] - mnew);
      st.mneg[t] = mnew == -INFINITY ? 0.f : -mnew;
      m_run[t] = mnew;
    }
  };
  auto sm_exp = [&](int t, int ih, f32x4 (&s)[4][2], bf16x8 (&pf)[2][2], SoftmaxState& st) {
#pragma unroll
    for (int i = 2 * ih; i < 2 * ih + 2; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(fmaf(s[i][t][r], c, st.mneg[t]));
        s[i][t][r] = e;
        st.rs[t] = (ih == 0 && i == 0 && r == 0) ? e : st.rs[t] + e;
      }
    }
    pf[t][ih] = pack_bf16x8(s[2 * ih][t], s[2 * ih + 1][t]);
  };
  auto sm_fin = [&](SoftmaxState& st) {
#pragma unroll
    for (int t = 0; t < 2; ++t) l_run[t] = fmaf(l_run[t], st.alpha[t], st.rs[t]);
  };

  // S^T = K Q^T of block jb into s (FULL: every key legal for every row, the
  // initial accumulator is the inline constant 0; otherwise mask_bias), with
  // the K fragments of k-step st + 1 read while the MFMAs of k-step st run.
  // When `cur` is given, the softmax of the previous block (scores in cur) is
  // spread over the k-steps: its row max with k-step 0, its four weight
  // groups over the others, for the compiler to interleave with the MFMAs.
  auto qk = [&](int jb, auto full_tag, f32x4 (&s)[4][2], auto with_softmax, f32x4 (&cur)[4][2],
                bf16x8 (&pf)[2][2], SoftmaxState& sm) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr bool SM = decltype(with_softmax)::value;
    const uint32_t kbase = ka0 + kstage_off(jb);
    auto kaddr = [&](int st) { return kbase ^ (uint32_t)(st << 6); };
    if constexpr (!FULL) mask_bias(jb * BN, s);
    bf16x8 ak[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ak[0][i] = lds_read_b128(kaddr(0) + 16 * i * S::KROWB);
    static_for<S::KS>([&](auto st_tag) {
      constexpr int st = decltype(st_tag)::value;
      if constexpr (st + 1 < S::KS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ak[(st + 1) & 1][i] = lds_read_b128(kaddr(st + 1) + 16 * i * S::KROWB);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x4 c0 = (FULL && st == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : s[i][t];
          s[i][t] = mfma16x16x32(ak[st & 1][i], qf[t][st], c0);
        }
      }
      if constexpr (SM) {
        if constexpr (st == 0) sm_max(cur, sm);
        static_for<4>([&](auto e_tag) {
          constexpr int e = decltype(e_tag)::value;
          if constexpr (S::KS > 1 && 1 + e * (S::KS - 1) / 4 == st) sm_exp(e >> 1, e & 1, cur, pf, sm);
        });
        if constexpr (st == S::KS - 1) sm_fin(sm);
      }
    });
  };

  // O^T += V^T P^T of block jb from V stage VST, two dv tiles per step with
  // the next step's fragments in flight.  The contraction index e of the B
  // operand maps to key 32kk + 4*g4 + e (e < 4) or 32kk + 16 + 4*g4 + e - 4,
  // the S^T register layout; the V^T fragment is read in the same order.
  auto pv = [&](auto vst_tag, const bf16x8 (&pf)[2][2]) {
    constexpr uint32_t VOFF = decltype(vst_tag)::value * S::V_TILE;
    auto read_v = [&](int kk, int j) {
      const uint32_t lo = (va0 ^ (uint32_t)(j << 5)) + VOFF + 32 * kk * S::VROWB;
      return concat_bf16x4(lds_read_tr16(lo), lds_read_tr16(lo + 16 * S::VROWB));
    };
    constexpr int NP = S::JV;  // steps of two dv tiles over both 32-key halves
    bf16x8 av[2][2];
    av[0][0] = read_v(0, 0);
    av[0][1] = read_v(0, 1);
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
        acc[j + u][0] = mfma16x16x32(av[n & 1][u], pf[0][kk], acc[j + u][0]);
        acc[j + u][1] = mfma16x16x32(av[n & 1][u], pf[1][kk], acc[j + u][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto kill = [](f32x4 (&x)[4][2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i][0] = x[i][1] = __builtin_nondeterministic_value(x[i][0]);
  };

  // One pipeline step: the softmax of block jb (scores in cur) runs while the
  // MFMA unit computes S^T of block jb + 1 (into nxt); then P.V of block jb.
  // The loads issued here (K of jb + 2, V of jb + 1) have the whole step to
  // land.
  auto step = [&](int jb, auto vst_tag, f32x4 (&cur)[4][2], f32x4 (&nxt)[4][2]) {
    constexpr int VST = decltype(vst_tag)::value;
    if (jb + 2 < jb1) issue_k(jb + 2);
    if (jb + 1 < jb1) issue_v(jb + 1, VST ^ 1);
    const bool now = wave_sees(jb);
    const bool next = jb + 1 < jb1 && wave_sees(jb + 1);
    // A step reads cur only if the wave sees block jb, and the next step reads
    // nxt only if it sees block jb + 1; telling the compiler so frees the
    // registers of a score buffer that holds nothing of use.
    if (!next) kill(nxt);
    bf16x8 pf[2][2];
    SoftmaxState sm;
    if (now) {
      if (next) {
        if (wave_full(jb + 1)) qk(jb + 1, std::true_type{}, nxt, std::true_type{}, cur, pf, sm);
        else qk(jb + 1, std::false_type{}, nxt, std::true_type{}, cur, pf, sm);
      } else {
        sm_max(cur, sm);
        sm_exp(0, 0, cur, pf, sm);
        sm_exp(0, 1, cur, pf, sm);
        sm_exp(1, 0, cur, pf, sm);
        sm_exp(1, 1, cur, pf, sm);
        sm_fin(sm);
      }
      if (sm.rebase) {
#pragma unroll
        for (int j = 0; j < S::JV; ++j) {
          acc[j][0] *= sm.alpha[0];
          acc[j][1] *= sm.alpha[1];
        }
      }
      pv(vst_tag, pf);
    } else if (next) {
      if (wave_full(jb + 1)) qk(jb + 1, std::true_type{}, nxt, std::false_type{}, cur, pf, sm);
      else qk(jb + 1, std::false_type{}, nxt, std::false_type{}, cur, pf, sm);
    }
    kill(cur);
    // K of jb + 2 and V of jb + 1 have landed for every wave, and every wave
    // is done with the stages they overwrite next step.
    wait_vmcnt<0>();
    __syncthreads();
  };

  f32x4 s0[4][2], s1[4][2];
  if (jb0 < jb1) {
    issue_k(jb0);
    issue_v(jb0, 0);
    if (jb0 + 1 < jb1) issue_k(jb0 + 1);
    wait_vmcnt<0>();
    __syncthreads();
    if (wave_sees(jb0)) {
      bf16x8 pf[2][2];
      SoftmaxState sm;
      if (wave_full(jb0)) qk(jb0, std::true_type{}, s0, std::false_type{}, s1, pf, sm);
      else qk(jb0, std::false_type{}, s0, std::false_type{}, s1, pf, sm);
    }
  }
  // Unrolled by two: the score buffers swap roles and the V stage is a
  // compile-time constant in each half.
  for (int jb = jb0; jb < jb1; jb += 2) {
    step(jb, std::integral_constant<int, 0>{}, s0, s1);
    if (jb + 1 < jb1) step(jb + 1, std::integral_constant<int, 1>{}, s1, s0);
  }

  if (!wave_has_rows) return;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float lt = group4_sum(l_run[t]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int row = qw0 + 16 * t + l16;
    if (row < p.Q) {
#pragma unroll
      for (int j = 0; j < S::JV; ++j) {
        const int dv = 16 * j + 4 * g4;
        if (dv < Dv) {
          bf16x4 ov;
          ov[0] = (__bf16)(acc[j][t][0] * inv);
          ov[1] = (__bf16)(acc[j][t][1] * inv);
          ov[2] = (__bf16)(acc[j][t][2] * inv);
          ov[3] = (__bf16)(acc[j][t][3] * inv);
          *reinterpret_cast<bf16x4*>(og + (int64_t)row * Dv + dv) = ov;
        }
      }
      if (g4 == 0) lg[row] = lt > 0.f ? (m_run[t] + __log2f(lt)) * 0.69314718055994530942f : -INFINITY;
    }
  }
}

template <int DP, int DVP>
static hipError_t launch_prefill_t(const Params& p, hipStream_t stream) {
  const int n_qt = (p.Q + kPrefillBM - 1) / kPrefillBM;
  const dim3 grid((unsigned)((int64_t)n_qt * p.Hq * p.B));
  Params arg = p;
  void* args[] = {&arg};
  const void* fn = (p.D == DP && p.Dv == DVP) ? reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, true>)
                                              : reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP, false>);
  return hipLaunchKernel(fn, grid, dim3(256), args, 0, stream);
}

hipError_t launch_prefill_bf16(const Params& p, hipStream_t stream) {
  const int dp = pad_width(p.D), dvp = pad_width(p.Dv);
  if (dp == 64 && dvp == 64) return launch_prefill_t<64, 64>(p, stream);
  if (dp == 64 && dvp == 128) return launch_prefill_t<64, 128>(p, stream);
  if (dp == 128 && dvp == 64) return launch_prefill_t<128, 64>(p, stream);
  return launch_prefill_t<128, 128>(p, stream);
}

}  // namespace attn
