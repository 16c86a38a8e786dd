// bf16 prefill kernel for gfx950: causal GQA attention forward with online
// softmax (LuisaCompute "Attention execution mapping" review, section 1: the
// fixture's bottom-right causal GQA and the (row_max, row_sum, acc) state
// carried across KV blocks; section 2: the phase graph load Q -> per KV block
// load K/V -> QK -> mask -> max/exp/sum -> rescale -> PV -> update).
//
// Mapping on CDNA4:
//   * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//     owns 32 rows as two 16-column MFMA tiles, Q held in registers; two
//     workgroups share a CU, so one's softmax overlaps the other's MFMAs;
//   * K/V blocks of 64 keys go HBM -> LDS by direct buffer loads into a
//     two-stage ring: block j+1 is in flight while block j is computed, one
//     barrier per block; rows past K_b and channels past D read as zero from
//     the buffer range check;
//   * tiles are XOR-swizzled in LDS so the 16-byte K fragment reads and the
//     transposed V reads are free of bank conflicts;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16, so each lane holds 16 keys of
//     one query column and the row max/sum is in-lane plus two permlane swaps;
//   * P^T stays in the S^T register layout and feeds O^T = V^T P^T directly;
//     V^T fragments come from row-major LDS through ds_read_b64_tr_b16;
//   * masks are evaluated only on blocks that straddle the causal diagonal, a
//     window edge or the sequence end; blocks no row of a wave can see are
//     skipped by that wave;
//   * tiles are ordered heaviest causal tile first, and the (batch, kv-head)
//     groups are dealt to the 8 XCDs so the query heads sharing a kv-head run
//     on one XCD and reuse its L2.
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
  static constexpr int STAGE = K_TILE + V_TILE;
  static constexpr int K_LOADS = K_TILE / 4096;  // 16-byte loads per thread per block
  static constexpr int V_LOADS = V_TILE / 4096;
  static_assert(K_TILE % 4096 == 0 && V_TILE % 4096 == 0, "load split");
};

// Block index -> (query tile, batch, head).  When the (batch, kv-head) groups
// divide evenly over the 8 XCDs (workgroup i runs on XCD i % 8), each XCD gets
// whole groups and walks their query tiles heaviest first; otherwise the
// order is heaviest tile first with heads fastest.
__device__ __forceinline__ void prefill_tile(const Params& p, int n_qt, int* qt, int* b, int* h) {
  const int x = blockIdx.x;
  const int groups = p.B * p.Hkv;
  if ((groups & 7) == 0) {
    const int xcd = x & 7, slot = x >> 3;
    const int per_qt = (groups >> 3) * p.group;
    const int qrank = slot / per_qt, rem = slot - qrank * per_qt;
    const int grp = (rem / p.group) * 8 + xcd;
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

template <int DP, int DVP>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(Params p) {
  using S = PrefillShape<DP, DVP>;
  constexpr int BN = kPrefillBN;
  __shared__ __attribute__((aligned(16))) unsigned char ring[2 * S::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.Hq + h) * p.Q * p.D;
  const rsrc_t krs = slice_rsrc(static_cast<const uint16_t*>(p.k) + kv_slice * p.K * p.D, (uint32_t)Kb * p.D * 2);
  const rsrc_t vrs = slice_rsrc(static_cast<const uint16_t*>(p.v) + kv_slice * p.K * p.Dv, (uint32_t)Kb * p.Dv * 2);
  uint16_t* og = static_cast<uint16_t*>(p.o) + ((int64_t)b * p.Hq + h) * p.Q * p.Dv;
  float* lg = p.lse + ((int64_t)b * p.Hq + h) * p.Q;
  const int dch = p.D / 8, dvch = p.Dv / 8;

  const int qw0 = q0 + wave * kPrefillRowsPerWave;
  const bool wave_has_rows = qw0 < p.Q;
  const int qw_last = min(qw0 + kPrefillRowsPerWave, p.Q) - 1;
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
      uint4 u = (row < p.Q && col < p.D) ? load_u4(qg + (int64_t)row * p.D + col) : zero_u4();
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

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4 acc[S::JV][2];
#pragma unroll
  for (int j = 0; j < S::JV; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Direct loads of block jb into ring stage `stg`: each wave-wide load fills
  // 1 KiB of the tile; lane l's 16 bytes land at position l of it, so the lane
  // fetches the global chunk that the swizzle places there.
  const uint32_t ring_base = lds_offset(ring);
  auto issue = [&](int jb, int stg) {
    const int kb0 = jb * BN;
    const uint32_t kbase = ring_base + stg * S::STAGE;
#pragma unroll
    for (int i = 0; i < S::K_LOADS; ++i) {
      const int byte0 = (i * kPrefillWaves + wave) * 1024;
      const int off = byte0 + 16 * lane;
      const int row = off / S::KROWB, ch = ((off % S::KROWB) >> 4) ^ swz_k<S::KCH>(row);
      const uint32_t vo = ch < dch ? ((uint32_t)(kb0 + row) * p.D + ch * 8) * 2 : kOutOfRange;
      load_lds16(krs, kbase + __builtin_amdgcn_readfirstlane(byte0), vo);
    }
    const uint32_t vbase = kbase + S::K_TILE;
#pragma unroll
    for (int i = 0; i < S::V_LOADS; ++i) {
      const int byte0 = (i * kPrefillWaves + wave) * 1024;
      const int off = byte0 + 16 * lane;
      const int row = off / S::VROWB, ch = ((off % S::VROWB) >> 4) ^ swz_v<S::VCH>(row);
      const uint32_t vo = ch < dvch ? ((uint32_t)(kb0 + row) * p.Dv + ch * 8) * 2 : kOutOfRange;
      load_lds16(vrs, vbase + __builtin_amdgcn_readfirstlane(byte0), vo);
    }
  };

  if (jb0 < jb1) issue(jb0, 0);
  wait_vmcnt<0>();
  __syncthreads();

  for (int jb = jb0; jb < jb1; ++jb) {
    const int stg = (jb - jb0) & 1;
    if (jb + 1 < jb1) issue(jb + 1, stg ^ 1);
    const unsigned char* kst = ring + stg * S::STAGE;
    const unsigned char* vst = kst + S::K_TILE;
    const int kb0 = jb * BN;
    const int pw_first = qw0 + delta, pw_last = qw_last + delta;
    const bool skip = !wave_has_rows || kb0 > pw_last || kb0 >= Kb || (W > 0 && kb0 + BN - 1 < pw_first - W + 1);
    if (!skip) {
      const bool full = (kb0 + BN - 1 <= pw_first) && (kb0 + BN <= Kb) && (W <= 0 || kb0 >= pw_last - W + 1);
      f32x4 sacc[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[i][0] = sacc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S::KS; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * i + l16;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              kst + row * S::KROWB + (((4 * s + g4) ^ swz_k<S::KCH>(row)) << 4));
          sacc[i][0] = mfma16x16x32(a, qf[0][s], sacc[i][0]);
          sacc[i][1] = mfma16x16x32(a, qf[1][s], sacc[i][1]);
        }
      }
      if (!full) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int pq = qw0 + 16 * t + l16 + delta;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = kb0 + 16 * i + 4 * g4 + r;
              const bool legal = key <= pq && key < Kb && (W <= 0 || key > pq - W);
              if (!legal) sacc[i][t][r] = -INFINITY;
            }
          }
        }
      }
      bf16x8 pf[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float mx = sacc[0][t][0];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[i][t][r]);
        mx = group4_max(mx);
        const float mb = (mx == -INFINITY) ? -INFINITY : mx * c;
        float alpha;
        if (softmax_rebase(m_run[t], mb, alpha)) {
          l_run[t] *= alpha;
#pragma unroll
          for (int j = 0; j < S::JV; ++j) acc[j][t] *= alpha;
        }
        const float mref = m_run[t];
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sv = sacc[i][t][r];
            float e = fast_exp2(fmaf(sv, c, -mref));
            if (!full) e = (sv == -INFINITY) ? 0.f : e;
            sacc[i][t][r] = e;
            rs += e;
          }
        }
        l_run[t] += rs;
        pf[t][0] = pack_bf16x8(sacc[0][t], sacc[1][t]);
        pf[t][1] = pack_bf16x8(sacc[2][t], sacc[3][t]);
      }
      // O^T += V^T P^T over two 32-key halves.  The contraction index e of the
      // B operand maps to key 32kk + 4*g4 + e (e < 4) or 32kk + 16 + 4*g4 + e - 4,
      // the S^T register layout; the V^T fragment is read in the same order.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int row = 32 * kk + 4 * g4 + (l16 >> 2);
#pragma unroll
        for (int j = 0; j < S::JV; ++j) {
          const int ch = 2 * j + ((l16 & 3) >> 1), half = (l16 & 1) * 8;
          const unsigned char* lo = vst + row * S::VROWB + ((ch ^ swz_v<S::VCH>(row)) << 4) + half;
          const unsigned char* hi = vst + (row + 16) * S::VROWB + ((ch ^ swz_v<S::VCH>(row + 16)) << 4) + half;
          const bf16x8 va = concat_bf16x4(lds_read_tr16(reinterpret_cast<const uint16_t*>(lo)),
                                          lds_read_tr16(reinterpret_cast<const uint16_t*>(hi)));
          acc[j][0] = mfma16x16x32(va, pf[0][kk], acc[j][0]);
          acc[j][1] = mfma16x16x32(va, pf[1][kk], acc[j][1]);
        }
      }
    }
    // Block jb+1 has landed for every wave, and every wave is done with stage stg.
    wait_vmcnt<0>();
    __syncthreads();
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
        if (dv < p.Dv) {
          bf16x4 ov;
          ov[0] = (__bf16)(acc[j][t][0] * inv);
          ov[1] = (__bf16)(acc[j][t][1] * inv);
          ov[2] = (__bf16)(acc[j][t][2] * inv);
          ov[3] = (__bf16)(acc[j][t][3] * inv);
          *reinterpret_cast<bf16x4*>(og + (int64_t)row * p.Dv + dv) = ov;
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
  return hipLaunchKernel(reinterpret_cast<const void*>(&prefill_bf16_kernel<DP, DVP>), grid, dim3(256), args, 0,
                         stream);
}

hipError_t launch_prefill_bf16(const Params& p, hipStream_t stream) {
  const int dp = pad_width(p.D), dvp = pad_width(p.Dv);
  if (dp == 64 && dvp == 64) return launch_prefill_t<64, 64>(p, stream);
  if (dp == 64 && dvp == 128) return launch_prefill_t<64, 128>(p, stream);
  if (dp == 128 && dvp == 64) return launch_prefill_t<128, 64>(p, stream);
  return launch_prefill_t<128, 128>(p, stream);
}

}  // namespace attn
