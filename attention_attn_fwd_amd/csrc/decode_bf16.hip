// Split-KV decode on gfx950 (short query runs: up to 32 packed rows g*Q for
// heads up to 128 channels, up to 16 for heads up to 256), plus the
// log-sum-exp combine pass.
//
// The recurrence is the one of the LuisaCompute "Attention execution mapping"
// review, section 1 (online (row_max, row_sum, acc) carried across KV
// blocks); section 5 notes that splitting a long KV range needs a legal merge
// of that state, which is what the combine pass does, and that one kv-head
// serves Hq/Hkv query heads; section 4 notes that a single query row cannot
// fill a matrix atom.  Hence:
//   * the g*Q query rows of a (batch, kv-head) group are packed as the 16-wide
//     N side of v_mfma_f32_16x16x32_bf16 and keys are the M side, so K and V
//     are read from HBM once per group;
//   * the work is cut stream-K fashion: every group's legal key range is a
//     run of 32-key sub-blocks, the runs of all groups are laid end to end,
//     and each of a fixed number of single-wave workers takes an equal
//     contiguous share.  A worker streams its share without a break, across
//     group boundaries, so all workers finish together and no worker waits
//     for a dispatch: with one workgroup per fixed-size chunk, a batch of
//     uneven lengths left the GPU half idle for the last third of the pass;
//   * a worker streams through a two-stage LDS ring of sub-blocks filled by
//     direct buffer-to-LDS loads (K and V with the non-temporal hint: each
//     byte is read once); the sub-block that opens a group in the
//     worker's share also carries that group's Q rows in its stage, so the Q
//     of the next group arrives in order with its keys; rows past K_b and
//     channels past D read as zero from the buffer range check;
//   * a worker writes one fp32 partial (m, l, acc[Dv]) per row for each group
//     piece it processed, at partial slot (group + worker): the pieces of
//     group g come from workers first(g)..last(g), so slots g + w never
//     collide and there are at most groups + workers of them;
//   * the combine pass recomputes the same partition and merges a row's
//     partials in worker order, so results are bitwise reproducible (no
//     atomics).
#include "attn_internal.h"

namespace attn {

template <int DP, int DVP, int NT>
struct DecodeShape {
  static constexpr int KS = DP / 32;
  static constexpr int JV = DVP / 16;
  static constexpr int KCH = DP / 8;            // 16-byte chunks per K row
  static constexpr int VCH = DVP / 8;
  static constexpr int KROWB = DP * 2;          // LDS bytes per K (and Q) row
  static constexpr int VROWB = DVP * 2;
  static constexpr int K_STAGE = kDecodeSub * KROWB;
  static constexpr int V_STAGE = kDecodeSub * VROWB;
  static constexpr int QROWS = 16 * NT;         // packed query rows (N side)
  static constexpr int Q_STAGE = QROWS * KROWB;
  static constexpr int STAGE = K_STAGE + V_STAGE + Q_STAGE;
  static constexpr int K_LOADS = K_STAGE / 1024;  // wave-wide 1 KiB loads per stage
  static constexpr int V_LOADS = V_STAGE / 1024;
  static constexpr int Q_LOADS = Q_STAGE / 1024;
  static constexpr int LOADS = K_LOADS + V_LOADS;
  static_assert(Q_STAGE % 1024 == 0 && Q_LOADS <= K_LOADS, "Q tile uses the first K load offsets");
};

// Union of the legal key ranges of all rows of one (batch, kv-head) group,
// widened down to a sub-block boundary: [lo, hi).  Row q's position is
// q + K_b - Q, so the first row bounds the window from below and the sequence
// end bounds everything from above.  Sub-blocks start at multiples of 32
// keys, so none straddles a page of a paged cache; keys below the window
// are masked like any other.
__device__ __forceinline__ void group_key_range(int Kb, int Q, int W, int* lo, int* hi) {
  *hi = Kb;
  *lo = (W > 0 ? max(0, Kb - Q - W + 1) : 0) & ~(kDecodeSub - 1);
}

// A sequence's groups: key range [lo, hi) with hi = K_b, and nsb sub-blocks.
struct SeqRange {
  int lo, hi, nsb;
};
__device__ __forceinline__ SeqRange seq_range(const Params& p, int b) {
  const int Kb = clamp_len(p.seqlens, b, p.K);
  int lo, hi;
  group_key_range(Kb, p.Q, p.window, &lo, &hi);
  return SeqRange{lo, hi, hi > lo ? (hi - lo + kDecodeSub - 1) / kDecodeSub : 0};
}

// Sub-blocks of sequence b (all its kv-head groups) as the lane's value of a
// wave-wide pass over sequences b0 + lane.
__device__ __forceinline__ int64_t seq_subblocks(const Params& p, int b) {
  return b < p.B ? (int64_t)seq_range(p, b).nsb * p.Hkv : 0;
}

// A wave-uniform 64-bit value the compiler can keep in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t u = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t wave_incl_scan(int64_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Total sub-blocks over all groups (wave-uniform).
__device__ __forceinline__ int64_t total_subblocks(const Params& p, int lane) {
  int64_t tot = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) tot += __shfl(wave_incl_scan(seq_subblocks(p, b0 + lane), lane), 63);
  return uniform64(tot);
}

// First global sub-block of sequence b's groups (sum over earlier sequences).
__device__ __forceinline__ int64_t seq_base(const Params& p, int b, int lane) {
  int64_t base = 0;
  for (int b0 = 0; b0 < b; b0 += 64) {
    const int bb = b0 + lane;
    base += __shfl(wave_incl_scan(bb < b ? seq_subblocks(p, bb) : 0, lane), 63);
  }
  return uniform64(base);
}

// Per-row share of the stream-K partition: sub-blocks per worker.
__device__ __forceinline__ int64_t worker_share(int64_t total, int workers) {
  return (total + workers - 1) / workers;
}

// Position of one sub-block in the partition (wave-uniform; the fields are
// passed through readfirstlane so descriptors built from them are scalar).
struct Cursor {
  int b, kh, sb;  // sequence, kv-head, sub-block within the group
  int nsb, lo, Kb;
};
__device__ __forceinline__ void make_uniform(Cursor& c) {
  c.b = __builtin_amdgcn_readfirstlane(c.b);
  c.kh = __builtin_amdgcn_readfirstlane(c.kh);
  c.sb = __builtin_amdgcn_readfirstlane(c.sb);
  c.nsb = __builtin_amdgcn_readfirstlane(c.nsb);
  c.lo = __builtin_amdgcn_readfirstlane(c.lo);
  c.Kb = __builtin_amdgcn_readfirstlane(c.Kb);
}

template <int DP, int DVP, int NT, bool F16>
__global__ __launch_bounds__(64) void decode_split_kernel(Params p) {
  using S = DecodeShape<DP, DVP, NT>;
  using E = Elem<F16>;
  __shared__ __attribute__((aligned(16))) unsigned char ring[2 * S::STAGE];

  const int lane = threadIdx.x;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int w = blockIdx.x;

  const int64_t T = total_subblocks(p, lane);
  const int64_t per = worker_share(T, p.n_workers);
  const int64_t s0 = (int64_t)w * per;
  const int64_t s1 = min(T, s0 + per);
  if (s0 >= s1) return;
  const int n = (int)(s1 - s0);

  // Cursor of global sub-block s0.
  Cursor start;
  {
    int64_t run = 0;
    for (int b0 = 0;; b0 += 64) {
      const int64_t cnt = seq_subblocks(p, b0 + lane);
      const int64_t incl = wave_incl_scan(cnt, lane);
      const int64_t tot = uniform64(__shfl(incl, 63));
      if (s0 < run + tot) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(run + incl > s0);
        const int first = __builtin_ctzll(m);
        const int b = b0 + first;
        const int64_t base = uniform64(run + __shfl(incl - cnt, first));
        const SeqRange r = seq_range(p, b);
        const int64_t off = s0 - base;
        start = Cursor{b, (int)(off / r.nsb), (int)(off % r.nsb), r.nsb, r.lo, r.hi};
        make_uniform(start);
        break;
      }
      run += tot;
    }
  }
  // Next sub-block of the partition (only called while one exists).
  auto advance = [&](Cursor& c) {
    if (++c.sb < c.nsb) return;
    c.sb = 0;
    if (++c.kh < p.Hkv) return;
    c.kh = 0;
    SeqRange r;
    do {
      ++c.b;
      r = seq_range(p, c.b);
    } while (r.nsb == 0);
    c.nsb = r.nsb;
    c.lo = r.lo;
    c.Kb = r.hi;
    make_uniform(c);
  };

  // This lane's byte offset, from the start of a sub-block, for each 1 KiB
  // direct load of a stage: load i fills tile bytes [1024 i, 1024 i + 1024),
  // lane l position l of it, which holds chunk (position ^ swizzle) of its row.
  // Chunks past D (Dv) get an offset beyond any buffer and read as zero.  The
  // Q tile has the K tile's layout, so it uses the first Q_LOADS K offsets.
  uint32_t koff[S::K_LOADS], voff[S::V_LOADS];
#pragma unroll
  for (int i = 0; i < S::K_LOADS; ++i) {
    const int off = i * 1024 + 16 * lane;
    const int row = off / S::KROWB, ch = ((off % S::KROWB) >> 4) ^ swz_k<S::KCH>(row);
    koff[i] = ch < p.D / 8 ? (uint32_t)(row * p.D + ch * 8) * 2 : kOutOfRange;
  }
#pragma unroll
  for (int i = 0; i < S::V_LOADS; ++i) {
    const int off = i * 1024 + 16 * lane;
    const int row = off / S::VROWB, ch = ((off % S::VROWB) >> 4) ^ swz_v<S::VCH>(row);
    voff[i] = ch < p.Dv / 8 ? (uint32_t)(row * p.Dv + ch * 8) * 2 : kOutOfRange;
  }

  const int R = p.rows;
  const uint32_t ring0 = lds_offset(ring);
  // Loads of the sub-block at cursor c into stage stg; with_q adds the Q rows
  // of c's group (rows past R read as zero).
  // `page`: the page holding the sub-block's keys when the cache is paged.
  auto issue = [&](const Cursor& c, int stg, bool with_q, int page) {
    const int kb0 = c.lo + c.sb * kDecodeSub;
    const KvSpan sp = kv_span(p, c.b, c.kh, kb0, page);
    const uint32_t rows_left = (uint32_t)min(c.Kb - kb0, sp.rows);
    const rsrc_t krs = slice_rsrc(sp.k, rows_left * p.D * 2);
    const rsrc_t vrs = slice_rsrc(sp.v, rows_left * p.Dv * 2);
    const uint32_t st = ring0 + stg * S::STAGE;
#pragma unroll
    for (int i = 0; i < S::K_LOADS; ++i) load_lds16_nt(krs, st + i * 1024, koff[i]);
#pragma unroll
    for (int i = 0; i < S::V_LOADS; ++i) load_lds16_nt(vrs, st + S::K_STAGE + i * 1024, voff[i]);
    if (with_q) {
      const rsrc_t qrs = slice_rsrc(
          static_cast<const uint16_t*>(p.q) + ((int64_t)c.b * p.Hq + c.kh * p.group) * p.Q * p.D, (uint32_t)R * p.D * 2);
#pragma unroll
      for (int i = 0; i < S::Q_LOADS; ++i) load_lds16(qrs, st + S::K_STAGE + S::V_STAGE + i * 1024, koff[i]);
    }
  };

  const float c = p.scale_log2;
  const uint32_t qx = p.q_sign ? 0x80008000u : 0u;
  const int W = p.window, Qn = p.Q;

  bf16x8 qf[NT][S::KS];
  float m_run[NT], l_run[NT];
  f32x4 acc[S::JV][NT];

  // Prologue: the first two sub-blocks; each stage remembers whether it
  // carries Q (a group opens there), which fixes its number of loads.
  Cursor cc = start, ic = start;
  bool stage_q[2] = {false, false};
  auto page_of = [&](const Cursor& c) {
    return __builtin_amdgcn_readfirstlane(kv_page(p, c.b, c.lo + c.sb * kDecodeSub));
  };
  issue(ic, 0, true, page_of(ic));
  stage_q[0] = true;
  if (n > 1) {
    advance(ic);
    stage_q[1] = ic.sb == 0;
    issue(ic, 1, stage_q[1], page_of(ic));
  }

  int stg = 0;
  for (int j = 0; j < n; ++j) {
    // Sub-block j's loads have landed; those of j + 1 may stay in flight.
    if (j + 1 < n) {
      if (stage_q[stg ^ 1]) wait_vmcnt<S::LOADS + S::Q_LOADS>();
      else wait_vmcnt<S::LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    const unsigned char* kst = ring + stg * S::STAGE;
    const unsigned char* vst = kst + S::K_STAGE;
    const bool opens = stage_q[stg];  // first sub-block of a group in this share
    const int Kb = cc.Kb, delta = row_delta(Kb, Qn, p.causal_shift);
    const int kb0 = cc.lo + cc.sb * kDecodeSub;

    if (opens) {
      // Q^T fragments from the stage's Q tile: N column l16 of tile t is
      // packed row 16t + l16 = hh*Q + q of the group.
      const unsigned char* qst = vst + S::V_STAGE;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int row = 16 * t + l16;
#pragma unroll
        for (int s = 0; s < S::KS; ++s) {
          uint4 u = *reinterpret_cast<const uint4*>(qst + row * S::KROWB + (((4 * s + g4) ^ swz_k<S::KCH>(row)) << 4));
          u.x ^= qx; u.y ^= qx; u.z ^= qx; u.w ^= qx;
          qf[t][s] = __builtin_bit_cast(bf16x8, u);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
#pragma unroll
        for (int jv = 0; jv < S::JV; ++jv) acc[jv][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

    // Every LDS read of the sub-block is issued up front (K fragments, then the
    // transposed V fragments), so a single wave pays the LDS latency once per
    // step rather than once per fragment; the V reads overlap QK and softmax.
    // Heads wider than 128: the V fragments are read after the softmax, once
    // the K fragments are dead (both sets at once would not fit the registers).
    constexpr bool kLateV = DP > 128 || DVP > 128;
    bf16x8 kf[2][S::KS];
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 16 * i + l16;
        kf[i][s] = *reinterpret_cast<const bf16x8*>(kst + row * S::KROWB + (((4 * s + g4) ^ swz_k<S::KCH>(row)) << 4));
      }
    }
    // V^T fragments: contraction index e maps to key 4*g4 + e (e < 4) or
    // 16 + 4*g4 + e - 4, the S^T register layout; each is two transposed reads
    // of 4-row pieces of the swizzled V tile.
    bf16x8 vf[S::JV];
    if constexpr (!kLateV) {
#pragma unroll
      for (int jv = 0; jv < S::JV; ++jv) {
        const int row = 4 * g4 + (l16 >> 2);
        const int ch = 2 * jv + ((l16 & 3) >> 1), half = (l16 & 1) * 8;
        const unsigned char* lo = vst + row * S::VROWB + ((ch ^ swz_v<S::VCH>(row)) << 4) + half;
        const unsigned char* hi = vst + (row + 16) * S::VROWB + ((ch ^ swz_v<S::VCH>(row + 16)) << 4) + half;
        vf[jv] = concat_bf16x4(lds_read_tr16(reinterpret_cast<const uint16_t*>(lo)),
                               lds_read_tr16(reinterpret_cast<const uint16_t*>(hi)));
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x4 sacc[2][NT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) sacc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S::KS; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) sacc[i][t] = E::mfma(kf[i][s], qf[t][s], sacc[i][t]);
    // Every row sees keys <= K_b - Q causally; the last row's window starts at K_b - W.
    const bool full = (kb0 + kDecodeSub - 1 <= delta) && (kb0 + kDecodeSub <= Kb) && (W <= 0 || kb0 >= Kb - W);
    if (!full) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int pq = (16 * t + l16) % Qn + delta;  // absolute position of packed row
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kb0 + 16 * i + 4 * g4 + r;
            const bool legal = (key <= pq) & (key < Kb) & ((W <= 0) | (key > pq - W));
            if (!legal) sacc[i][t][r] = -INFINITY;
          }
        }
      }
    }
    bf16x8 pf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float mx = max3f(sacc[0][t][0], sacc[0][t][1], sacc[0][t][2]);
      mx = max3f(mx, sacc[0][t][3], sacc[1][t][0]);
      mx = max3f(mx, sacc[1][t][1], sacc[1][t][2]);
      mx = max2f(mx, sacc[1][t][3]);
      mx = group4_max(mx);
      const float mb = (mx == -INFINITY) ? -INFINITY : mx * c;
      float alpha;
      if (softmax_rebase(m_run[t], mb, alpha)) {
        l_run[t] *= alpha;
#pragma unroll
        for (int jv = 0; jv < S::JV; ++jv) acc[jv][t] *= alpha;
      }
      const float mneg = m_run[t] == -INFINITY ? 0.f : -m_run[t];
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = fast_exp2(fmaf(sacc[i][t][r], c, mneg));
          sacc[i][t][r] = e;
          rs += e;
        }
      }
      l_run[t] += rs;
      pf[t] = E::pack(sacc[0][t], sacc[1][t]);
    }
    // O^T += V^T P^T.
    if constexpr (kLateV) {
#pragma unroll
      for (int jv = 0; jv < S::JV; ++jv) {
        const int row = 4 * g4 + (l16 >> 2);
        const int ch = 2 * jv + ((l16 & 3) >> 1), half = (l16 & 1) * 8;
        const unsigned char* lo = vst + row * S::VROWB + ((ch ^ swz_v<S::VCH>(row)) << 4) + half;
        const unsigned char* hi = vst + (row + 16) * S::VROWB + ((ch ^ swz_v<S::VCH>(row + 16)) << 4) + half;
        vf[jv] = concat_bf16x4(lds_read_tr16(reinterpret_cast<const uint16_t*>(lo)),
                               lds_read_tr16(reinterpret_cast<const uint16_t*>(hi)));
      }
    }
#pragma unroll
    for (int jv = 0; jv < S::JV; ++jv)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[jv][t] = E::mfma(vf[jv], pf[t], acc[jv][t]);

    // The stage is free once its LDS reads have returned: refill it with
    // sub-block j + 2.
    if (j + 2 < n) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      advance(ic);
      stage_q[stg] = ic.sb == 0;
      issue(ic, stg, stage_q[stg], page_of(ic));
    }

    // The piece of the group ends with its last sub-block or the share's.
    if (cc.sb == cc.nsb - 1 || j == n - 1) {
      const int64_t slot = (int64_t)cc.b * p.Hkv + cc.kh + w;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float lt = group4_sum(l_run[t]);
        const int rr = 16 * t + l16;
        if (rr < R) {
          const int64_t part = slot * R + rr;
          if (g4 == 0) {
            p.ws_m[part] = m_run[t];
            p.ws_l[part] = lt;
          }
#pragma unroll
          for (int jv = 0; jv < S::JV; ++jv) {
            const int dv = 16 * jv + 4 * g4;
            if (dv < p.Dv) *reinterpret_cast<f32x4*>(p.ws_acc + part * p.Dv + dv) = acc[jv][t];
          }
        }
      }
    }
    if (j + 1 < n) advance(cc);
    stg ^= 1;
  }
}

// One wave per output row (b, h, q): merge the row's partials in worker
// order.  The pieces of group g were made by workers first..last of the same
// partition (recomputed here) and sit at slots g + w.  Pieces are taken eight
// at a time: every lane loads the eight pieces' (m, l) (the same addresses in
// every lane) and its NC dv columns of each (lane + 64c), all in one round of
// loads, and folds them into a running (M, L, o) that is rescaled when M
// moves, so a row with at most eight pieces costs one round trip to memory.
template <int NC>
__global__ __launch_bounds__(256) void decode_combine_kernel(Params p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row_id = (int64_t)blockIdx.x * 4 + wave;
  const int64_t total = (int64_t)p.B * p.Hq * p.Q;
  if (row_id >= total) return;
  const int qi = (int)(row_id % p.Q);
  const int h = (int)((row_id / p.Q) % p.Hq);
  const int b = (int)(row_id / ((int64_t)p.Q * p.Hq));
  const int kh = h / p.group;
  const int rr = (h - kh * p.group) * p.Q + qi;
  const int R = p.rows;
  const int64_t g = (int64_t)b * p.Hkv + kh;

  int w_first = 0, w_last = -1;
  if (p.n_workers > 0 && p.K > 0) {
    const SeqRange r = seq_range(p, b);
    if (r.nsb > 0) {
      const int64_t T = total_subblocks(p, lane);
      const int64_t per = worker_share(T, p.n_workers);
      const int64_t G = seq_base(p, b, lane) + (int64_t)kh * r.nsb;
      w_first = (int)(G / per);
      w_last = (int)((G + r.nsb - 1) / per);
    }
  }

  // Running merge; a piece with no legal key for this row has m = -inf and
  // contributes nothing.
  float M = -INFINITY, L = 0.f, o[NC] = {};
  constexpr int U = 8;
  for (int w0 = w_first; w0 <= w_last; w0 += U) {
    float m[U], l[U], a[U][NC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = w0 + u <= w_last;
      const int64_t sp = (g + w0 + u) * R + rr;
      const float* ap = p.ws_acc + sp * p.Dv;
      m[u] = ok ? p.ws_m[sp] : -INFINITY;
      l[u] = ok ? p.ws_l[sp] : 0.f;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) a[u][cc] = ok && lane + 64 * cc < p.Dv ? ap[lane + 64 * cc] : 0.f;
    }
    float mc = m[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mc = fmaxf(mc, m[u]);
    if (mc == -INFINITY) continue;
    const float mn = fmaxf(M, mc);
    const float alpha = M == -INFINITY ? 0.f : fast_exp2(M - mn);
    L *= alpha;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) o[cc] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = m[u] == -INFINITY ? 0.f : fast_exp2(m[u] - mn);
      L = fmaf(l[u], f, L);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) o[cc] = fmaf(a[u][cc], f, o[cc]);
    }
    M = mn;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(p.o) + row_id * p.Dv;
  auto cvt = [&](float x) { return p.f16 ? Elem<true>::cvt(x) : Elem<false>::cvt(x); };
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
    if (lane + 64 * cc < p.Dv) orow[lane + 64 * cc] = cvt(o[cc] * inv);
  if (lane == 0) p.lse[row_id] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

template <int DP, int DVP, int NT>
static hipError_t launch_decode_t(const Params& p, hipStream_t stream) {
  Params arg = p;
  void* args[] = {&arg};
  // With K == 0 there is nothing to split: the combine pass alone writes 0 / -inf.
  if (p.n_workers > 0) {
    const void* fn = p.f16 ? reinterpret_cast<const void*>(&decode_split_kernel<DP, DVP, NT, true>)
                           : reinterpret_cast<const void*>(&decode_split_kernel<DP, DVP, NT, false>);
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p.n_workers), dim3(64), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t rows = (int64_t)p.B * p.Hq * p.Q;
  const dim3 cgrid((unsigned)((rows + 3) / 4));
  constexpr int NC = DVP <= 128 ? 2 : 4;
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_combine_kernel<NC>), cgrid, dim3(256), args, 0,
                         stream);
}

template <int DP, int DVP>
static hipError_t launch_decode_nt(const Params& p, hipStream_t stream) {
  if (p.rows <= 16) return launch_decode_t<DP, DVP, 1>(p, stream);
  return launch_decode_t<DP, DVP, 2>(p, stream);
}

// Heads up to 128 on kernels sized for them; up to 256 (padded to 256 on both
// sides) for at most 16 packed rows (the plan sends more to the prefill kernel).
hipError_t launch_decode_bf16(const Params& p, hipStream_t stream) {
  const int dp = pad_width(p.D), dvp = pad_width(p.Dv);
  if (dp > 128 || dvp > 128) return launch_decode_t<256, 256, 1>(p, stream);
  if (dp == 64 && dvp == 64) return launch_decode_nt<64, 64>(p, stream);
  if (dp == 64 && dvp == 128) return launch_decode_nt<64, 128>(p, stream);
  if (dp == 128 && dvp == 64) return launch_decode_nt<128, 64>(p, stream);
  return launch_decode_nt<128, 128>(p, stream);
}

}  // namespace attn
