// Split-KV decode for Q = 1..4 on gfx950, plus the log-sum-exp combine pass.
//
// The recurrence is the one of the LuisaCompute "Attention execution mapping"
// review, section 1 (online (row_max, row_sum, acc) carried across KV
// blocks); section 5 notes that splitting a long KV range needs a legal merge
// of that state, which is what the combine pass does, and that one kv-head
// serves Hq/Hkv query heads; section 4 notes that a single query row cannot
// fill a matrix atom.  Hence:
//   * one single-wave workgroup per (chunk of keys, kv-head, batch); the g*Q
//     query rows of the kv-head's group are packed as the 16-wide N side of
//     v_mfma_f32_16x16x32_bf16 and keys are the M side, so K and V are read
//     from HBM once per (batch, kv-head);
//   * the chunk streams through a two-stage LDS ring of 32-key sub-blocks
//     filled by direct buffer-to-LDS loads: while sub-block j is computed the
//     loads of j+1 are in flight, and j+2 is issued as soon as j is consumed;
//     rows past K_b and channels past D read as zero from the buffer range
//     check, so the loads have no branches;
//   * each workgroup writes one fp32 partial (m, l, acc[Dv]) per row;
//   * the combine pass merges a row's partials in chunk order, so results are
//     bitwise reproducible (no atomics).
#include "attn_internal.h"

namespace attn {

template <int DP, int DVP, int NT, int NSTG = kDecodeStages>
struct DecodeShape {
  static constexpr int NS = NSTG;               // ring stages (sub-blocks in LDS)
  static constexpr int KS = DP / 32;
  static constexpr int JV = DVP / 16;
  static constexpr int KCH = DP / 8;            // 16-byte chunks per K row
  static constexpr int VCH = DVP / 8;
  static constexpr int KROWB = DP * 2;          // LDS bytes per K row
  static constexpr int VROWB = DVP * 2;
  static constexpr int K_STAGE = kDecodeSub * KROWB;
  static constexpr int V_STAGE = kDecodeSub * VROWB;
  static constexpr int STAGE = K_STAGE + V_STAGE;
  static constexpr int K_LOADS = K_STAGE / 1024;  // wave-wide 1 KiB loads per stage
  static constexpr int V_LOADS = V_STAGE / 1024;
  static constexpr int LOADS = K_LOADS + V_LOADS;
};

// Union of the legal key ranges of all rows of one (batch, kv-head) group:
// [lo, hi).  Row q's position is q + K_b - Q, so the first row bounds the
// window from below and the sequence end bounds everything from above.
__device__ __forceinline__ void group_key_range(int Kb, int Q, int W, int* lo, int* hi) {
  *hi = Kb;
  *lo = W > 0 ? max(0, Kb - Q - W + 1) : 0;
}

template <int DP, int DVP, int NT>
__global__ __launch_bounds__(64) void decode_split_kernel(Params p) {
  using S = DecodeShape<DP, DVP, NT>;
  __shared__ __attribute__((aligned(16))) unsigned char ring[S::NS * S::STAGE];

  const int lane = threadIdx.x;
  const int l16 = lane & 15, g4 = lane >> 4;
  // Items (chunk, batch, kv-head) are numbered with the chunk slowest (see
  // below for its order).  The launch has one workgroup per item; the loop
  // also serves a smaller grid.
  const int groups = p.B * p.Hkv;
  const int n_items = p.n_splits * groups;

  // This lane's byte offset, from the start of a sub-block, for each 1 KiB
  // direct load of a stage: load i fills stage bytes [1024 i, 1024 i + 1024),
  // lane l position l of it, which holds chunk (position ^ swizzle) of its row.
  // Chunks past D (Dv) get an offset beyond any buffer and read as zero.
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

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
  const int ri = item / groups;
  const int b = (item - ri * groups) / p.Hkv;
  const int kh = item - ri * groups - b * p.Hkv;
  const int Kb = clamp_len(p.seqlens, b, p.K);
  const int Q = p.Q, W = p.window, delta = Kb - Q;
  int lo_u, hi_u;
  group_key_range(Kb, Q, W, &lo_u, &hi_u);
  if (hi_u <= lo_u) continue;  // no key: the combine pass writes 0 / -inf
  // Items are counted back from each sequence's last chunk, the slowest
  // index running from the most distant chunk to the last: the workgroups
  // dispatched last take the sequences' final (partial) chunks, so the
  // kernel's tail is short.
  const int c_last = (hi_u - 1) / p.chunk;
  const int chunk = c_last - (p.n_splits - 1 - ri);
  if (chunk < lo_u / p.chunk) continue;
  const int cs = chunk * p.chunk;
  const int ce = min(cs + p.chunk, hi_u);
  const int st = max(cs, lo_u);
  if (st >= ce) continue;  // the combine pass never reads this split
  // The previous item's reads of the ring have returned before it is refilled.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  const int64_t kv_slice = (int64_t)b * p.Hkv + kh;
  const uint16_t* kslice = static_cast<const uint16_t*>(p.k) + kv_slice * p.K * p.D;
  const uint16_t* vslice = static_cast<const uint16_t*>(p.v) + kv_slice * p.K * p.Dv;
  const float c = p.scale_log2;
  const uint32_t qx = p.q_sign ? 0x80008000u : 0u;

  // Q^T fragments: N column l16 of tile t is packed row rr = hh*Q + q.
  bf16x8 qf[NT][S::KS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int rr = 16 * t + l16;
    const bool ok = rr < p.rows;
    const int hh = ok ? rr / Q : 0, qi = ok ? rr % Q : 0;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(p.q) + (((int64_t)b * p.Hq + kh * p.group + hh) * Q + qi) * p.D;
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
      const int col = 32 * s + 8 * g4;
      uint4 u = (ok && col < p.D) ? load_u4(qrow + col) : zero_u4();
      u.x ^= qx; u.y ^= qx; u.z ^= qx; u.w ^= qx;
      qf[t][s] = __builtin_bit_cast(bf16x8, u);
    }
  }
  // Q is in registers before any direct load is issued.
  wait_vmcnt<0>();
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int s = 0; s < S::KS; ++s) launder(qf[t][s]);

  float m_run[NT], l_run[NT];
  f32x4 acc[S::JV][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int j = 0; j < S::JV; ++j) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Issue the direct loads of sub-block j into ring stage `stg`.  The buffer
  // descriptors start at the sub-block and end at K_b, so the per-lane offsets
  // are the same for every sub-block and rows past K_b read as zero.
  auto issue = [&](int j, int stg) {
    const int kb0 = cs + j * kDecodeSub;
    const uint32_t rows_left = (uint32_t)(Kb - kb0);
    const rsrc_t krs = slice_rsrc(kslice + (int64_t)kb0 * p.D, rows_left * p.D * 2);
    const rsrc_t vrs = slice_rsrc(vslice + (int64_t)kb0 * p.Dv, rows_left * p.Dv * 2);
    const uint32_t kst = lds_offset(ring) + stg * S::STAGE;
#pragma unroll
    for (int i = 0; i < S::K_LOADS; ++i) load_lds16(krs, kst + i * 1024, koff[i]);
#pragma unroll
    for (int i = 0; i < S::V_LOADS; ++i) load_lds16(vrs, kst + S::K_STAGE + i * 1024, voff[i]);
  };

  const int j0 = (st - cs) / kDecodeSub;
  const int j1 = (ce - cs + kDecodeSub - 1) / kDecodeSub;
#pragma unroll
  for (int u = 0; u < S::NS; ++u)
    if (j0 + u < j1) issue(j0 + u, u);

  // Absolute position of each packed row (row rr is query rr % Q).
  int pq[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) pq[t] = (16 * t + l16) % Q + delta;

  // Sub-block j sits in stage (j - j0) % NS; once every LDS read of it has
  // returned, sub-block j + NS is issued into the same stage.  Before
  // computing j, the loads of the up to NS - 1 later sub-blocks may stay in
  // flight.
  int stg = 0;
  for (int j = j0; j < j1; ++j) {
    const int later = min(S::NS - 1, j1 - 1 - j);
    static_for<S::NS>([&](auto n_tag) {
      constexpr int n = decltype(n_tag)::value;
      if (later == n) wait_vmcnt<n * S::LOADS>();
    });
    const unsigned char* kst = ring + stg * S::STAGE;
    const unsigned char* vst = kst + S::K_STAGE;
    const int kb0 = cs + j * kDecodeSub;

    // Every LDS read of the sub-block is issued up front (K fragments, then the
    // transposed V fragments), so a single wave pays the LDS latency once per
    // step rather than once per fragment; the V reads overlap QK and softmax.
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
#pragma unroll
    for (int jv = 0; jv < S::JV; ++jv) {
      const int row = 4 * g4 + (l16 >> 2);
      const int ch = 2 * jv + ((l16 & 3) >> 1), half = (l16 & 1) * 8;
      const unsigned char* lo = vst + row * S::VROWB + ((ch ^ swz_v<S::VCH>(row)) << 4) + half;
      const unsigned char* hi = vst + (row + 16) * S::VROWB + ((ch ^ swz_v<S::VCH>(row + 16)) << 4) + half;
      vf[jv] = concat_bf16x4(lds_read_tr16(reinterpret_cast<const uint16_t*>(lo)),
                             lds_read_tr16(reinterpret_cast<const uint16_t*>(hi)));
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
        for (int t = 0; t < NT; ++t) sacc[i][t] = mfma16x16x32(kf[i][s], qf[t][s], sacc[i][t]);
    // Every row sees keys <= K_b - Q causally; the last row's window starts at K_b - W.
    const bool full = (kb0 + kDecodeSub - 1 <= delta) && (kb0 + kDecodeSub <= Kb) && (W <= 0 || kb0 >= Kb - W);
    if (!full) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kb0 + 16 * i + 4 * g4 + r;
            const bool legal = key <= pq[t] && key < Kb && (W <= 0 || key > pq[t] - W);
            if (!legal) sacc[i][t][r] = -INFINITY;
          }
        }
      }
    }
    bf16x8 pf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float mx = sacc[0][t][0];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[i][t][r]);
      mx = group4_max(mx);
      const float mb = (mx == -INFINITY) ? -INFINITY : mx * c;
      float alpha;
      if (softmax_rebase(m_run[t], mb, alpha)) {
        l_run[t] *= alpha;
#pragma unroll
        for (int jv = 0; jv < S::JV; ++jv) acc[jv][t] *= alpha;
      }
      const float mref = m_run[t];
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
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
      pf[t] = pack_bf16x8(sacc[0][t], sacc[1][t]);
    }
    // O^T += V^T P^T.
#pragma unroll
    for (int jv = 0; jv < S::JV; ++jv)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[jv][t] = mfma16x16x32(vf[jv], pf[t], acc[jv][t]);
    if (j + S::NS < j1) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(j + S::NS, stg);
    }
    stg = stg + 1 == S::NS ? 0 : stg + 1;
  }

  // One partial per (row, chunk): m in log2 units, l = sum of 2^(s*c - m), unnormalised acc.
  const int64_t split = kv_slice * p.n_splits + chunk;
  const int R = p.rows;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = group4_sum(l_run[t]);
    const int rr = 16 * t + l16;
    if (rr < R) {
      const int64_t part = split * R + rr;
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
  }  // items
}

// One wave per output row (b, h, q): merge the row's partials in chunk order.
// Lane c holds chunk c's (m, l) (64 chunks per round), so the row max and
// the weights f_c = 2^(m_c - M) take one round of loads and a wave
// reduction; then every lane accumulates two dv columns over the chunks with
// all of a round's loads in flight.  The merge order is fixed, so results
// are bitwise reproducible.
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
  const int Kb = clamp_len(p.seqlens, b, p.K);
  int lo_u, hi_u;
  group_key_range(Kb, p.Q, p.window, &lo_u, &hi_u);
  const int c_lo = lo_u / p.chunk;
  const int c_hi = hi_u > lo_u ? (hi_u + p.chunk - 1) / p.chunk : c_lo;
  const int64_t split0 = ((int64_t)b * p.Hkv + kh) * p.n_splits;
  const int R = p.rows;

  // Row max over the chunks (a chunk with no legal key for this row has m = -inf).
  float M = -INFINITY;
  for (int c0 = c_lo; c0 < c_hi; c0 += 64) {
    const int cix = c0 + lane;
    const float m = cix < c_hi ? p.ws_m[(split0 + cix) * R + rr] : -INFINITY;
    M = fmaxf(M, m);
  }
  M = wave_max(M);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  if (M != -INFINITY) {
    for (int c0 = c_lo; c0 < c_hi; c0 += 64) {
      const int cix = c0 + lane;
      const int64_t sp = (split0 + cix) * R + rr;
      const float m = cix < c_hi ? p.ws_m[sp] : -INFINITY;
      const float f = m == -INFINITY ? 0.f : fast_exp2(m - M);
      L += cix < c_hi ? p.ws_l[sp] * f : 0.f;
      const int n = min(64, c_hi - c0);
      // Lane `u` of the round holds f for chunk c0 + u.
      constexpr int U = 8;
      for (int u0 = 0; u0 < n; u0 += U) {
        float a0[U], a1[U], fu[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = u0 + u < n;
          const float* a = p.ws_acc + ((split0 + c0 + u0 + u) * R + rr) * p.Dv;
          a0[u] = ok && lane < p.Dv ? a[lane] : 0.f;
          a1[u] = ok && lane + 64 < p.Dv ? a[lane + 64] : 0.f;
          fu[u] = __shfl(f, (u0 + u) & 63);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          o0 = fmaf(a0[u], fu[u], o0);
          o1 = fmaf(a1[u], fu[u], o1);
        }
      }
    }
    L = wave_sum(L);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(p.o) + row_id * p.Dv;
  if (lane < p.Dv) orow[lane] = __builtin_bit_cast(uint16_t, (__bf16)(o0 * inv));
  if (lane + 64 < p.Dv) orow[lane + 64] = __builtin_bit_cast(uint16_t, (__bf16)(o1 * inv));
  if (lane == 0) p.lse[row_id] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

template <int DP, int DVP, int NT>
static hipError_t launch_decode_t(const Params& p, hipStream_t stream) {
  Params arg = p;
  void* args[] = {&arg};
  // With K == 0 there is no split: the combine pass alone writes 0 / -inf.
  if (p.n_splits > 0) {
    const int64_t items = (int64_t)p.n_splits * p.Hkv * p.B;
    const dim3 grid((unsigned)items);
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_split_kernel<DP, DVP, NT>), grid,
                                         dim3(64), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t rows = (int64_t)p.B * p.Hq * p.Q;
  const dim3 cgrid((unsigned)((rows + 3) / 4));
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_combine_kernel), cgrid, dim3(256), args, 0, stream);
}

template <int DP, int DVP>
static hipError_t launch_decode_nt(const Params& p, hipStream_t stream) {
  if (p.rows <= 16) return launch_decode_t<DP, DVP, 1>(p, stream);
  return launch_decode_t<DP, DVP, 2>(p, stream);
}

hipError_t launch_decode_bf16(const Params& p, hipStream_t stream) {
  const int dp = pad_width(p.D), dvp = pad_width(p.Dv);
  if (dp == 64 && dvp == 64) return launch_decode_nt<64, 64>(p, stream);
  if (dp == 64 && dvp == 128) return launch_decode_nt<64, 128>(p, stream);
  if (dp == 128 && dvp == 64) return launch_decode_nt<128, 64>(p, stream);
  return launch_decode_nt<128, 128>(p, stream);
}

}  // namespace attn
