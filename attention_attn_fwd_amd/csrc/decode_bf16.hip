// Split-KV decode for Q = 1..4 on gfx950, plus the log-sum-exp combine pass.
//
// The recurrence is the one of the LuisaCompute "Attention execution mapping"
// review, section 1 (online (row_max, row_sum, acc) carried across KV
// blocks); section 5 notes that splitting a long KV range needs a legal merge
// of that state, which is what the combine pass does, and that one kv-head
// serves Hq/Hkv query heads; section 4 notes that a single query row cannot
// fill a matrix atom.  Hence:
//   * one workgroup per (chunk of keys, kv-head, batch); the g*Q query rows
//     of the kv-head's group are packed as the 16-wide N side of
//     v_mfma_f32_16x16x32_bf16, keys on the M side, so K and V are read from
//     HBM once per (batch, kv-head);
//   * the 4 waves of a workgroup take interleaved 32-key sub-blocks of the
//     chunk; K fragments go straight from HBM to registers in MFMA layout, V
//     goes through a wave-private LDS tile and is read back transposed with
//     ds_read_b64_tr_b16; the next sub-block's loads are issued before the
//     current one is computed;
//   * at the end the waves' states are merged in LDS in a fixed order and
//     written as one partial (m, l, acc[Dv]) per (row, chunk);
//   * the combine pass merges the partials of each row in chunk order, so
//     results are bitwise reproducible (no atomics).
#include "attn_internal.h"

namespace attn {

template <int DP, int DVP, int NT>
struct DecodeShape {
  static constexpr int KS = DP / 32;
  static constexpr int JV = DVP / 16;
  static constexpr int VROW = DVP + 8;
  static constexpr int VCH = DVP / 8;
  static constexpr int VLOADS = kDecodeSub * VCH / 64;  // per lane per sub-block
  static constexpr int ROWS = 16 * NT;
  static constexpr int VS_BYTES = kDecodeWaves * kDecodeSub * VROW * 2;
  static constexpr int BUF_BYTES = ROWS * DVP * 4;
  static constexpr int SMEM_BYTES = VS_BYTES > BUF_BYTES ? VS_BYTES : BUF_BYTES;
};

// Union of the legal key ranges of all rows of one (batch, kv-head) group:
// [lo, hi).  Row q's position is q + K_b - Q, so the first row bounds the
// window from below and the sequence end bounds everything from above.
__device__ __forceinline__ void group_key_range(int Kb, int Q, int W, int* lo, int* hi) {
  *hi = Kb;
  *lo = W > 0 ? max(0, Kb - Q - W + 1) : 0;
}

template <int DP, int DVP, int NT>
__global__ __launch_bounds__(256) void decode_split_kernel(Params p) {
  using S = DecodeShape<DP, DVP, NT>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::SMEM_BYTES];
  __shared__ float red_m[kDecodeWaves][S::ROWS];
  __shared__ float red_l[kDecodeWaves][S::ROWS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int chunk = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int Kb = clamp_len(p.seqlens, b, p.K);
  const int Q = p.Q, W = p.window, delta = Kb - Q;
  int lo_u, hi_u;
  group_key_range(Kb, Q, W, &lo_u, &hi_u);
  const int cs = chunk * p.chunk;
  const int ce = min(cs + p.chunk, hi_u);
  const int st = max(cs, lo_u);
  if (st >= ce) return;  // the combine pass never reads this split

  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.Hkv + kh) * p.K * p.D;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.Hkv + kh) * p.K * p.Dv;
  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * kDecodeSub * S::VROW;
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

  float m_run[NT], l_run[NT];
  f32x4 acc[S::JV][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int j = 0; j < S::JV; ++j) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int j0 = (st - cs) / kDecodeSub;
  const int j1 = (ce - cs + kDecodeSub - 1) / kDecodeSub;

  uint4 kcur[2][S::KS], vcur[S::VLOADS];
  auto gload = [&](int j, uint4 (&kr)[2][S::KS], uint4 (&vr)[S::VLOADS]) {
    const int kb0 = cs + j * kDecodeSub;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = kb0 + 16 * i + l16;
#pragma unroll
      for (int s = 0; s < S::KS; ++s) {
        const int col = 32 * s + 8 * g4;
        kr[i][s] = (key < Kb && col < p.D) ? load_u4(kg + (int64_t)key * p.D + col) : zero_u4();
      }
    }
#pragma unroll
    for (int i = 0; i < S::VLOADS; ++i) {
      const int idx = lane + 64 * i, r = idx / S::VCH, ch = idx % S::VCH, key = kb0 + r;
      vr[i] = (key < Kb && ch * 8 < p.Dv) ? load_u4(vg + (int64_t)key * p.Dv + ch * 8) : zero_u4();
    }
  };

  int j = j0 + wave;
  if (j < j1) gload(j, kcur, vcur);
  for (; j < j1; j += kDecodeWaves) {
    // Stage this sub-block's V tile in the wave-private LDS tile.
#pragma unroll
    for (int i = 0; i < S::VLOADS; ++i) {
      const int idx = lane + 64 * i, r = idx / S::VCH, ch = idx % S::VCH;
      *reinterpret_cast<uint4*>(&vs[r * S::VROW + ch * 8]) = vcur[i];
    }
    uint4 knext[2][S::KS], vnext[S::VLOADS];
    const bool more = j + kDecodeWaves < j1;
    if (more) gload(j + kDecodeWaves, knext, vnext);

    const int kb0 = cs + j * kDecodeSub;
    f32x4 sacc[2][NT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) sacc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, kcur[i][s]);
#pragma unroll
        for (int t = 0; t < NT; ++t) sacc[i][t] = mfma16x16x32(a, qf[t][s], sacc[i][t]);
      }
    }
    // Every row sees keys <= K_b - Q causally; the last row's window starts at K_b - W.
    const bool full = (kb0 + kDecodeSub - 1 <= delta) && (kb0 + kDecodeSub <= Kb) && (W <= 0 || kb0 >= Kb - W);
    if (!full) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int rr = 16 * t + l16;
        const int pq = (rr % Q) + delta;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kb0 + 16 * i + 4 * g4 + r;
            const bool legal = key <= pq && key < Kb && (W <= 0 || key > pq - W);
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
      const float mnew = fmaxf(m_run[t], mb);
      const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m_run[t] - mnew);
      m_run[t] = mnew;
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sv = sacc[i][t][r];
          float e = fast_exp2(fmaf(sv, c, -mnew));
          if (!full) e = (sv == -INFINITY) ? 0.f : e;
          sacc[i][t][r] = e;
          rs += e;
        }
      }
      l_run[t] = l_run[t] * alpha + rs;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int jv = 0; jv < S::JV; ++jv) acc[jv][t] *= alpha;
      }
      pf[t] = pack_bf16x8(sacc[0][t], sacc[1][t]);
    }
    // LDS operations of one wave complete in issue order; this keeps the
    // compiler from moving the tile stores past the transposed reads.
    asm volatile("" ::: "memory");
#pragma unroll
    for (int jv = 0; jv < S::JV; ++jv) {
      const uint16_t* vlo = &vs[(4 * g4 + (l16 >> 2)) * S::VROW + 16 * jv + 4 * (l16 & 3)];
      const bf16x8 va = concat_bf16x4(lds_read_tr16(vlo), lds_read_tr16(vlo + 16 * S::VROW));
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[jv][t] = mfma16x16x32(va, pf[t], acc[jv][t]);
    }
    asm volatile("" ::: "memory");
    if (more) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int s = 0; s < S::KS; ++s) kcur[i][s] = knext[i][s];
#pragma unroll
      for (int i = 0; i < S::VLOADS; ++i) vcur[i] = vnext[i];
    }
  }

  // Merge the four waves' states in a fixed order.
  float lt[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    lt[t] = group4_sum(l_run[t]);
    if (g4 == 0) {
      red_m[wave][16 * t + l16] = m_run[t];
      red_l[wave][16 * t + l16] = lt[t];
    }
  }
  __syncthreads();
  float* buf = reinterpret_cast<float*>(smem);  // [ROWS][DVP], reuses the V tiles
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int rr = 16 * t + l16;
        float M = red_m[0][rr];
#pragma unroll
        for (int u = 1; u < kDecodeWaves; ++u) M = fmaxf(M, red_m[u][rr]);
        const float f = (m_run[t] == -INFINITY) ? 0.f : fast_exp2(m_run[t] - M);
#pragma unroll
        for (int jv = 0; jv < S::JV; ++jv) {
          f32x4* dst = reinterpret_cast<f32x4*>(&buf[rr * DVP + 16 * jv + 4 * g4]);
          const f32x4 v = acc[jv][t] * f;
          *dst = (w == 0) ? v : (*dst + v);
        }
      }
    }
    __syncthreads();
  }
  const int64_t split = ((int64_t)b * p.Hkv + kh) * p.n_splits + chunk;
  const int R = p.rows;
  for (int rr = tid; rr < R; rr += 256) {
    float M = red_m[0][rr];
    for (int u = 1; u < kDecodeWaves; ++u) M = fmaxf(M, red_m[u][rr]);
    float L = 0.f;
    for (int u = 0; u < kDecodeWaves; ++u)
      if (red_m[u][rr] != -INFINITY) L += red_l[u][rr] * fast_exp2(red_m[u][rr] - M);
    p.ws_m[split * R + rr] = M;
    p.ws_l[split * R + rr] = L;
  }
  float* wacc = p.ws_acc + split * R * p.Dv;
  for (int idx = tid; idx < R * p.Dv; idx += 256) {
    const int rr = idx / p.Dv, dv = idx % p.Dv;
    wacc[idx] = buf[rr * DVP + dv];
  }
}

// One wave per output row (b, h, q): merge the row's partials in chunk order.
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

  float M = -INFINITY;
  for (int cix = c_lo; cix < c_hi; ++cix) M = fmaxf(M, p.ws_m[(split0 + cix) * R + rr]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  if (M != -INFINITY) {
    for (int cix = c_lo; cix < c_hi; ++cix) {
      const int64_t sp = (split0 + cix) * R + rr;
      const float m = p.ws_m[sp];
      if (m == -INFINITY) continue;
      const float f = fast_exp2(m - M);
      L += p.ws_l[sp] * f;
      const float* a = p.ws_acc + sp * p.Dv;
      if (lane < p.Dv) o0 += a[lane] * f;
      if (lane + 64 < p.Dv) o1 += a[lane + 64] * f;
    }
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
  const dim3 grid((unsigned)p.n_splits, (unsigned)p.Hkv, (unsigned)p.B);
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_split_kernel<DP, DVP, NT>), grid, dim3(256),
                                 args, 0, stream);
  if (e != hipSuccess) return e;
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
