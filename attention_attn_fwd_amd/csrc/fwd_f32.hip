// fp32 attention forward (float in, float out, float arithmetic throughout):
// the same bottom-right causal GQA with online softmax as the bf16 path
// (LuisaCompute "Attention execution mapping" review, section 1), written for
// exactness rather than speed: CPU intermediates stay fp32 on the Laya "Fast
// backends" page, and this path keeps that precision on the GPU.  Its sizes
// are small, so the layout aims at latency: many workgroups, short dependent
// chains, and the next K/V block in flight while the current one is used.
//
// One workgroup of 256 threads per (batch, head, 16 query rows).  K/V blocks
// of 32 keys are staged in LDS; thread (row r = tid/16, slot cg = tid%16)
// computes the scores of keys cg and cg+16 for its row (four independent
// partial sums each), the row's 16 threads share the 32 scores through LDS,
// and each thread keeps the accumulator columns dv = cg + 16*i of its row.
// The next block's K/V are loaded into registers before the current block's
// scores and stored to LDS after its weights are applied.  The kernel is
// instantiated for a padded width WP (64 or 128, covering D and Dv; Q and K
// are zero past D) so every loop over channels has a constant trip count.
#include <algorithm>

#include "attn_internal.h"

namespace attn {

constexpr int kF32MaxD = 128;
constexpr int kF32Threads = 256;
constexpr int kF32Cols = 16;                                       // threads per row

template <int WP>
__global__ __launch_bounds__(256) void fwd_f32_kernel(Params p) {
  constexpr int kStage = kF32Keys * WP / kF32Threads;  // K (or V) floats per thread per block
  __shared__ float Qs[kF32Rows][WP + 1];
  __shared__ float Ks[kF32Keys][WP + 1];
  __shared__ float Vs[kF32Keys][WP];
  __shared__ float Ss[kF32Rows][kF32Keys + 1];

  const int tid = threadIdx.x, r = tid / kF32Cols, cg = tid % kF32Cols;
  const int n_qt = (p.Q + kF32Rows - 1) / kF32Rows;
  int x = blockIdx.x;
  const int h = x % p.Hq;
  x /= p.Hq;
  const int b = x % p.B;
  x /= p.B;
  const int qt = n_qt - 1 - x;
  const int kh = h / p.group;
  const int Kb = clamp_len(p.seqlens, b, p.K);
  const int delta = row_delta(Kb, p.Q, p.causal_shift), W = p.window;
  const int q0 = qt * kF32Rows, q_end = min(q0 + kF32Rows, p.Q);
  const int kv_hi = min(Kb, q_end - 1 + delta + 1);
  const int kv_lo = W > 0 ? max(0, q0 + delta - W + 1) : 0;
  const int D = p.D, Dv = p.Dv;
  const float c = p.scale * 1.4426950408889634f;

  const float* qg = static_cast<const float*>(p.q) + ((int64_t)b * p.Hq + h) * p.Q * D;
  const float* kg = static_cast<const float*>(p.k) + ((int64_t)b * p.Hkv + kh) * p.K * D;
  const float* vg = static_cast<const float*>(p.v) + ((int64_t)b * p.Hkv + kh) * p.K * Dv;
  float* og = static_cast<float*>(p.o) + ((int64_t)b * p.Hq + h) * p.Q * Dv;

  for (int idx = tid; idx < kF32Rows * WP; idx += kF32Threads) {
    const int rr = idx / WP, d = idx % WP, row = q0 + rr;
    Qs[rr][d] = (row < p.Q && d < D) ? qg[(int64_t)row * D + d] : 0.f;
  }
  const int row = q0 + r;
  const int pq = row + delta;
  float m = -INFINITY, l = 0.f;
  float acc[WP / kF32Cols];
#pragma unroll
  for (int i = 0; i < WP / kF32Cols; ++i) acc[i] = 0.f;

  // Block jb's K/V into registers: element idx = tid + 256 i of the block's
  // keys x width (zero past K_b and past the width).
  float kr[kStage], vr[kStage];
  auto fetch = [&](int jb) {
    const int kb0 = jb * kF32Keys;
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int idx = tid + kF32Threads * i;
      const int kk = idx / WP, d = idx % WP, key = kb0 + kk;
      kr[i] = (key < Kb && d < D) ? kg[(int64_t)key * D + d] : 0.f;
      vr[i] = (key < Kb && d < Dv) ? vg[(int64_t)key * Dv + d] : 0.f;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int idx = tid + kF32Threads * i;
      const int kk = idx / WP, d = idx % WP;
      Ks[kk][d] = kr[i];
      Vs[kk][d] = vr[i];
    }
  };

  const int jb0 = kv_lo / kF32Keys;
  const int jb1 = kv_hi > kv_lo ? (kv_hi + kF32Keys - 1) / kF32Keys : jb0;
  if (jb0 < jb1) {
    fetch(jb0);
    stage();
  }
  for (int jb = jb0; jb < jb1; ++jb) {
    const int kb0 = jb * kF32Keys;
    __syncthreads();  // Q and this block's K/V staged; the previous block's reads done
    if (jb + 1 < jb1) fetch(jb + 1);
    // Scores of keys cg and cg + 16: four partial sums each (d mod 4).
    {
      float s0[4] = {0.f, 0.f, 0.f, 0.f}, s1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < WP; d += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float qv = Qs[r][d + u];
          s0[u] = fmaf(qv, Ks[cg][d + u], s0[u]);
          s1[u] = fmaf(qv, Ks[cg + kF32Cols][d + u], s1[u]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float* sp = t ? s1 : s0;
        const int kk = cg + kF32Cols * t, key = kb0 + kk;
        const float s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
        const bool legal = key <= pq && key < Kb && (W <= 0 || key > pq - W);
        Ss[r][kk] = legal ? s * c : -INFINITY;
      }
    }
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kF32Keys; ++kk) mx = fmaxf(mx, Ss[r][kk]);
    const float mnew = fmaxf(m, mx);
    if (mnew != -INFINITY) {  // else no legal key for this row yet
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < WP / kF32Cols; ++i) acc[i] *= alpha;
#pragma unroll
      for (int kk = 0; kk < kF32Keys; ++kk) {
        const float sv = Ss[r][kk];
        const float e = sv == -INFINITY ? 0.f : fast_exp2(sv - mnew);
        l += e;
#pragma unroll
        for (int i = 0; i < WP / kF32Cols; ++i) {
          const int dv = cg + kF32Cols * i;
          if (dv < Dv) acc[i] = fmaf(e, Vs[kk][dv], acc[i]);
        }
      }
    }
    if (jb + 1 < jb1) {
      __syncthreads();  // every thread is done with this block's K/V
      stage();
    }
  }
  if (row >= p.Q) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < WP / kF32Cols; ++i) {
    const int dv = cg + kF32Cols * i;
    if (dv < Dv) og[(int64_t)row * Dv + dv] = acc[i] * inv;
  }
  if (cg == 0) p.lse[((int64_t)b * p.Hq + h) * p.Q + row] = l > 0.f ? (m + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

hipError_t launch_fwd_f32(const Params& p, hipStream_t stream) {
  const int n_qt = (p.Q + kF32Rows - 1) / kF32Rows;
  const dim3 grid((unsigned)((int64_t)n_qt * p.Hq * p.B));
  Params arg = p;
  void* args[] = {&arg};
  const void* fn = std::max(p.D, p.Dv) <= 64 ? reinterpret_cast<const void*>(&fwd_f32_kernel<64>)
                                              : reinterpret_cast<const void*>(&fwd_f32_kernel<kF32MaxD>);
  return hipLaunchKernel(fn, grid, dim3(kF32Threads), args, 0, stream);
}

}  // namespace attn
