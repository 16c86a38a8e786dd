// fp32 attention forward (float in, float out, float arithmetic throughout):
// the same bottom-right causal GQA with online softmax as the bf16 path
// (LuisaCompute "Attention execution mapping" review, section 1), written for
// exactness rather than speed: CPU intermediates stay fp32 on the Laya "Fast
// backends" page, and this path keeps that precision on the GPU.
//
// One workgroup of 256 threads per (batch, head, 32 query rows).  K/V blocks
// of 32 keys are staged in LDS; thread (row r = tid/8, slot cg = tid%8)
// computes the scores of keys cg, cg+8, cg+16, cg+24 for its row, the row's
// 8 threads then share the 32 scores through LDS, and each thread keeps the
// accumulator columns dv = cg + 8*i of its row.
#include "attn_internal.h"

namespace attn {

constexpr int kF32MaxD = 128;

__global__ __launch_bounds__(256) void fwd_f32_kernel(Params p) {
  __shared__ float Qs[kF32Rows][kF32MaxD + 1];
  __shared__ float Ks[kF32Keys][kF32MaxD + 1];
  __shared__ float Vs[kF32Keys][kF32MaxD];
  __shared__ float Ss[kF32Rows][kF32Keys + 1];

  const int tid = threadIdx.x, r = tid >> 3, cg = tid & 7;
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

  for (int idx = tid; idx < kF32Rows * D; idx += 256) {
    const int rr = idx / D, d = idx % D, row = q0 + rr;
    Qs[rr][d] = row < p.Q ? qg[(int64_t)row * D + d] : 0.f;
  }
  const int row = q0 + r;
  const int pq = row + delta;
  float m = -INFINITY, l = 0.f;
  float acc[kF32MaxD / 8];
#pragma unroll
  for (int i = 0; i < kF32MaxD / 8; ++i) acc[i] = 0.f;

  const int jb0 = kv_lo / kF32Keys;
  const int jb1 = kv_hi > kv_lo ? (kv_hi + kF32Keys - 1) / kF32Keys : jb0;
  for (int jb = jb0; jb < jb1; ++jb) {
    const int kb0 = jb * kF32Keys;
    __syncthreads();
    for (int idx = tid; idx < kF32Keys * D; idx += 256) {
      const int kk = idx / D, d = idx % D, key = kb0 + kk;
      Ks[kk][d] = key < Kb ? kg[(int64_t)key * D + d] : 0.f;
    }
    for (int idx = tid; idx < kF32Keys * Dv; idx += 256) {
      const int kk = idx / Dv, d = idx % Dv, key = kb0 + kk;
      Vs[kk][d] = key < Kb ? vg[(int64_t)key * Dv + d] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = cg + 8 * i, key = kb0 + kk;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(Qs[r][d], Ks[kk][d], s);
      const bool legal = key <= pq && key < Kb && (W <= 0 || key > pq - W);
      Ss[r][kk] = legal ? s * c : -INFINITY;
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int kk = 0; kk < kF32Keys; ++kk) mx = fmaxf(mx, Ss[r][kk]);
    const float mnew = fmaxf(m, mx);
    if (mnew == -INFINITY) continue;  // no legal key for this row yet
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < kF32MaxD / 8; ++i) acc[i] *= alpha;
    for (int kk = 0; kk < kF32Keys; ++kk) {
      const float sv = Ss[r][kk];
      if (sv == -INFINITY) continue;
      const float e = fast_exp2(sv - mnew);
      l += e;
#pragma unroll
      for (int i = 0; i < kF32MaxD / 8; ++i) {
        const int dv = cg + 8 * i;
        if (dv < Dv) acc[i] = fmaf(e, Vs[kk][dv], acc[i]);
      }
    }
  }
  if (row >= p.Q) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < kF32MaxD / 8; ++i) {
    const int dv = cg + 8 * i;
    if (dv < Dv) og[(int64_t)row * Dv + dv] = acc[i] * inv;
  }
  if (cg == 0) p.lse[((int64_t)b * p.Hq + h) * p.Q + row] = l > 0.f ? (m + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

hipError_t launch_fwd_f32(const Params& p, hipStream_t stream) {
  const int n_qt = (p.Q + kF32Rows - 1) / kF32Rows;
  const dim3 grid((unsigned)((int64_t)n_qt * p.Hq * p.B));
  Params arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_f32_kernel), grid, dim3(256), args, 0, stream);
}

}  // namespace attn
