// fp32 attention forward (float in, float out, float arithmetic throughout):
// the same bottom-right causal GQA with online softmax as the bf16 path
// (LuisaCompute "Attention execution mapping" review, section 1).  CPU
// intermediates stay fp32 on the Laya "Fast backends" page, and this path
// keeps that precision on the GPU: the products run on the fp32 matrix
// instruction v_mfma_f32_16x16x4_f32 (fp32 operands, fp32 accumulation).
// Its sizes are small, so the layout aims at latency.
//
// One workgroup of four waves per (batch, head, 16 query rows).  The tile's
// 32-key blocks are dealt to the waves in turn (wave w takes blocks jb0 + w,
// jb0 + w + 4, ...), so a short key range takes one block's latency rather
// than four.  Each wave keeps its own online state (m, l, O^T) for the 16
// rows, loads its K and V fragments straight from memory into registers
// (buffer loads: keys past K_b read as zero) with the next block's in flight,
// and at the end the four states are merged through LDS in wave order.
//
// Matrix layouts (lane l, l16 = l % 16, g = l / 16):
//   S^T = K Q^T, one 16-key tile per product: A = K[key l16][d], B = Q^T[d]
//   [row l16], with contraction index g at k-step (a, b) meaning channel
//   16a + 4g + b, so each lane's four k-steps of one a are one float4 of K
//   and of Q; the lane receives S^T[key 4g + i][row l16], i = 0..3;
//   O^T += V^T P^T, one 16-wide dv tile per product: A = V^T[dv l16][key],
//   B = P^T[key][row l16], with contraction index g at k-step (kt, i)
//   meaning key 16kt + 4g + i, which is exactly the S^T element the lane
//   holds; the lane receives O^T[dv 4g + r][row l16].
#include <algorithm>

#include "attn_internal.h"

namespace attn {

constexpr int kF32MaxD = 128;
constexpr int kF32Waves = 4;

__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int WP>
__global__ __launch_bounds__(64 * kF32Waves) void fwd_f32_kernel(Params p) {
  constexpr int NA = WP / 16;  // 16-channel groups of D (four k-steps each)
  constexpr int JV = WP / 16;  // 16-wide dv tiles
  static_assert(kF32Rows == 16 && kF32Keys == 32, "one 16-row N tile, two 16-key tiles per block");
  __shared__ float Ms[kF32Waves][16], Ls[kF32Waves][16];
  __shared__ float As[kF32Waves][16][WP + 4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
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
  const int D = p.D, Dv = p.Dv, na = D / 16, nj = Dv / 16;
  const float c = p.scale * 1.4426950408889634f;

  const float* qg = static_cast<const float*>(p.q) + ((int64_t)b * p.Hq + h) * p.Q * D;
  const float* kg = static_cast<const float*>(p.k) + ((int64_t)b * p.Hkv + kh) * p.K * D;
  const float* vg = static_cast<const float*>(p.v) + ((int64_t)b * p.Hkv + kh) * p.K * Dv;

  // Q fragments of row q0 + l16 (zero past the last query row).
  f32x4 qf[NA];
  {
    const auto qrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(qg + (int64_t)q0 * D), (short)0,
                                                       (q_end - q0) * D * 4, kRsrcWord3);
#pragma unroll
    for (int a = 0; a < NA; ++a)
      qf[a] = a < na ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, (l16 * D + 16 * a + 4 * g) * 4, 0, 0))
                     : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Fragments of block jb: K rows 16kt + l16, channels 16a + 4g .. + 3; V
  // rows 16kt + 4g + i, channel 16j + l16.  Keys past K_b read as zero.
  struct Frag {
    f32x4 k[2][NA];
    float v[2][4][JV];
  };
  auto fetch = [&](int jb, Frag& f) {
    const int kb0 = jb * kF32Keys, rows = min(kF32Keys, Kb - kb0);
    const auto krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(kg + (int64_t)kb0 * D), (short)0,
                                                       rows * D * 4, kRsrcWord3);
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(vg + (int64_t)kb0 * Dv), (short)0,
                                                       rows * Dv * 4, kRsrcWord3);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int a = 0; a < NA; ++a)
        f.k[kt][a] = a < na ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                            krs, ((16 * kt + l16) * D + 16 * a + 4 * g) * 4, 0, 0))
                            : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JV; ++j)
          f.v[kt][i][j] = j < nj ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                 vrs, ((16 * kt + 4 * g + i) * Dv + 16 * j + l16) * 4, 0, 0))
                                 : 0.f;
  };

  float m = -INFINITY, l = 0.f;  // row l16's state (m uniform over the row's four lanes; l this lane's part)
  f32x4 acc[JV];
#pragma unroll
  for (int j = 0; j < JV; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int pq = q0 + l16 + delta;  // absolute position of this lane's row

  const int jb0 = kv_lo / kF32Keys;
  const int jb1 = kv_hi > kv_lo ? (kv_hi + kF32Keys - 1) / kF32Keys : jb0;
  Frag cur, nxt;
  int jb = jb0 + wave;
  if (jb < jb1) fetch(jb, cur);
  for (; jb < jb1; jb += kF32Waves) {
    if (jb + kF32Waves < jb1) fetch(jb + kF32Waves, nxt);
    const int kb0 = jb * kF32Keys;
    f32x4 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        if (a < na) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) s[kt] = mfma16x16x4(cur.k[kt][a][bb], qf[a][bb], s[kt]);
        }
      }
    }
    // Scaled scores, -inf at illegal keys; the block's row max.
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb0 + 16 * kt + 4 * g + i;
        const bool legal = key <= pq && key < Kb && (W <= 0 || key > pq - W);
        s[kt][i] = legal ? s[kt][i] * c : -INFINITY;
        mx = fmaxf(mx, s[kt][i]);
      }
    const float mnew = fmaxf(m, group4_max(mx));
    const float mref = mnew == -INFINITY ? 0.f : mnew;  // no legal key yet: every weight is 0
    const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mnew);
    m = mnew;
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[kt][i] = fast_exp2(s[kt][i] - mref);
        rs += s[kt][i];
      }
    l = fmaf(l, alpha, rs);
#pragma unroll
    for (int j = 0; j < JV; ++j) acc[j] *= alpha;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JV; ++j)
          if (j < nj) acc[j] = mfma16x16x4(cur.v[kt][i][j], s[kt][i], acc[j]);
    cur = nxt;
  }

  // Merge the four waves' states in wave order.
  const float lt = group4_sum(l);
  if (g == 0) {
    Ms[wave][l16] = m;
    Ls[wave][l16] = lt;
  }
#pragma unroll
  for (int j = 0; j < JV; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) As[wave][l16][16 * j + 4 * g + r] = acc[j][r];
  __syncthreads();
  const int tid = threadIdx.x, rr = tid / 16, cg = tid % 16, row = q0 + rr;
  if (row >= p.Q) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kF32Waves; ++w) M = fmaxf(M, Ms[w][rr]);
  float f[kF32Waves], L = 0.f;
#pragma unroll
  for (int w = 0; w < kF32Waves; ++w) {
    f[w] = Ms[w][rr] == -INFINITY ? 0.f : fast_exp2(Ms[w][rr] - M);
    L = fmaf(Ls[w][rr], f[w], L);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* orow = static_cast<float*>(p.o) + (((int64_t)b * p.Hq + h) * p.Q + row) * Dv;
  for (int dv = cg; dv < Dv; dv += 16) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kF32Waves; ++w) o = fmaf(As[w][rr][dv], f[w], o);
    orow[dv] = o * inv;
  }
  if (cg == 0) p.lse[((int64_t)b * p.Hq + h) * p.Q + row] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

hipError_t launch_fwd_f32(const Params& p, hipStream_t stream) {
  const int n_qt = (p.Q + kF32Rows - 1) / kF32Rows;
  const dim3 grid((unsigned)((int64_t)n_qt * p.Hq * p.B));
  Params arg = p;
  void* args[] = {&arg};
  const void* fn = std::max(p.D, p.Dv) <= 64 ? reinterpret_cast<const void*>(&fwd_f32_kernel<64>)
                                              : reinterpret_cast<const void*>(&fwd_f32_kernel<kF32MaxD>);
  return hipLaunchKernel(fn, grid, dim3(64 * kF32Waves), args, 0, stream);
}

}  // namespace attn
