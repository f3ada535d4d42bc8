// LSE merge of partial attention results over disjoint key sets (the fold a
// ring step applies to its running output; diffusers "Parallelism" API page,
// ContextParallelConfig.convert_to_fp32: output and LSE per step, fp32).
//
// Part c covers key set K_c with LSE_c = log sum_{j in K_c} e^{s_j} and
// O_c = sum_{j in K_c} e^{s_j - LSE_c} v_j.  With M = max_c LSE_c and
// w_c = e^{LSE_c - M}:
//   LSE = M + log sum_c w_c,    O = (sum_c w_c O_c) / (sum_c w_c),
// which equals sum_c e^{LSE_c - LSE} O_c; the sums run over c in ascending
// order.  Parts with LSE_c = -inf hold no keys (w_c = 0).
//
// Memory-bound: each part's O row is read once, O and LSE written once.
// One thread owns 4 consecutive elements of one row; rows are ordered
// (b, h, s) with s fastest so the LSE reads and writes of a wave are
// contiguous, and every O row is read as whole 16-byte vectors.
#include "cru_kernels.h"

namespace cru {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int kThreads = 256;
constexpr int kBatch = 8;   // parts whose loads are issued together

template <bool OF32>
__global__ void __launch_bounds__(kThreads) merge_kernel(const MergeArgs a) {
  const int gpr = a.D >> 2;                       // float4 groups per row
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = gid / gpr;
  const int g = (int)(gid - row * gpr);
  const int64_t nrows = (int64_t)a.B * a.H * a.S;
  if (row >= nrows) return;
  const int s = (int)(row % a.S);
  const int64_t bh = row / a.S;
  const int h = (int)(bh % a.H);
  const int b = (int)(bh / a.H);

  const int64_t loff = b * a.pl_sb + h * a.pl_sh + s;
  const int64_t ooff = b * a.p_sb + (int64_t)s * a.p_ss + h * a.p_sh + 4 * g;

  float M = -__builtin_inff();
  for (int c = 0; c < a.n; ++c) M = fmaxf(M, a.l_part[c][loff]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  if (M != -__builtin_inff()) {
    for (int c0 = 0; c0 < a.n; c0 += kBatch) {
      f32x4 x[kBatch];
      float w[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int c = c0 + u;
        if (c < a.n) {
          const float lc = a.l_part[c][loff];
          w[u] = expf(lc - M);                  // 0 for an empty part
          x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (lc != -__builtin_inff()) x[u] = *reinterpret_cast<const f32x4*>(a.o_part[c] + ooff);
        } else {
          x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          w[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        sum += w[u];
        acc[0] = __builtin_fmaf(w[u], x[u][0], acc[0]);
        acc[1] = __builtin_fmaf(w[u], x[u][1], acc[1]);
        acc[2] = __builtin_fmaf(w[u], x[u][2], acc[2]);
        acc[3] = __builtin_fmaf(w[u], x[u][3], acc[3]);
      }
    }
  }
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  const int64_t odst = b * a.o_sb + (int64_t)s * a.o_ss + h * a.o_sh + 4 * g;
  if constexpr (OF32) {
    f32x4 y = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + odst) = y;
  } else {
    bf16x4 y = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv),
                (__bf16)(acc[3] * inv)};
    *reinterpret_cast<bf16x4*>(static_cast<u16*>(a.o) + odst) = y;
  }
  if (g == 0 && a.lse != nullptr)
    a.lse[b * a.l_sb + h * a.l_sh + s] = sum > 0.f ? M + logf(sum) : -__builtin_inff();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.B * a.H * a.S * (a.D / 4);
  if (threads == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
  if (a.o_f32)
    hipLaunchKernelGGL(merge_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cru
