// Softmax attention forward with per-row LSE in fp32 throughout (fp32
// inputs, fp32 products and sums, no reduced-precision matrix mode), for the
// cases that need single-precision results; same maths and split handling as
// the bf16 kernel (diffusers "Attention backends" page, "Available backends":
// scaled_dot_product_attention; diffusers "Parallelism" API page,
// ContextParallelConfig.convert_to_fp32 for the per-split output and LSE).
//
// One thread owns one query row: its q (D floats) and its O accumulator stay
// in registers.  A workgroup of 128 threads shares K/V tiles of 32 keys in
// LDS; every thread reads the same key at the same time (an LDS broadcast).
// Per tile the 32 scores are formed first, the running max is updated once,
// then the tile's probabilities are folded into O.
#include "cru_kernels.h"

namespace cru {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 128;   // query rows (threads) per workgroup
constexpr int kKeys = 32;    // keys per LDS tile
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
__global__ void __launch_bounds__(kRows) attn_fwd_f32_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float ks[kKeys][D];
  __shared__ __attribute__((aligned(16))) float vs[kKeys][D];

  const int tid = threadIdx.x;
  const int nqt = (a.Sq + kRows - 1) / kRows;
  const int qt = blockIdx.x % nqt;
  int rest = blockIdx.x / nqt;
  const int h = rest % a.H;
  rest /= a.H;
  const int b = rest % a.B;
  const int split = rest / a.B;
  const int kv0 = a.split_start[split];
  const int kv1 = a.split_start[split + 1];
  const int row = qt * kRows + tid;

  const float* qg = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh;
  const float* kg = static_cast<const float*>(a.k) + b * a.k_sb + h * a.k_sh;
  const float* vg = static_cast<const float*>(a.v) + b * a.v_sb + h * a.v_sh;

  float q[D];
  float o[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (row < a.Sq) x = *reinterpret_cast<const f32x4*>(qg + (int64_t)row * a.q_ss + d);
    q[d] = x[0]; q[d + 1] = x[1]; q[d + 2] = x[2]; q[d + 3] = x[3];
    o[d] = o[d + 1] = o[d + 2] = o[d + 3] = 0.f;
  }
  float m = -__builtin_inff();   // running max of s * scale * log2(e)
  float l = 0.f;

  constexpr int kVec = D / 4;                  // float4s per row
  for (int base = kv0; base < kv1; base += kKeys) {
    const int n = min(kKeys, kv1 - base);
    __syncthreads();
    for (int c = tid; c < kKeys * kVec; c += kRows) {
      const int r = c / kVec, col = (c % kVec) * 4;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (r < n) {
        kx = *reinterpret_cast<const f32x4*>(kg + (int64_t)(base + r) * a.k_ss + col);
        vx = *reinterpret_cast<const f32x4*>(vg + (int64_t)(base + r) * a.v_ss + col);
      }
      *reinterpret_cast<f32x4*>(&ks[r][col]) = kx;
      *reinterpret_cast<f32x4*>(&vs[r][col]) = vx;
    }
    __syncthreads();

    float s[kKeys];
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], ks[j][d], acc);
      s[j] = j < n ? acc : -__builtin_inff();
      mx = fmaxf(mx, s[j]);
    }
    const float mn = fmaxf(m, mx * a.scale_log2);
    const float alpha = exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
    m = mn;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = exp2f(__builtin_fmaf(s[j], a.scale_log2, -m));
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, vs[j][d], o[d]);
    }
  }

  if (row < a.Sq) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    float* og = static_cast<float*>(a.o) + split * a.o_split_stride + b * a.o_sb +
                (int64_t)row * a.o_ss + h * a.o_sh;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      f32x4 x = {o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv};
      *reinterpret_cast<f32x4*>(og + d) = x;
    }
    if (a.lse != nullptr)
      a.lse[split * a.l_split_stride + b * a.l_sb + h * a.l_sh + row] =
          l > 0.f ? (m + log2f(l)) * kLn2 : -__builtin_inff();
  }
}

template <int D>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  const int nqt = (a.Sq + kRows - 1) / kRows;
  const long total = (long)a.n_split * a.B * a.H * nqt;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3((unsigned)total), dim3(kRows), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.D == 128) return launch<128>(a, stream);
  if (a.D == 64) return launch<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cru
