// Ulysses sequence<->head regrouping on one device (diffusers "Context
// parallelism" guide, "Ulysses Attention" section: the first all-to-all
// leaves each device with every token of a subset of heads, the second
// regroups the results by token).
//
// seq2head: y[p, b, s, j, d] = x[b, s, p*Hp + j, d],  Hp = H / P
// head2seq: x[b, s, p*Hp + j, d] = y[p, b, s, j, d]
// The [B, S, H, D] side may be strided (d contiguous); the [P, B, S, Hp, D]
// side is contiguous.  Pure bit-exact copies, moved 16 bytes at a time.
//
// Memory-bound.  A workgroup owns a run of consecutive tokens of one batch
// of one tensor; each (token, head) row of D elements is a contiguous run on
// both sides, and the Hp rows of one group are contiguous on the y side, so
// every wave reads and writes whole contiguous runs.
#include "cru_kernels.h"

namespace cru {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <int VPR>   // 16-byte vectors per (token, head) row
__global__ void __launch_bounds__(kThreads) layout_kernel(const LayoutArgs a, int tokens_per_block) {
  const int t = blockIdx.z;                       // tensor
  const int b = blockIdx.y;
  const int s0 = blockIdx.x * tokens_per_block;
  const int ntok = min(tokens_per_block, a.S - s0);
  const int Hp = a.H / a.P;
  const int vec_elems = 16 / a.elem_bytes;
  const char* src = static_cast<const char*>(a.src[t]);
  char* dst = static_cast<char*>(a.dst[t]);
  const int work = ntok * a.H * VPR;
  for (int u = threadIdx.x; u < work; u += kThreads) {
    const int dv = u % VPR;                       // VPR is a power of two
    const int rowi = u / VPR;
    const int h = rowi % a.H;
    const int s = s0 + rowi / a.H;
    const int p = h / Hp;
    const int j = h - p * Hp;
    const int64_t strided = (int64_t)b * a.sb + (int64_t)s * a.ss + (int64_t)h * a.sh +
                            (int64_t)dv * vec_elems;
    const int64_t packed = ((((int64_t)p * a.B + b) * a.S + s) * Hp + j) * a.D +
                           (int64_t)dv * vec_elems;
    const int64_t from = (a.dir == 0 ? strided : packed) * a.elem_bytes;
    const int64_t to = (a.dir == 0 ? packed : strided) * a.elem_bytes;
    *reinterpret_cast<u32x4*>(dst + to) = *reinterpret_cast<const u32x4*>(src + from);
  }
}

template <int VPR>
hipError_t launch_vpr(const LayoutArgs& a, hipStream_t stream) {
  // about 2048 vectors per workgroup
  const int per_token = a.H * VPR;
  int tpb = 2048 / per_token;
  if (tpb < 1) tpb = 1;
  const unsigned gx = (unsigned)((a.S + tpb - 1) / tpb);
  hipLaunchKernelGGL(layout_kernel<VPR>, dim3(gx, a.B, a.n), dim3(kThreads), 0, stream, a, tpb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
  if ((int64_t)a.B * a.S * a.H * a.D == 0 || a.n == 0) return hipSuccess;
  const int vpr = a.D * a.elem_bytes / 16;
  switch (vpr) {
    case 8: return launch_vpr<8>(a, stream);
    case 16: return launch_vpr<16>(a, stream);
    case 32: return launch_vpr<32>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cru
