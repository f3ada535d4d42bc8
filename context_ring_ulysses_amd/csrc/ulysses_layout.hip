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
// Uneven head groups (same guide, "Ulysses Anything Attention" section: the
// head count need not divide by the degree).  With q = H / P and r = H mod P,
// group p holds the Hp_p = q + [p < r] heads starting at h0_p = p*q + min(p, r)
// -- the first r groups one head more, as for uneven ring chunks -- and the
// groups lie back to back: group p is a contiguous [B, S, Hp_p, D] block at
// element B*S*D*h0_p.  With r = 0 this is the [P, B, S, Hp, D] layout.
//
// Memory-bound.  Vectors are numbered in the order of the source: [B, S, H,
// D] for seq2head, [P, B, S, Hp, D] for head2seq, so the reads of a
// workgroup are one contiguous run and the writes land in runs of Hp whole
// rows (Hp*D elements) on the other side.  (Uneven groups are walked in
// [B, S, H, D] order both ways.)  The index decomposition uses
// multiply-high division by the invariant H, S, Hp and B; a thread issues
// all its loads before its stores.  Plain (cached) loads and stores: on
// MI355X they measured faster here than the nontemporal forms.
#include "cru_kernels.h"

namespace cru {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kNV = 2;    // vectors per thread

template <int VPR>   // 16-byte vectors per (token, head) row: 8, 16 or 32
__global__ void __launch_bounds__(kThreads) layout_kernel(const LayoutArgs a) {
  const char* __restrict__ src = static_cast<const char*>(a.src[blockIdx.y]);
  char* __restrict__ dst = static_cast<char*>(a.dst[blockIdx.y]);
  const uint32_t total = (uint32_t)a.B * a.S * a.H * VPR;
  const int Hp = a.H / a.P;
  const int vec_elems = 16 / a.elem_bytes;
  const uint32_t base = blockIdx.x * (kThreads * kNV) + threadIdx.x;

  u32x4 v[kNV];
  int64_t to[kNV];
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    const uint32_t g = base + i * kThreads;
    const uint32_t row = g / VPR;
    const int dv = (int)(g % VPR);
    int b, s, h, p, j;
    int64_t packed_row;           // row of the packed side, in D-element rows
    if (a.uneven) {               // row = (b, s, h) in both directions
      const uint32_t tok = fdiv(row, a.div_h);
      h = (int)(row - tok * a.H);
      b = (int)fdiv(tok, a.div_s);
      s = (int)(tok - (uint32_t)b * a.S);
      const int big = a.rem * (a.quo + 1);          // heads in the larger groups
      p = h < big ? (int)fdiv((uint32_t)h, a.div_q1)
                  : a.rem + (int)fdiv((uint32_t)(h - big), a.div_q);
      const int h0 = p * a.quo + (p < a.rem ? p : a.rem);
      const int hp = a.quo + (p < a.rem ? 1 : 0);
      j = h - h0;
      packed_row = (int64_t)a.B * a.S * h0 + ((int64_t)b * a.S + s) * hp + j;
    } else if (a.dir == 0) {      // row = (b, s, h)
      const uint32_t tok = fdiv(row, a.div_h);
      h = (int)(row - tok * a.H);
      b = (int)fdiv(tok, a.div_s);
      s = (int)(tok - (uint32_t)b * a.S);
      p = (int)fdiv((uint32_t)h, a.div_hp);
      j = h - p * Hp;
    } else {                      // row = (p, b, s, j)
      const uint32_t r1 = fdiv(row, a.div_hp);
      j = (int)(row - r1 * Hp);
      const uint32_t r2 = fdiv(r1, a.div_s);
      s = (int)(r1 - r2 * a.S);
      p = (int)fdiv(r2, a.div_b);
      b = (int)(r2 - (uint32_t)p * a.B);
      h = p * Hp + j;
    }
    if (!a.uneven) packed_row = (((int64_t)p * a.B + b) * a.S + s) * Hp + j;
    const int64_t strided = ((int64_t)b * a.sb + (int64_t)s * a.ss + (int64_t)h * a.sh +
                             (int64_t)dv * vec_elems) * a.elem_bytes;
    const int64_t packed = (packed_row * a.D + (int64_t)dv * vec_elems) * a.elem_bytes;
    const int64_t from = a.dir == 0 ? strided : packed;
    to[i] = a.dir == 0 ? packed : strided;
    v[i] = u32x4{0u, 0u, 0u, 0u};
    if (g < total) v[i] = *reinterpret_cast<const u32x4*>(src + from);
  }
#pragma unroll
  for (int i = 0; i < kNV; ++i)
    if (base + i * kThreads < total)
      *reinterpret_cast<u32x4*>(dst + to[i]) = v[i];
}

template <int VPR>
hipError_t launch_vpr(const LayoutArgs& a, hipStream_t stream) {
  const uint64_t total = (uint64_t)a.B * a.S * a.H * VPR;
  const unsigned gx = (unsigned)((total + kThreads * kNV - 1) / (kThreads * kNV));
  hipLaunchKernelGGL(layout_kernel<VPR>, dim3(gx, a.n), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& args, hipStream_t stream) {
  if ((int64_t)args.B * args.S * args.H * args.D == 0 || args.n == 0) return hipSuccess;
  LayoutArgs a = args;
  a.div_h = make_fastdiv((uint32_t)a.H);
  a.div_s = make_fastdiv((uint32_t)a.S);
  a.quo = a.H / a.P;
  a.rem = a.H % a.P;
  a.uneven = a.rem != 0;
  a.div_hp = make_fastdiv((uint32_t)(a.quo > 0 ? a.quo : 1));
  a.div_b = make_fastdiv((uint32_t)a.B);
  a.div_q = make_fastdiv((uint32_t)(a.quo > 0 ? a.quo : 1));
  a.div_q1 = make_fastdiv((uint32_t)(a.quo + 1));
  const int vpr = a.D * a.elem_bytes / 16;
  switch (vpr) {
    case 8: return launch_vpr<8>(a, stream);
    case 16: return launch_vpr<16>(a, stream);
    case 32: return launch_vpr<32>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cru
