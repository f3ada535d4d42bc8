// LSE merge of partial attention results over disjoint key sets (the fold a
// ring step applies to its running output; diffusers "Parallelism" API page,
// ContextParallelConfig.convert_to_fp32: output and LSE per step, fp32).
//
// Part c covers key set K_c with LSE_c = log sum_{j in K_c} e^{s_j} and
// O_c = sum_{j in K_c} e^{s_j - LSE_c} v_j.  With M = max_c LSE_c and
// w_c = e^{LSE_c - M}:
//   LSE = M + log sum_c w_c,    O = (sum_c w_c O_c) / (sum_c w_c),
// which equals sum_c e^{LSE_c - LSE} O_c; the sums run over c in ascending
// order.  Parts with LSE_c = -inf hold no keys (w_c = 0, their O_c unused).
//
// Partial outputs are fp32 (the default, ContextParallelConfig's
// convert_to_fp32) or bf16, the model dtype, when that conversion is off;
// the LSEs are fp32 either way and the sums are fp32.
//
// Memory-bound: each part's O row is read once, O and LSE written once.
// One thread owns VPT groups of 4 elements of one row and reads each part
// with one 16-byte load (VPT = 1 for fp32 parts, 2 for bf16 parts).  Rows
// are ordered (b, s, h) with h fastest, the order of [B, S, H, D] memory, so
// a workgroup reads one contiguous run of every part (the few strided LSE reads are cache-resident
// and reused by neighbouring workgroups).  All of a thread's loads are
// issued before the first use: the part loop is unrolled over a
// compile-time bound with wave-uniform predicates, so nothing waits on an
// earlier load to decide whether to issue the next.  Loads are ordinary
// (cached) loads and the output stores are nontemporal: on MI355X that pair
// measured fastest for this many-stream read, one-stream write pattern.
#include "cru_kernels.h"

namespace cru {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 64;   // one wave per workgroup: measured fastest (vs 128, 256, 512)
constexpr int kBatch = 16;    // parts loaded at once by the generic kernel
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;

struct RowPos {
  int b, h, s, g;
  bool live;
};

template <int VPT>
__device__ __forceinline__ RowPos row_pos(const MergeArgs& a) {
  const int gpr = (a.D >> 2) / VPT;                      // threads per row (power of 2)
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t row = gid >> __builtin_ctz(gpr);
  RowPos p;
  p.g = (int)(gid - row * gpr);
  p.live = row < (uint32_t)a.B * a.H * a.S;
  const uint32_t bs = fdiv(row, a.div_h);
  p.h = (int)(row - bs * a.H);
  p.b = (int)fdiv(bs, a.div_s);
  p.s = (int)(bs - p.b * a.S);
  return p;
}

// 4 elements of a partial output, as fp32
template <bool PBF16>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t off) {
  if constexpr (PBF16) {
    const u16x4 x = *reinterpret_cast<const u16x4*>(static_cast<const u16*>(base) + off);
    // bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits
    return f32x4{__uint_as_float((unsigned)x[0] << 16), __uint_as_float((unsigned)x[1] << 16),
                 __uint_as_float((unsigned)x[2] << 16), __uint_as_float((unsigned)x[3] << 16)};
  } else {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
  }
}

template <int VPT, bool OF32>
__device__ __forceinline__ void store_row(const MergeArgs& a, const RowPos& p,
                                          const f32x4 (&acc)[VPT], float inv, float lse) {
  const int64_t odst = p.b * a.o_sb + (int64_t)p.s * a.o_ss + p.h * a.o_sh + 4 * VPT * p.g;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    if constexpr (OF32) {
      f32x4 y = {acc[u][0] * inv, acc[u][1] * inv, acc[u][2] * inv, acc[u][3] * inv};
      __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + odst + 4 * u));
    } else {
      bf16x4 y = {(__bf16)(acc[u][0] * inv), (__bf16)(acc[u][1] * inv),
                  (__bf16)(acc[u][2] * inv), (__bf16)(acc[u][3] * inv)};
      __builtin_nontemporal_store(y, reinterpret_cast<bf16x4*>(static_cast<u16*>(a.o) + odst + 4 * u));
    }
  }
  if (p.g == 0 && a.lse != nullptr) a.lse[p.b * a.l_sb + p.h * a.l_sh + p.s] = lse;
}

// n <= NMAX parts, everything in registers.
template <int NMAX, int VPT, bool OF32, bool PBF16>
__global__ void __launch_bounds__(kThreads) merge_small(const MergeArgs a) {
  const RowPos p = row_pos<VPT>(a);
  if (!p.live) return;
  const int64_t loff = p.b * a.pl_sb + p.h * a.pl_sh + p.s;
  const int64_t ooff = p.b * a.p_sb + (int64_t)p.s * a.p_ss + p.h * a.p_sh + 4 * VPT * p.g;

  float l[NMAX];
  f32x4 x[NMAX][VPT];
#pragma unroll
  for (int c = 0; c < NMAX; ++c)
    l[c] = c < a.n ? a.l_part[c][loff] : -__builtin_inff();
#pragma unroll
  for (int c = 0; c < NMAX; ++c) {
    if constexpr (PBF16 && VPT == 2) {
      // 8 bf16 elements in one 16-byte load, widened exactly
      u32x4 w = {0u, 0u, 0u, 0u};
      if (c < a.n) w = *reinterpret_cast<const u32x4*>(static_cast<const u16*>(a.o_part[c]) + ooff);
      x[c][0] = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                      __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
      x[c][VPT - 1] = f32x4{__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                            __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u)};
    } else {
#pragma unroll
      for (int u = 0; u < VPT; ++u)
        x[c][u] = c < a.n ? load4<PBF16>(a.o_part[c], ooff + 4 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  float M = l[0];
#pragma unroll
  for (int c = 1; c < NMAX; ++c) M = fmaxf(M, l[c]);
  f32x4 acc[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  if (M != -__builtin_inff()) {
#pragma unroll
    for (int c = 0; c < NMAX; ++c) {
      const float w = __builtin_amdgcn_exp2f((l[c] - M) * kLog2e);   // 0 for an empty part
      if (w > 0.f) {
        sum += w;
#pragma unroll
        for (int u = 0; u < VPT; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[u][e] = __builtin_fmaf(w, x[c][u][e], acc[u][e]);
      }
    }
  }
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  const float lse = sum > 0.f ? M + __builtin_amdgcn_logf(sum) * kLn2 : -__builtin_inff();
  store_row<VPT, OF32>(a, p, acc, inv, lse);
}

// Any n: a first pass over the LSEs for the max, then batches of kBatch parts.
template <bool OF32, bool PBF16>
__global__ void __launch_bounds__(kThreads) merge_many(const MergeArgs a) {
  const RowPos p = row_pos<1>(a);
  if (!p.live) return;
  const int64_t loff = p.b * a.pl_sb + p.h * a.pl_sh + p.s;
  const int64_t ooff = p.b * a.p_sb + (int64_t)p.s * a.p_ss + p.h * a.p_sh + 4 * p.g;

  float M = -__builtin_inff();
  for (int c0 = 0; c0 < a.n; c0 += kBatch) {
    float l[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      l[u] = c0 + u < a.n ? a.l_part[c0 + u][loff] : -__builtin_inff();
#pragma unroll
    for (int u = 0; u < kBatch; ++u) M = fmaxf(M, l[u]);
  }
  f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
  float sum = 0.f;
  if (M != -__builtin_inff()) {
    for (int c0 = 0; c0 < a.n; c0 += kBatch) {
      float l[kBatch];
      f32x4 x[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const bool in = c0 + u < a.n;
        l[u] = in ? a.l_part[c0 + u][loff] : -__builtin_inff();
        x[u] = in ? load4<PBF16>(a.o_part[c0 + u], ooff) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float w = __builtin_amdgcn_exp2f((l[u] - M) * kLog2e);
        if (w > 0.f) {
          sum += w;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[0][e] = __builtin_fmaf(w, x[u][e], acc[0][e]);
        }
      }
    }
  }
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  const float lse = sum > 0.f ? M + __builtin_amdgcn_logf(sum) * kLn2 : -__builtin_inff();
  store_row<1, OF32>(a, p, acc, inv, lse);
}

template <int NMAX, bool OF32, bool PBF16>
hipError_t launch_small(const MergeArgs& a, hipStream_t stream) {
  // fp32 parts: 4 elements (one 16-byte load per part) per thread; bf16
  // parts: 8 elements, so their loads are 16 bytes too (measured 13% faster
  // than two 8-byte halves)
  constexpr int VPT = PBF16 ? 2 : 1;
  const int64_t threads = (int64_t)a.B * a.H * a.S * (a.D / 4 / VPT);
  const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
  hipLaunchKernelGGL((merge_small<NMAX, VPT, OF32, PBF16>), dim3(blocks), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <bool OF32, bool PBF16>
hipError_t launch_of(const MergeArgs& a, hipStream_t stream) {
  if (a.n <= 2) return launch_small<2, OF32, PBF16>(a, stream);
  if (a.n <= 4) return launch_small<4, OF32, PBF16>(a, stream);
  if (a.n <= 8) return launch_small<8, OF32, PBF16>(a, stream);
  if (a.n <= 16) return launch_small<16, OF32, PBF16>(a, stream);
  const int64_t threads = (int64_t)a.B * a.H * a.S * (a.D / 4);
  const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
  hipLaunchKernelGGL((merge_many<OF32, PBF16>), dim3(blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& args, hipStream_t stream) {
  const int64_t rows = (int64_t)args.B * args.H * args.S;
  if (rows == 0) return hipSuccess;
  MergeArgs a = args;
  a.div_s = make_fastdiv((uint32_t)a.S);
  a.div_h = make_fastdiv((uint32_t)a.H);
  if (a.p_bf16) return a.o_f32 ? launch_of<true, true>(a, stream) : launch_of<false, true>(a, stream);
  return a.o_f32 ? launch_of<true, false>(a, stream) : launch_of<false, false>(a, stream);
}

}  // namespace cru
