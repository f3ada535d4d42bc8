// Blockwise softmax attention forward with per-row LSE, bf16 inputs, for
// CDNA4 (gfx950) matrix cores.
//
// What is computed: O = softmax(Q K^T * scale) V and LSE = log sum_j
// exp(s_ij), non-causal and unmasked (diffusers "Attention backends" page,
// "Available backends": scaled_dot_product_attention is the default
// backend), over one or several key ranges ("splits").  Each split's
// (O, LSE) is what one ring step produces (diffusers "Parallelism" API page,
// ContextParallelConfig.convert_to_fp32: output and LSE are carried per step).
// The tiling with a running max and sum is the FlashAttention technique the
// "Attention backends" page names (tiling so the score matrix never reaches
// memory).
//
// Work decomposition
//   workgroup = 4 waves = one tile of 128 query rows of one (split, b, h);
//   wave      = 32 query rows; lane (i = lane%32, half = lane/32).
//   Key tiles of BC = 8192/D keys are staged in LDS, double buffered:
//   K row-major (rows permuted, below), V transposed (V^T[d][key]).
//
// The contraction is written as S^T = K Q^T with v_mfma_f32_32x32x16_bf16:
// A = 32 keys x 16 dims of K (from LDS), B = 16 dims x 32 queries of Q^T
// (held in registers for the whole key loop).  The accumulator layout of a
// 32x32 MFMA gives lane (i, half) the column i -- one query row -- and rows
// 8*(r/4) + 4*half + r%4 for its 16 registers r.  So every lane owns one
// query row: the running max, the sum and the O rescale factor are per-lane
// scalars, and only the two halves of a row need one exchange per tile.
//
// O^T = V^T P^T then uses A = 32 dims x 16 keys of V^T (LDS) and B = P^T,
// which the lane already holds in its S^T registers.  For registers 0..7
// (and 8..15) of a 32-key block to be the B operand of one MFMA, the keys they
// hold must be 8 consecutive keys per half.  Register r of half h holds MFMA
// row rho = 8*(r/4) + 4*h + r%4; storing key j of the tile in LDS row pi(j),
// with pi swapping bits 2 and 3, makes that row hold key
//   16*(r/8) + 8*h + r%8,
// so half h of MFMA #(r/8) holds keys 16*(r/8) + 8*h + 0..7: one 16-byte
// read of V^T.  Softmax is invariant to the order of keys, so the permutation
// only has to be the same for K and V, which it is by construction.
//
// Rescaling is lazy: the running max m (in log2 units) only moves when some
// row's tile max exceeds it by more than kTau; otherwise P = 2^(x - m) may
// reach 2^kTau, which fp32 sums and bf16 P hold exactly as well as values
// below 1.  The final O / l and LSE = (m + log2 l) ln 2 are exact either way.
#include "cru_kernels.h"

namespace cru {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr int kThreads = 256;
constexpr float kTau = 8.0f;
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
struct Tile {
  static constexpr int BC = 8192 / D;          // keys per tile
  static constexpr int BM = 128;               // query rows per workgroup
  static constexpr int KP = D + 8;             // LDS pitch of a K row (elements)
  static constexpr int VP = BC + 8;            // LDS pitch of a V^T row
  static constexpr int K_LDS = BC * KP;
  static constexpr int V_LDS = D * VP;
  static constexpr int STAGE = K_LDS + V_LDS;  // one buffer
  static constexpr int NJ = BC / 32;           // 32-key blocks per tile
  static constexpr int NK = D / 16;            // 16-wide steps of the QK^T contraction
  static constexpr int ND = D / 32;            // 32-wide blocks of O columns
  static constexpr int KCH = D / 8;            // 16-byte chunks per row
  static constexpr int KLOADS = BC * KCH / kThreads;
  static constexpr int VJG = BC / 4;           // groups of 4 keys for the V transpose
  static_assert(KLOADS * kThreads == BC * KCH, "tile must split evenly");
  static_assert(VJG * KCH == kThreads, "one 4-key x 8-dim block per thread");
};

__device__ __forceinline__ int key_row(int j) {
  // swap bits 2 and 3 of the key index (an involution)
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ u32x4 ld16(const u16* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) {
  return __builtin_bit_cast(bf16x8, x);
}

template <int D, bool OF32>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_bf16_kernel(const AttnArgs a) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) u16 lds[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int lh = lane >> 5;

  // Workgroup -> (split, b, h, query tile).  Workgroups are dealt to the 8
  // XCDs round robin; renumber so that consecutive logical tiles (the tiles
  // of one head, which share that head's K/V) land on the same XCD and its L2.
  const int nqt = (a.Sq + T::BM - 1) / T::BM;
  const int total = a.n_split * a.B * a.H * nqt;
  int id = blockIdx.x;
  {
    const int xcd = id & 7, local = id >> 3, per = total >> 3, rem = total & 7;
    id = xcd * per + (xcd < rem ? xcd : rem) + local;
  }
  const int qt = id % nqt;
  int rest = id / nqt;
  const int h = rest % a.H;
  rest /= a.H;
  const int b = rest % a.B;
  const int split = rest / a.B;
  const int kv0 = a.split_start[split];
  const int kv1 = a.split_start[split + 1];

  const u16* qg = static_cast<const u16*>(a.q) + b * a.q_sb + h * a.q_sh;
  const u16* kg = static_cast<const u16*>(a.k) + b * a.k_sb + h * a.k_sh;
  const u16* vg = static_cast<const u16*>(a.v) + b * a.v_sb + h * a.v_sh;

  // Q^T fragments for this lane's query row, kept for the whole key loop.
  const int row = qt * T::BM + wave * 32 + li;
  bf16x8 qf[T::NK];
#pragma unroll
  for (int ks = 0; ks < T::NK; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row < a.Sq) x = ld16(qg + (int64_t)row * a.q_ss + ks * 16 + lh * 8);
    qf[ks] = as_bf16x8(x);
  }

  f32x16 oacc[T::ND];
#pragma unroll
  for (int db = 0; db < T::ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m = -__builtin_inff();   // running max of s * scale * log2(e)
  float l = 0.0f;                // this half-lane's share of the running sum

  const int nkv = kv1 - kv0;
  const int ntiles = (nkv + T::BC - 1) / T::BC;

  // Global -> register staging of one K/V tile.
  u32x4 kreg[T::KLOADS];
  u32x4 vreg[4];
  const int vjg = tid % T::VJG;   // V: keys 4*vjg .. 4*vjg+3
  const int vdc = tid / T::VJG;   //    dims 8*vdc .. 8*vdc+7
  auto gload = [&](int t) {
    const int base = kv0 + t * T::BC;
#pragma unroll
    for (int it = 0; it < T::KLOADS; ++it) {
      const int c = it * kThreads + tid;
      const int r = c / T::KCH, col = c % T::KCH;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (base + r < kv1) x = ld16(kg + (int64_t)(base + r) * a.k_ss + col * 8);
      kreg[it] = x;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = base + 4 * vjg + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < kv1) x = ld16(vg + (int64_t)key * a.v_ss + vdc * 8);
      vreg[r] = x;
    }
  };
  auto lstore = [&](int buf) {
    u16* ks = lds + buf * T::STAGE;
    u16* vt = ks + T::K_LDS;
#pragma unroll
    for (int it = 0; it < T::KLOADS; ++it) {
      const int c = it * kThreads + tid;
      const int r = c / T::KCH, col = c % T::KCH;
      *reinterpret_cast<u32x4*>(ks + key_row(r) * T::KP + col * 8) = kreg[it];
    }
    // 4 keys x 8 dims -> 8 rows of V^T, 4 keys each
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      unsigned lo, hi;
      if (e & 1) {
        lo = (vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u);
        hi = (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u);
      } else {
        lo = (vreg[0][w] & 0xffffu) | (vreg[1][w] << 16);
        hi = (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16);
      }
      u32x2 pair = {lo, hi};
      *reinterpret_cast<u32x2*>(vt + (vdc * 8 + e) * T::VP + 4 * vjg) = pair;
    }
  };

  if (ntiles > 0) gload(0);
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    lstore(buf);
    __syncthreads();
    if (t + 1 < ntiles) gload(t + 1);
    const u16* ks = lds + buf * T::STAGE;
    const u16* vt = ks + T::K_LDS;

    // S^T = K Q^T for NJ blocks of 32 keys
    f32x16 s[T::NJ];
#pragma unroll
    for (int jb = 0; jb < T::NJ; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[jb][r] = 0.0f;
#pragma unroll
      for (int k = 0; k < T::NK; ++k) {
        const bf16x8 kf = as_bf16x8(ld16(ks + (jb * 32 + li) * T::KP + k * 16 + lh * 8));
        s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[k], s[jb], 0, 0, 0);
      }
    }

    // keys past the end of the range do not exist
    const int valid = nkv - t * T::BC;
    if (valid < T::BC) {
#pragma unroll
      for (int jb = 0; jb < T::NJ; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = jb * 32 + 16 * (r >> 3) + 8 * lh + (r & 7);
          if (key >= valid) s[jb][r] = -__builtin_inff();
        }
    }

    // online softmax: tile max of this row (both halves), lazy rescale
    float mx = s[0][0];
#pragma unroll
    for (int jb = 0; jb < T::NJ; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxs = mx * a.scale_log2;
    if (__ballot(mxs > m + kTau) != 0ull) {
      const float mn = fmaxf(m, mxs);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < T::ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m = mn;
    }

    // P = 2^(s*scale*log2e - m), rounded to bf16 for the P V product
    bf16x8 pf[T::NJ][2];
#pragma unroll
    for (int jb = 0; jb < T::NJ; ++jb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jb][hf * 8 + t8], a.scale_log2, -m));
          l += p;
          pf[jb][hf][t8] = (__bf16)p;
        }

    // O^T += V^T P^T
#pragma unroll
    for (int jb = 0; jb < T::NJ; ++jb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < T::ND; ++db) {
          const bf16x8 vf = as_bf16x8(ld16(vt + (db * 32 + li) * T::VP + jb * 32 + hf * 16 + lh * 8));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[jb][hf], oacc[db], 0, 0, 0);
        }
  }

  // epilogue: O = O_acc / l, LSE = (m + log2 l) ln 2; no keys -> O = 0, -inf
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  const float lse = lt > 0.0f ? (m + log2f(lt)) * kLn2 : -__builtin_inff();
  if (row < a.Sq) {
    const int64_t obase = split * a.o_split_stride + b * a.o_sb + (int64_t)row * a.o_ss + h * a.o_sh;
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * lh;
        if constexpr (OF32) {
          f32x4 x = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                     oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + obase + d0) = x;
        } else {
          bf16x4 x = {(__bf16)(oacc[db][4 * g] * inv), (__bf16)(oacc[db][4 * g + 1] * inv),
                      (__bf16)(oacc[db][4 * g + 2] * inv), (__bf16)(oacc[db][4 * g + 3] * inv)};
          *reinterpret_cast<bf16x4*>(static_cast<u16*>(a.o) + obase + d0) = x;
        }
      }
    if (lh == 0 && a.lse != nullptr)
      a.lse[split * a.l_split_stride + b * a.l_sb + h * a.l_sh + row] = lse;
  }
}

template <int D, bool OF32>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  using T = Tile<D>;
  const int nqt = (a.Sq + T::BM - 1) / T::BM;
  const long total = (long)a.n_split * a.B * a.H * nqt;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, OF32>), dim3((unsigned)total), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.o_f32 ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  if (a.D == 64) return a.o_f32 ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cru
