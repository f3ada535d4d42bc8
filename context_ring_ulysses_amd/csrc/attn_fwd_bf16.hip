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
//   workgroup = W waves = one tile of 32*W query rows of one (split, b, h);
//               W = 8 (two waves on each of the CU's four SIMDs) for large
//               launches, 4 or 2 where that leaves fewer idle CUs or rows;
//   wave      = 32 query rows; lane (i = lane%32, half = lane/32).
//   Key tiles of 64 keys go from global memory straight into LDS (buffer
//   loads with the LDS destination bit: 64 lanes write 1 KiB contiguously,
//   each lane choosing its 16-byte source), so no registers or VALU work
//   stage them.  Both K and V are kept row-major in LDS, XOR-swizzled at
//   16-byte granularity so the reads below hit distinct banks.
//
// The contraction is written as S^T = K Q^T with v_mfma_f32_32x32x16_bf16:
// A = 32 keys x 16 dims of K (from LDS), B = 16 dims x 32 queries of Q^T
// (held in registers for the whole key loop).  The accumulator layout of a
// 32x32 MFMA gives lane (i, half) the column i -- one query row -- and rows
// 8*(r/4) + 4*half + r%4 for its 16 registers r.  So every lane owns one
// query row: the running max, the sum and the O rescale factor are per-lane
// scalars, and the two halves of a row meet only in the epilogue and when the
// running max moves.
//
// O^T = V^T P^T then uses A = 32 dims x 16 keys of V^T and B = P^T, which the
// lane already holds in its S^T registers.  For registers 0..7 (and 8..15)
// of a 32-key block to be the B operand of one MFMA, the keys they hold must
// be 8 consecutive keys per half.  Register r of half h holds MFMA row
// rho = 8*(r/4) + 4*h + r%4; storing key j of the tile in LDS row pi(j),
// with pi swapping bits 2 and 3, makes that row hold key
//   16*(r/8) + 8*h + r%8,
// so half h of MFMA #(r/8) holds keys 16*(r/8) + 8*h + 0..7.  Softmax is
// invariant to the order of keys, so the permutation only has to be the same
// for K and V, which it is by construction.  The A operand of V^T (row d,
// 8 consecutive keys per lane) is read from row-major V with two
// ds_read_b64_tr_b16: within a group of 16 lanes that instruction hands lane
// j element 16e + j of the 16 x 4 block the lanes point at, so pointing lane
// i at V[key0 + i/4][d0 + 4*(i%4) ..] gives lane j the 4 keys
// key0 .. key0+3 of column d0 + j.
//
// Software pipeline.  K and V have two LDS buffers each, one tile apart: in
// the iteration for tile t the waves compute S^T of tile t (K buffer t%2)
// and the P V product of tile t-1 (V buffer (t-1)%2), while the loads of K of
// tile t+1 and V of tile t fill the other two buffers.  One barrier per tile
// separates them.  The softmax runs half a tile behind the scores, by 32-key
// blocks: beside the QK^T of tile t each wave exponentiates the second block
// of tile t-1 (whose S^T it kept), and beside the P V of tile t-1 the first
// block of tile t.  So each of the two matrix phases has vector work of the
// same wave to interleave with: the matrix cores overlap a wave's own vector
// work, hardly the other wave's on the SIMD.  Global loads go through buffer descriptors built per tile
// whose range ends at the last valid key row: rows past it read as zero
// with no per-load bounds arithmetic.
//
// The running max m is kept in log2 units (scores times scale*log2(e)), so
// P = 2^(x - m) is one FMA and one v_exp_f32 per score.  Rescaling is lazy
// and no max is computed on the common path: each 32-key block is
// exponentiated against the current m, and only if some half-row's running
// sum of P, this block's included, passes kSumCap = 2^32 (the sum bounds
// every P of the block, an overflow to inf included) does the wave take the
// rare path that finds the block max, moves m there (and past the log2 of
// the row's sum so far) and exponentiates the block again.  Any m gives
// the same O and LSE up to rounding (fp32 and bf16 keep their relative
// precision at any scale below overflow); the cap keeps P, l and O from the
// fp32 limit: a half-row's sum stays below 2^32 between moves, so O's
// accumulator (both halves, about 2^33 max|V|) is finite for max|V| < 2^90.
// The first tile sets m to its own max.  A move at a tile's first block
// comes after the P V of the tile before it was issued: the 64-register
// rescale of O it owes is settled at the start of the next tile, ahead of
// its QK^T, so the branch never splits a phase the compiler interleaves.  A
// move at the previous tile's second block (beside QK^T) rescales O and that
// tile's first-block P (already bf16, rounded again) before the P V.
// P is rounded to bf16 for the P V product, and O is normalised by the sum
// of those same rounded values (taken by the matrix cores beside O), so O's
// weights sum to one and a row that one key dominates keeps that key's
// rounding out of O.  The LSE takes the sum of the fp32 P, which the
// rounding would otherwise bias by up to 2^-9.
#include "attn_shape.h"
#include "cru_kernels.h"

namespace cru {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr float kSumCap = 4294967296.0f;   // 2^32: bound on a half-row's tile sum of P
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int kWaitVmem = 0x0F70;        // s_waitcnt vmcnt(0), other counters not waited

template <int D, int W>
struct Tile {
  static constexpr int kWaves = W;             // waves per workgroup
  static constexpr int kThreads = 64 * W;
  static constexpr int BC = 64;                // keys per tile
  static constexpr int BM = 32 * W;            // query rows per workgroup
  static constexpr int RB = 2 * D;             // bytes per K or V row in LDS
  static constexpr int KCH = D / 8;            // 16-byte chunks per row
  static constexpr int NJ = BC / 32;           // 32-key blocks per tile
  static constexpr int NK = D / 16;            // 16-wide steps of the QK^T contraction
  static constexpr int ND = D / 32;            // 32-wide blocks of O columns
  static constexpr int TILE_BYTES = BC * RB;   // one K or V tile
  static constexpr int NLOAD = TILE_BYTES / (kThreads * 16);   // 16-byte loads per thread
  static_assert(NLOAD * kThreads * 16 == TILE_BYTES, "tile must split evenly");
  // K row R (LDS row, holding key key_row(R)) keeps logical chunk c at
  // physical chunk c ^ kx(R): rows read together by one 16-lane group of the
  // QK^T operand fetch land on 16 distinct 16-byte bank groups.
  static __device__ __forceinline__ int kx(int R) {
    return D == 128 ? (R & 15) : ((R >> 1) & 7);
  }
  // V row (key) k keeps logical chunk c at c ^ vx(k): the 4 keys x 64 bytes
  // one transposing read fetches per half-wave land on distinct banks.
  static __device__ __forceinline__ int vx(int k) {
    return D == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
  }
};

struct NotFirst { static constexpr bool value = false; };
struct First { static constexpr bool value = true; };
struct NotLast { static constexpr int value = 0; };
struct Last { static constexpr int value = 1; };
struct MaybeLast { static constexpr int value = 2; };   // decided at run time

__device__ __forceinline__ int key_row(int j) {
  // swap bits 2 and 3 of the key index (an involution)
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) {
  return __builtin_bit_cast(bf16x8, x);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 lds_read16(const char* base, int byte_off) {
  return *reinterpret_cast<const u32x4*>(base + byte_off);
}

__device__ __forceinline__ v4i16 lds_read_tr(const char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(base + byte_off));
}

template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const u16* base, int64_t row0,
                                                           int64_t row_stride, int nrows, int cap) {
  // rows [row0, row0 + min(nrows, cap)) of a strided [rows, D] bf16 matrix:
  // the range ends with the last element of the last row, so a stride below
  // D (rows that overlap, or a stride-0 broadcast) still reads every row; the
  // host guarantees cap * row_stride * 2 < 2^31
  const u16* p = base + row0 * row_stride;
  const int n = nrows < cap ? nrows : cap;
  const int bytes = n > 0 ? (int)(((n - 1) * row_stride + D) * 2) : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(p), (short)0, bytes, kRsrcWord3);
}

template <int D, bool OF32, int W>
__global__ void __launch_bounds__(64 * W)
__attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_bf16_kernel(const AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  // The body is compiled for the device only; the host pass needs just the
  // signature for the launch stub (it cannot type-check the gfx950 LDS
  // builtins used below).
  using T = Tile<D, W>;
  constexpr int kWaves = W;
  __shared__ __attribute__((aligned(1024))) char kbuf0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf1[T::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keep it scalar
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
  const u16* kg = static_cast<const u16*>(a.k) + b * a.k_sb + h * a.k_sh + kv0 * a.k_ss;
  const u16* vg = static_cast<const u16*>(a.v) + b * a.v_sb + h * a.v_sh + kv0 * a.v_ss;

  // Q^T fragments for this lane's query row, kept for the whole key loop.
  const int row = qt * T::BM + wave * 32 + li;
  bf16x8 qf[T::NK];
  {
    const __amdgpu_buffer_rsrc_t qr =
        rows_rsrc<D>(qg, (int64_t)qt * T::BM, a.q_ss, a.Sq - qt * T::BM, T::BM);
    const int qoff = ((wave * 32 + li) * (int)a.q_ss + lh * 8) * 2;
#pragma unroll
    for (int ks = 0; ks < T::NK; ++ks)
      qf[ks] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(qr, qoff + ks * 32, 0, 0));
  }

  f32x16 oacc[T::ND];
#pragma unroll
  for (int db = 0; db < T::ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m = -__builtin_inff();   // running max of s * scale * log2(e)
  float l = 0.0f;                // this half-lane's share of the running sum of P
  // Sum of the P rounded to bf16 (O's normaliser), accumulated by the matrix
  // cores beside O: a 16x16x32 product of a 0/1 pattern with the P^T
  // registers leaves every lane its own row's sum in all four registers.
  f32x4 lbacc = {0.0f, 0.0f, 0.0f, 0.0f};
  // The pattern: lane (row mm = lane%16, k block kk = lane/16) of the A
  // operand is 1 where (mm/4) and kk have the same parity.  Lane l of a
  // P^T register holds query l%32 and k block l/16 carries queries n and
  // n+16 alternately, so output row 4*(l/16)+r of column l%16 sums exactly
  // the keys of query l%32 (the lane's own row).
  const bf16x8 ones_pat = [&] {
    const __bf16 x = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? (__bf16)1.0f : (__bf16)0.0f;
    return bf16x8{x, x, x, x, x, x, x, x};
  }();
  // Rescale of O still owed for the last max move (applied just before the
  // next P V product, see the step below).
  float alpha_owed = 1.0f;
  bool owed = false;

  const int nkv = kv1 - kv0;
  const int ntiles = (nkv + T::BC - 1) / T::BC;

  // Global byte offsets of this lane's 16-byte loads (constant over tiles):
  // load `it` of wave w fills LDS chunks (it*kWaves + w)*64 + lane of the tile.
  int koff[T::NLOAD], voff[T::NLOAD];
#pragma unroll
  for (int it = 0; it < T::NLOAD; ++it) {
    const int P = (it * kWaves + wave) * 64 + lane;
    const int R = P / T::KCH, pc = P % T::KCH;
    koff[it] = key_row(R) * (int)a.k_ss * 2 + (pc ^ T::kx(R)) * 16;
    voff[it] = R * (int)a.v_ss * 2 + (pc ^ T::vx(R)) * 16;
  }
  // LDS byte offsets of this lane's operand reads (constant over tiles).
  int kread[T::NK];
#pragma unroll
  for (int k = 0; k < T::NK; ++k) kread[k] = li * T::RB + 16 * ((2 * k + lh) ^ T::kx(li));
  int vread[T::ND];
  {
    const int g = lane >> 4, i = lane & 15;
    const int key = 8 * (g >> 1) + (i >> 2);          // + jb*32 + hf*16 + 4u
    const int x = 2 * (g & 1) + ((i & 3) >> 1);       // chunk within the 64-byte d block
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
      vread[db] = key * T::RB + 16 * ((4 * db + x) ^ T::vx(i >> 2)) + 8 * (i & 1);
  }

  auto dma = [&](char* dst, const u16* src, int64_t stride, int t, const int (&off)[T::NLOAD]) {
    const __amdgpu_buffer_rsrc_t r = rows_rsrc<D>(src, (int64_t)t * T::BC, stride, nkv - t * T::BC, T::BC);
#pragma unroll
    for (int it = 0; it < T::NLOAD; ++it)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + (it * kWaves + wave) * 1024), 16,
                                               off[it], 0, 0, 0);
  };
  // S^T = K Q^T for the NJ 32-key blocks of the tile in kb
  auto qk = [&](const char* kb, f32x16 (&s)[T::NJ]) {
#pragma unroll
    for (int jb = 0; jb < T::NJ; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[jb][r] = 0.0f;
#pragma unroll
    for (int k = 0; k < T::NK; ++k)
#pragma unroll
      for (int jb = 0; jb < T::NJ; ++jb) {
        const bf16x8 kf = as_bf16x8(lds_read16(kb, jb * 32 * T::RB + kread[k]));
        s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[k], s[jb], 0, 0, 0);
      }
  };
  // P V for one 32-key block jb of the tile in vb (P^T of that block in pf)
  auto pv_blk = [&](const char* vb, int jb, const bf16x8 (&pf)[2]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < T::ND; ++db) {
        const int kb0 = (jb * 32 + hf * 16) * T::RB;
        const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(vb, kb0 + vread[db]));
        const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(vb, kb0 + 4 * T::RB + vread[db]));
        const bf16x8 va = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[hf], oacc[db], 0, 0, 0);
        if (db == T::ND - 1)
          lbacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_pat, pf[hf], lbacc, 0, 0, 0);
      }
  };
  // P = 2^(s*scale*log2e - m) for one 32-key block, rounded to bf16; lt
  // sums the fp32 P (this half-lane's share)
  auto exps_blk = [&](const f32x16& sblk, float mref, float& lt, bf16x8 (&pb)[2]) {
    lt = 0.0f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sblk[hf * 8 + 2 * t2], a.scale_log2, -mref));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sblk[hf * 8 + 2 * t2 + 1], a.scale_log2, -mref));
        lt += p0;
        lt += p1;
        const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
        pb[hf][2 * t2] = pp[0];
        pb[hf][2 * t2 + 1] = pp[1];
      }
  };
  auto blk_max = [&](const f32x16& sblk) {
    float mx = sblk[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sblk[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    return mx * a.scale_log2;
  };
  auto rescale_o = [&](float alpha) {
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    lbacc *= alpha;
  };
  // rare path: a block's running sum passed the cap; move m past the block's
  // max and past log2 of the row's sum so far (every P relative to the new m
  // is at most 1) and return the factor the earlier sums scale by
  auto move_max = [&](const f32x16& sblk) {
    const float lrow = l + __shfl_xor(l, 32);
    const float mn = fmaxf(fmaxf(m, blk_max(sblk)), m + __builtin_amdgcn_logf(lrow));
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
    m = mn;
    return alpha;
  };

  // Carried between steps: S^T of the previous tile's second 32-key block
  // (its exponentials run beside this step's QK^T) and P of the previous
  // tile's first block (computed beside the previous step's P V).
  f32x16 sb1;
  bf16x8 p0_prev[2];

  // One tile t: start the loads of K (tile t+1) and V (tile t); S^T of tile
  // t beside the exponentials of tile t-1's second block; then P V of tile
  // t-1 beside the exponentials of tile t's first block.  Each matrix phase
  // has vector work of its own wave to interleave with.
  auto step = [&](const char* kb_t, char* kb_n, char* vb_t, const char* vb_p, int t,
                  auto first_tag, auto last_tag) {
    constexpr bool kFirst = decltype(first_tag)::value;
    constexpr int kLast = decltype(last_tag)::value;
    __syncthreads();            // tile t's K and tile t-1's V are in; kb_n, vb_t are free
    dma(kb_n, kg, a.k_ss, t + 1, koff);
    dma(vb_t, vg, a.v_ss, t, voff);
    if constexpr (!kFirst) {
      if (owed) rescale_o(alpha_owed);   // a move in the previous step's second phase
    }
    f32x16 sc[T::NJ];
    qk(kb_t, sc);
    // keys past the end of the range (in the last tile) do not exist
    auto mask = [&]() {
      const int valid = nkv - t * T::BC;
#pragma unroll
      for (int jb = 0; jb < T::NJ; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = jb * 32 + 16 * (r >> 3) + 8 * lh + (r & 7);
          if (key >= valid) sc[jb][r] = -__builtin_inff();
        }
    };
    // the mask applies before the scores are used: at once in the first
    // step (the tile max), else after the first phase (whose exponentials
    // are the previous tile's), so its branch does not split that phase
    auto apply_mask = [&]() {
      if constexpr (kLast == 1) {
        mask();
      } else if constexpr (kLast == 2) {
        if (t == ntiles - 1) mask();   // uniform: the whole workgroup agrees
      }
    };
    if constexpr (kFirst) apply_mask();
    if constexpr (kFirst) {
      // O and l are empty: m starts at the tile's own max (both blocks)
      float mx = sc[0][0];
#pragma unroll
      for (int jb = 0; jb < T::NJ; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[jb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m = mx * a.scale_log2;
      float lt0;
      exps_blk(sc[0], m, lt0, p0_prev);
      l = lt0;
      owed = false;
    } else {
      // tile t-1's second block, beside this tile's QK^T
      bf16x8 p1[2];
      float lt1;
      exps_blk(sb1, m, lt1, p1);
      if constexpr (D == 64) {
        // at D = 64 the vector work outweighs the matrix work: spread it
        // evenly, one MFMA to four vector instructions (measured 0.7-1.6%
        // faster on the video forward; at D = 128 the default schedule wins)
#pragma unroll
        for (int i = 0; i < T::NK * T::NJ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
        }
      }
      if (__ballot(l + lt1 > kSumCap) != 0ull) {
        const float alpha = move_max(sb1);
        exps_blk(sb1, m, lt1, p1);
        // O (tiles up to t-2) and tile t-1's first block were relative to
        // the old max (rare path)
        rescale_o(alpha);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float x0 = (float)p0_prev[hf][e] * alpha, x1 = (float)p0_prev[hf][e + 1] * alpha;
            const bf16x2 pp = {(__bf16)x0, (__bf16)x1};
            p0_prev[hf][e] = pp[0];
            p0_prev[hf][e + 1] = pp[1];
          }
      }
      l += lt1;
      apply_mask();
      // P V of tile t-1, beside this tile's first-block exponentials
      pv_blk(vb_p, 0, p0_prev);
      pv_blk(vb_p, 1, p1);
      bf16x8 p0n[2];
      float lt0;
      exps_blk(sc[0], m, lt0, p0n);
      if constexpr (D == 64) {
#pragma unroll
        for (int i = 0; i < T::NJ * 2 * (T::ND + 1); ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
        }
      }
      const bool move = __ballot(l + lt0 > kSumCap) != 0ull;
      if (move) {
        asm volatile("" ::: "memory");
        alpha_owed = move_max(sc[0]);
        exps_blk(sc[0], m, lt0, p0n);
      }
      owed = move;   // O now holds tile t-1 relative to the max before this move
      l += lt0;
      p0_prev[0] = p0n[0];
      p0_prev[1] = p0n[1];
    }
    sb1 = sc[1];
    // this wave's loads must land before the next barrier publishes them
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
  };

  // after the last step: tile T-1's second block and its P V (V in vb)
  auto finish = [&](const char* vb) {
    __syncthreads();
    if (owed) rescale_o(alpha_owed);
    bf16x8 p1[2];
    float lt1;
    exps_blk(sb1, m, lt1, p1);
    if (__ballot(l + lt1 > kSumCap) != 0ull) {
      const float alpha = move_max(sb1);
      exps_blk(sb1, m, lt1, p1);
      rescale_o(alpha);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float x0 = (float)p0_prev[hf][e] * alpha, x1 = (float)p0_prev[hf][e + 1] * alpha;
          const bf16x2 pp = {(__bf16)x0, (__bf16)x1};
          p0_prev[hf][e] = pp[0];
          p0_prev[hf][e + 1] = pp[1];
        }
    }
    l += lt1;
    pv_blk(vb, 0, p0_prev);
    pv_blk(vb, 1, p1);
  };

  if (ntiles > 0) {
    dma(kbuf0, kg, a.k_ss, 0, koff);
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
    // Tiles come in (odd, even) pairs after tile 0; buffers alternate by
    // parity.  The last tile masks its keys past the end: an even last tile
    // is the second step of a pair (a uniform branch there), an odd one the
    // step after the loop.  Few step instances keep the code, and the
    // registers the compiler assigns across them, small.
    step(kbuf0, kbuf1, vbuf0, vbuf1, 0, First{}, MaybeLast{});
    int t = 1;
    for (; t + 1 < ntiles; t += 2) {
      step(kbuf1, kbuf0, vbuf1, vbuf0, t, NotFirst{}, NotLast{});
      step(kbuf0, kbuf1, vbuf0, vbuf1, t + 1, NotFirst{}, MaybeLast{});
    }
    if (t < ntiles) {             // t odd and last
      step(kbuf1, kbuf0, vbuf1, vbuf0, t, NotFirst{}, Last{});
      finish(vbuf1);
    } else {                      // the last tile was even
      finish(vbuf0);
    }
  }

  // epilogue: O = O_acc / lb, LSE = (m + log2 l) ln 2; no keys -> O = 0, -inf
  const float lt = l + __shfl_xor(l, 32);
  const float lbt = lbacc[0];   // the whole row's sum (both halves)
  const float inv = lbt > 0.0f ? 1.0f / lbt : 0.0f;
  const float lse = lt > 0.0f ? (m + log2f(lt)) * kLn2 : -__builtin_inff();
  if (row < a.Sq && lh == 0 && a.lse != nullptr)
    a.lse[split * a.l_split_stride + b * a.l_sb + h * a.l_sh + row] = lse;

  // O goes out through LDS when its tiles fit in the (now free) K/V buffers:
  // bf16 O always (32 x 2D bytes per wave), fp32 O in workgroups of at most
  // 4 waves (32 x 4D bytes per wave).  In registers a lane holds 4-element
  // pieces of its row, so direct stores write every row 16 bytes at a time
  // from 32 rows at once, lines that the L2 has to merge.  Each wave instead
  // writes its tile row-major to LDS (16-byte chunks XOR-swizzled by row, so
  // neither direction conflicts on banks) and reads it back 16 bytes per
  // lane, so that consecutive lanes store whole rows: FLUX-1024's forward ran
  // 2-3% faster, with the same values.  bf16 O (a final output) is stored
  // non-temporally; fp32 O (ring partials, read by the fold right after)
  // stays in the cache.
  constexpr bool kStage = !OF32 || W <= 4;
  if constexpr (kStage) {
    constexpr int OB = OF32 ? 4 : 2;             // bytes per element of O
    constexpr int RBO = D * OB;                  // bytes per row of O
    constexpr int NCH = RBO / 16;                // 16-byte chunks per row
    constexpr int ROWS_PER = 64 / NCH;           // rows one wave instruction covers
    static_assert(32 * RBO * W <= 4 * T::TILE_BYTES, "the tiles must fit the K/V buffers");
    __syncthreads();                             // every wave is done with K and V
    // wave w's 32 * RBO bytes: bf16 tiles two to a buffer, fp32 tiles one
    const int slot = OF32 ? wave : wave >> 1;
    char* st = slot == 0 ? kbuf0 : slot == 1 ? kbuf1 : slot == 2 ? vbuf0 : vbuf1;
    if constexpr (!OF32) st += (wave & 1) * (32 * RBO);
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // elements db*32 + 8g + 4lh .. +3 of row li: chunk c, byte offset cb
        if constexpr (OF32) {
          const f32x4 x = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                           oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
          const int c = db * 8 + 2 * g + lh;
          *reinterpret_cast<f32x4*>(st + li * RBO + (c ^ (li & (NCH - 1))) * 16) = x;
        } else {
          const bf16x4 x = {(__bf16)(oacc[db][4 * g] * inv), (__bf16)(oacc[db][4 * g + 1] * inv),
                            (__bf16)(oacc[db][4 * g + 2] * inv), (__bf16)(oacc[db][4 * g + 3] * inv)};
          const int c = db * 4 + g;
          *reinterpret_cast<bf16x4*>(st + li * RBO + (c ^ (li & (NCH - 1))) * 16 + lh * 8) = x;
        }
      }
    const int64_t obase0 = split * a.o_split_stride + b * a.o_sb + h * a.o_sh;
#pragma unroll
    for (int i = 0; i < 32 / ROWS_PER; ++i) {
      const int r = i * ROWS_PER + lane / NCH, c = lane % NCH;
      const u32x4 y = *reinterpret_cast<const u32x4*>(st + r * RBO + (c ^ (r & (NCH - 1))) * 16);
      const int orow = qt * T::BM + wave * 32 + r;
      if (orow < a.Sq) {
        char* dst = static_cast<char*>(a.o) + (obase0 + (int64_t)orow * a.o_ss) * OB + c * 16;
        if constexpr (OF32)
          *reinterpret_cast<u32x4*>(dst) = y;
        else
          __builtin_nontemporal_store(y, reinterpret_cast<u32x4*>(dst));
      }
    }
  } else if (row < a.Sq) {
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
  }
#endif
}

template <int D, bool OF32, int W>
hipError_t launch_w(const AttnArgs& a, hipStream_t stream) {
  using T = Tile<D, W>;
  const int nqt = (a.Sq + T::BM - 1) / T::BM;
  const long total = (long)a.n_split * a.B * a.H * nqt;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, OF32, W>), dim3((unsigned)total),
                     dim3(T::kThreads), 0, stream, a);
  return hipGetLastError();
}

int cu_count() {
  static int n = 0;   // the same for every MI355X; read once
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

template <int D, bool OF32>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  switch (attn_pick_waves((long)a.n_split * a.B * a.H, a.Sq, cu_count())) {
    case 8: return launch_w<D, OF32, 8>(a, stream);
    case 4: return launch_w<D, OF32, 4>(a, stream);
    default: return launch_w<D, OF32, 2>(a, stream);
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.o_f32 ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  if (a.D == 64) return a.o_f32 ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cru
