// Internal launch interface between the host API (cru_api.cpp) and the HIP
// kernels.  Arguments here are already validated; launchers only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cru.h"
#include "fastdiv.h"

namespace cru {

// One attention launch: query rows [0, Sq) against key rows of `n_split`
// consecutive key ranges [split_start[c], split_start[c+1]).  Split c writes
// its (O, LSE) to o + c*o_split_stride and lse + c*l_split_stride.  With one
// split this is a plain forward over keys [split_start[0], split_start[1]).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;                 // may be null
  int64_t q_sb, q_ss, q_sh;   // element strides
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t l_sb, l_sh;
  int64_t o_split_stride;     // elements of o between splits
  int64_t l_split_stride;     // elements of lse between splits
  int B, H, Sq, D;
  int o_f32;                  // 1: o is fp32, 0: o is bf16
  int n_split;
  float scale_log2;           // softmax scale times log2(e)
  int split_start[CRU_MAX_PARTS + 1];
};

// Every part shares one set of strides (checked on the host).
struct MergeArgs {
  const void* o_part[CRU_MAX_PARTS];   // fp32, or bf16 when p_bf16
  const float* l_part[CRU_MAX_PARTS];
  int64_t p_sb, p_ss, p_sh;
  int64_t pl_sb, pl_sh;
  void* o;
  float* lse;                 // may be null
  int64_t o_sb, o_ss, o_sh;
  int64_t l_sb, l_sh;
  int B, S, H, D;
  int n;
  int o_f32;
  int p_bf16;                 // partial outputs in bf16 (convert_to_fp32 off)
  FastDiv div_s, div_h;       // set by launch_merge
};

// Ulysses regrouping of up to 8 tensors of one shape and dtype.
//   dir = 0: seq2head, strided x -> contiguous y [P, B, S, H/P, D]
//   dir = 1: head2seq, contiguous y -> strided x
struct LayoutArgs {
  const void* src[8];
  void* dst[8];
  int64_t sb, ss, sh;         // strides of the [B, S, H, D] side
  int B, S, H, D, P;
  int n;
  int elem_bytes;             // 2 or 4
  int dir;
  // set by launch_layout: head groups of q = H / P heads, the first rem of
  // them one more (uneven when rem != 0)
  int quo, rem, uneven;
  FastDiv div_h, div_s, div_hp, div_b, div_q, div_q1;
};

// Host side shared by the C entry points.  ScratchFn hands back the current
// device's static scratch array (ring_noalloc.hip); with it,
// ring_emulate_ws takes workspace_bytes as that array's size and skips the
// workspace pointer checks.  report() sets the thread's error message.
typedef cru_status (*ScratchFn)(void** ptr);
cru_status ring_emulate_ws(const cru_tensor* q_share, const cru_tensor* k, const cru_tensor* v,
                           int n_chunks, int anything, const int64_t* chunk_sizes, int fused,
                           int convert_to_fp32, const cru_tensor* o, const cru_lse* lse,
                           float scale, void* workspace, size_t workspace_bytes,
                           ScratchFn scratch, hipStream_t stream);
cru_status report(cru_status st, const char* fmt, ...);
void clear_error();

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream);

}  // namespace cru
