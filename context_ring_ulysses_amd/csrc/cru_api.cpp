// Host side of the C ABI declared in include/cru.h: argument checks, launch
// set-up and the ring-share orchestration.  Nothing here computes attention;
// every step of the path runs in the HIP kernels.
//
// The checks mirror the three classes of the diffusers "Attention backends"
// page, "Checks" section (device, data type, shape) and the divisibility
// rules of the diffusers "Context parallelism" guide's variant table (ring:
// sequence length divisible by the ring degree unless "Ring Anything";
// Ulysses: sequence length and head count divisible by the Ulysses degree).
// They all run before anything is enqueued, so a failed call has no effect
// on the device.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "cru.h"
#include "cru_kernels.h"

namespace {

thread_local char g_err[512] = "";

cru_status fail(cru_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

#define CRU_TRY(expr)                 \
  do {                                \
    cru_status st_ = (expr);          \
    if (st_ != CRU_OK) return st_;    \
  } while (0)

constexpr int64_t kMaxDim = (int64_t)1 << 30;
// Largest tensor a descriptor may describe, in elements.  Every product of
// sizes formed later (grid sizes, element counts) is bounded by a small
// multiple of this, so none of them can overflow int64_t.
constexpr int64_t kMaxElems = (int64_t)1 << 48;

// Largest element offset a view may reach (the sum of (size - 1) * stride
// over its dims).  The kernels form element and byte offsets in int64_t, so
// bounding the span keeps every offset they form far from overflow.
constexpr int64_t kMaxSpan = (int64_t)1 << 60;

// a * b for non-negative a, b, saturating at INT64_MAX instead of overflowing
int64_t mul_sat(int64_t a, int64_t b) {
  if (a == 0 || b == 0) return 0;
  return a > INT64_MAX / b ? INT64_MAX : a * b;
}

// a + b for non-negative a, b, saturating at INT64_MAX
int64_t add_sat(int64_t a, int64_t b) { return a > INT64_MAX - b ? INT64_MAX : a + b; }

// largest element offset of a view whose sizes are all >= 1
int64_t view_span(int n, const int64_t* size, const int64_t* stride) {
  int64_t span = 0;
  for (int i = 0; i < n; ++i) span = add_sat(span, mul_sat(size[i] - 1, stride[i]));
  return span;
}

int elem_bytes(int dtype) { return dtype == CRU_BF16 ? 2 : 4; }
const char* dtype_name(int dtype) { return dtype == CRU_BF16 ? "bf16" : "fp32"; }

cru_status check_tensor(const cru_tensor* t, const char* name) {
  if (t == nullptr) return fail(CRU_EINVAL, "%s: descriptor is NULL", name);
  if (t->dtype != CRU_F32 && t->dtype != CRU_BF16)
    return fail(CRU_EUNSUPPORTED, "%s: unknown dtype code %d", name, t->dtype);
  if (t->reserved != 0) return fail(CRU_EINVAL, "%s: reserved field must be 0", name);
  if (t->B < 0 || t->S < 0 || t->H < 0 || t->D < 0)
    return fail(CRU_EINVAL, "%s: negative size", name);
  if (t->B > kMaxDim || t->S > kMaxDim || t->H > kMaxDim || t->D > kMaxDim)
    return fail(CRU_EINVAL, "%s: size above 2^30", name);
  if (t->sb < 0 || t->ss < 0 || t->sh < 0) return fail(CRU_EINVAL, "%s: negative stride", name);
  const int64_t numel = mul_sat(mul_sat(mul_sat(t->B, t->S), t->H), t->D);
  if (numel > kMaxElems)
    return fail(CRU_EINVAL, "%s: [%lld, %lld, %lld, %lld] is above 2^48 elements", name,
                (long long)t->B, (long long)t->S, (long long)t->H, (long long)t->D);
  if (numel > 0 && t->data == nullptr) return fail(CRU_EINVAL, "%s: data is NULL", name);
  if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
    return fail(CRU_EINVAL, "%s: data is not 16-byte aligned", name);
  const int64_t vec = 16 / elem_bytes(t->dtype);
  if (t->sb % vec || t->ss % vec || t->sh % vec)
    return fail(CRU_EINVAL, "%s: strides (%lld, %lld, %lld) are not multiples of %lld elements",
                name, (long long)t->sb, (long long)t->ss, (long long)t->sh, (long long)vec);
  if (numel > 0) {
    const int64_t size[4] = {t->B, t->S, t->H, t->D};
    const int64_t stride[4] = {t->sb, t->ss, t->sh, 1};
    if (view_span(4, size, stride) >= kMaxSpan)
      return fail(CRU_EINVAL, "%s: strides (%lld, %lld, %lld) reach past 2^60 elements", name,
                  (long long)t->sb, (long long)t->ss, (long long)t->sh);
  }
  return CRU_OK;
}

// True when the map from indices to element offsets is one to one: with the
// dims of size > 1 sorted by stride, every stride exceeds the largest offset
// the smaller-stride dims reach.  (Sufficient, and exact for the layouts
// strided views of one buffer produce.)
bool strides_injective(int n, const int64_t* size, const int64_t* stride) {
  int64_t sz[4], st[4];
  int m = 0;
  for (int i = 0; i < n; ++i)
    if (size[i] == 0) return true;   // no elements
  for (int i = 0; i < n; ++i)
    if (size[i] > 1) {
      sz[m] = size[i];
      st[m] = stride[i];
      ++m;
    }
  for (int i = 1; i < m; ++i)   // insertion sort by stride
    for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
      const int64_t a = st[j], b = sz[j];
      st[j] = st[j - 1]; sz[j] = sz[j - 1];
      st[j - 1] = a; sz[j - 1] = b;
    }
  int64_t reach = 0;   // largest offset of the dims taken so far
  for (int i = 0; i < m; ++i) {
    if (st[i] <= reach) return false;
    reach = add_sat(reach, mul_sat(sz[i] - 1, st[i]));
  }
  return true;
}

// An output view: each element must have its own address, or concurrent
// threads would race on one location (inputs may repeat elements, e.g. a
// stride-0 broadcast along the sequence).
cru_status check_output_tensor(const cru_tensor* t, const char* name) {
  CRU_TRY(check_tensor(t, name));
  const int64_t size[4] = {t->B, t->S, t->H, t->D};
  const int64_t stride[4] = {t->sb, t->ss, t->sh, 1};
  if (!strides_injective(4, size, stride))
    return fail(CRU_EINVAL, "%s: output strides (%lld, %lld, %lld, 1) make elements overlap", name,
                (long long)t->sb, (long long)t->ss, (long long)t->sh);
  return CRU_OK;
}

cru_status check_head_dim(const cru_tensor* t, const char* name) {
  if (t->D != 64 && t->D != 128)
    return fail(CRU_EUNSUPPORTED, "%s: head dim %lld (supported: 64, 128)", name, (long long)t->D);
  return CRU_OK;
}

cru_status check_lse(const cru_lse* l, const char* name, int64_t B, int64_t H, int64_t S) {
  if (l == nullptr) return fail(CRU_EINVAL, "%s: descriptor is NULL", name);
  if (l->B != B || l->H != H || l->S != S)
    return fail(CRU_EINVAL, "%s: shape [%lld, %lld, %lld], expected [%lld, %lld, %lld]", name,
                (long long)l->B, (long long)l->H, (long long)l->S, (long long)B, (long long)H,
                (long long)S);
  if (l->sb < 0 || l->sh < 0) return fail(CRU_EINVAL, "%s: negative stride", name);
  if (B * H * S > 0 && l->data == nullptr) return fail(CRU_EINVAL, "%s: data is NULL", name);
  if (reinterpret_cast<uintptr_t>(l->data) % 4 != 0)
    return fail(CRU_EINVAL, "%s: data is not 4-byte aligned", name);
  const int64_t size[3] = {B, H, S};
  const int64_t stride[3] = {l->sb, l->sh, 1};
  if (B * H * S > 0 && view_span(3, size, stride) >= kMaxSpan)
    return fail(CRU_EINVAL, "%s: strides (%lld, %lld, 1) reach past 2^60 elements", name,
                (long long)l->sb, (long long)l->sh);
  if (!strides_injective(3, size, stride))
    return fail(CRU_EINVAL, "%s: strides (%lld, %lld, 1) make elements overlap", name,
                (long long)l->sb, (long long)l->sh);
  return CRU_OK;
}

bool same_shape(const cru_tensor* a, const cru_tensor* b) {
  return a->B == b->B && a->S == b->S && a->H == b->H && a->D == b->D;
}

cru_status check_device(const void* p, const char* name) {
  if (p == nullptr) return CRU_OK;   // only empty tensors get here with NULL
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(CRU_EDEVICE, "%s: no current HIP device", name);
  }
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(CRU_EDEVICE, "%s: pointer is not HIP device memory", name);
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(CRU_EDEVICE, "%s: pointer is not device memory (memory type %d)", name,
                (int)attr.type);
  if (attr.device != dev)
    return fail(CRU_EDEVICE, "%s: pointer is on device %d, current device is %d", name,
                attr.device, dev);
  return CRU_OK;
}

cru_status check_scale(float scale, int64_t D, float* scale_log2) {
  if (!(scale >= 0.0f) || std::isinf(scale))
    return fail(CRU_EINVAL, "scale must be finite and >= 0 (0 selects 1/sqrt(D)), got %g",
                (double)scale);
  const double sc = scale == 0.0f ? 1.0 / std::sqrt((double)D) : (double)scale;
  *scale_log2 = (float)(sc * 1.4426950408889634);   // log2(e)
  return CRU_OK;
}

cru_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CRU_EHIP, "%s: %s", what, hipGetErrorString(e));
  return CRU_OK;
}

void fill_attn_views(cru::AttnArgs& a, const cru_tensor* q, const cru_tensor* k,
                     const cru_tensor* v) {
  a.q = q->data;
  a.k = k->data;
  a.v = v->data;
  a.q_sb = q->sb; a.q_ss = q->ss; a.q_sh = q->sh;
  a.k_sb = k->sb; a.k_ss = k->ss; a.k_sh = k->sh;
  a.v_sb = v->sb; a.v_ss = v->ss; a.v_sh = v->sh;
  a.B = (int)q->B;
  a.H = (int)q->H;
  a.Sq = (int)q->S;
  a.D = (int)q->D;
}

// The bf16 kernel addresses one tile of q (at most 256 rows of 2-byte
// elements) or of k, v (64 rows) through a buffer descriptor with a 32-bit
// byte range: 256 * ss * 2 must stay below 2^31.
cru_status check_row_strides(const cru_tensor* q, const cru_tensor* k, const cru_tensor* v) {
  const int64_t lim = ((int64_t)1 << 31) / (128 * 4);
  if (q->ss >= lim || k->ss >= lim || v->ss >= lim)
    return fail(CRU_EINVAL, "sequence stride above %lld elements", (long long)lim);
  return CRU_OK;
}

// Checks shared by the attention entry points: q, k, v, o views, dtypes, shapes.
cru_status check_qkvo(const cru_tensor* q, const cru_tensor* k, const cru_tensor* v,
                      const cru_tensor* o) {
  CRU_TRY(check_tensor(q, "q"));
  CRU_TRY(check_tensor(k, "k"));
  CRU_TRY(check_tensor(v, "v"));
  CRU_TRY(check_output_tensor(o, "o"));
  if (k->dtype != q->dtype || v->dtype != q->dtype)
    return fail(CRU_EUNSUPPORTED, "q, k, v dtypes differ (%s, %s, %s)", dtype_name(q->dtype),
                dtype_name(k->dtype), dtype_name(v->dtype));
  if (q->dtype == CRU_F32 && o->dtype != CRU_F32)
    return fail(CRU_EUNSUPPORTED, "fp32 inputs need an fp32 output");
  if (k->B != q->B || k->H != q->H || k->D != q->D)
    return fail(CRU_EINVAL, "k [%lld, %lld, %lld, %lld] does not match q [%lld, _, %lld, %lld]",
                (long long)k->B, (long long)k->S, (long long)k->H, (long long)k->D,
                (long long)q->B, (long long)q->H, (long long)q->D);
  if (!same_shape(v, k)) return fail(CRU_EINVAL, "v shape differs from k");
  if (!same_shape(o, q)) return fail(CRU_EINVAL, "o shape differs from q");
  CRU_TRY(check_head_dim(q, "q"));
  CRU_TRY(check_row_strides(q, k, v));
  return CRU_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The kernels index threads, rows and 16-byte vectors with 32-bit integers.
constexpr int64_t kMaxIndex = ((int64_t)1 << 31) - 4096;

cru_status check_index_range(int64_t count, const char* what) {
  if (count > kMaxIndex)
    return fail(CRU_EINVAL, "%s: %lld work items exceed one call's 2^31 limit; split the call",
                what, (long long)count);
  return CRU_OK;
}

// Threads of the attention kernels: (splits x B x H x query tiles), two
// threads per query row of a tile (32 rows per wave of 64 lanes); the tile
// height is at most 256 rows.
cru_status check_attn_grid(int64_t n_split, const cru_tensor* q) {
  return check_index_range(n_split * q->B * q->H * ((q->S + 255) / 256) * 512, "attention");
}

// Threads of the merge kernel: one per 4 elements of every row.
cru_status check_merge_grid(const cru_tensor* t) {
  return check_index_range(t->B * t->S * t->H * (t->D / 4), "merge");
}

}  // namespace

extern "C" {

const char* cru_status_str(int status) {
  switch (status) {
    case CRU_OK: return "CRU_OK";
    case CRU_EINVAL: return "CRU_EINVAL";
    case CRU_ENOTDIV: return "CRU_ENOTDIV";
    case CRU_EUNSUPPORTED: return "CRU_EUNSUPPORTED";
    case CRU_EDEVICE: return "CRU_EDEVICE";
    case CRU_EWORKSPACE: return "CRU_EWORKSPACE";
    case CRU_EHIP: return "CRU_EHIP";
    default: return "CRU_UNKNOWN";
  }
}

const char* cru_last_error(void) { return g_err; }

int cru_abi_version(void) { return CRU_ABI_VERSION; }

cru_status cru_attn_fwd_lse(const cru_tensor* q, const cru_tensor* k, const cru_tensor* v,
                            const cru_tensor* o, const cru_lse* lse, float scale,
                            hipStream_t stream) {
  g_err[0] = '\0';
  CRU_TRY(check_qkvo(q, k, v, o));
  if (lse != nullptr) CRU_TRY(check_lse(lse, "lse", q->B, q->H, q->S));
  float scale_log2 = 0.0f;
  CRU_TRY(check_scale(scale, q->D, &scale_log2));
  CRU_TRY(check_attn_grid(1, q));
  const int64_t nq = q->B * q->H * q->S;
  if (nq == 0) return CRU_OK;
  CRU_TRY(check_device(q->data, "q"));
  CRU_TRY(check_device(k->data, "k"));
  CRU_TRY(check_device(v->data, "v"));
  CRU_TRY(check_device(o->data, "o"));
  if (lse != nullptr) CRU_TRY(check_device(lse->data, "lse"));

  cru::AttnArgs a = {};
  fill_attn_views(a, q, k, v);
  a.o = o->data;
  a.o_sb = o->sb; a.o_ss = o->ss; a.o_sh = o->sh;
  a.o_f32 = o->dtype == CRU_F32;
  a.lse = lse ? lse->data : nullptr;
  a.l_sb = lse ? lse->sb : 0;
  a.l_sh = lse ? lse->sh : 0;
  a.n_split = 1;
  a.split_start[0] = 0;
  a.split_start[1] = (int)k->S;
  a.scale_log2 = scale_log2;
  const hipError_t e = q->dtype == CRU_BF16 ? cru::launch_attn_bf16(a, stream)
                                            : cru::launch_attn_f32(a, stream);
  return hip_status(e, "attention launch");
}

cru_status cru_attn_merge_lse(int n, const cru_tensor* o_parts, const cru_lse* lse_parts,
                              const cru_tensor* o, const cru_lse* lse, hipStream_t stream) {
  g_err[0] = '\0';
  if (n < 1 || n > CRU_MAX_PARTS)
    return fail(CRU_EINVAL, "n = %d parts, must be in [1, %d]", n, CRU_MAX_PARTS);
  if (o_parts == nullptr || lse_parts == nullptr)
    return fail(CRU_EINVAL, "o_parts / lse_parts is NULL");
  const cru_tensor* p0 = &o_parts[0];
  for (int c = 0; c < n; ++c) {
    const cru_tensor* p = &o_parts[c];
    CRU_TRY(check_tensor(p, "o_parts[c]"));
    if (p->dtype != p0->dtype)
      return fail(CRU_EUNSUPPORTED, "o_parts[%d] is %s, o_parts[0] %s; parts share one dtype", c,
                  dtype_name(p->dtype), dtype_name(p0->dtype));
    if (!same_shape(p, p0)) return fail(CRU_EINVAL, "o_parts[%d] shape differs from o_parts[0]", c);
    if (p->sb != p0->sb || p->ss != p0->ss || p->sh != p0->sh)
      return fail(CRU_EINVAL, "o_parts[%d] strides differ from o_parts[0]", c);
    CRU_TRY(check_lse(&lse_parts[c], "lse_parts[c]", p0->B, p0->H, p0->S));
    if (lse_parts[c].sb != lse_parts[0].sb || lse_parts[c].sh != lse_parts[0].sh)
      return fail(CRU_EINVAL, "lse_parts[%d] strides differ from lse_parts[0]", c);
  }
  CRU_TRY(check_head_dim(p0, "o_parts[0]"));
  CRU_TRY(check_output_tensor(o, "o"));
  if (!same_shape(o, p0)) return fail(CRU_EINVAL, "o shape differs from the parts");
  if (lse != nullptr) CRU_TRY(check_lse(lse, "lse", p0->B, p0->H, p0->S));
  CRU_TRY(check_merge_grid(p0));
  if (p0->B * p0->H * p0->S == 0) return CRU_OK;
  for (int c = 0; c < n; ++c) {
    CRU_TRY(check_device(o_parts[c].data, "o_parts[c]"));
    CRU_TRY(check_device(lse_parts[c].data, "lse_parts[c]"));
  }
  CRU_TRY(check_device(o->data, "o"));
  if (lse != nullptr) CRU_TRY(check_device(lse->data, "lse"));

  cru::MergeArgs a = {};
  for (int c = 0; c < n; ++c) {
    a.o_part[c] = o_parts[c].data;
    a.l_part[c] = lse_parts[c].data;
  }
  a.p_bf16 = p0->dtype == CRU_BF16;
  a.p_sb = p0->sb; a.p_ss = p0->ss; a.p_sh = p0->sh;
  a.pl_sb = lse_parts[0].sb; a.pl_sh = lse_parts[0].sh;
  a.o = o->data;
  a.o_sb = o->sb; a.o_ss = o->ss; a.o_sh = o->sh;
  a.lse = lse ? lse->data : nullptr;
  a.l_sb = lse ? lse->sb : 0;
  a.l_sh = lse ? lse->sh : 0;
  a.B = (int)p0->B; a.S = (int)p0->S; a.H = (int)p0->H; a.D = (int)p0->D;
  a.n = n;
  a.o_f32 = o->dtype == CRU_F32;
  return hip_status(cru::launch_merge(a, stream), "merge launch");
}

cru_status cru_ring_workspace_bytes(const cru_tensor* q_share, int n_chunks, size_t* bytes) {
  g_err[0] = '\0';
  if (bytes == nullptr) return fail(CRU_EINVAL, "bytes is NULL");
  CRU_TRY(check_tensor(q_share, "q_share"));
  if (n_chunks < 1 || n_chunks > CRU_MAX_PARTS)
    return fail(CRU_EINVAL, "n_chunks = %d, must be in [1, %d]", n_chunks, CRU_MAX_PARTS);
  const size_t rows = (size_t)q_share->B * q_share->S * q_share->H;
  *bytes = (size_t)n_chunks * (align256(rows * q_share->D * 4) + align256(rows * 4));
  return CRU_OK;
}

cru_status cru_ring_chunk_bounds(int64_t S, int n, int anything, int64_t* starts) {
  g_err[0] = '\0';
  if (starts == nullptr) return fail(CRU_EINVAL, "starts is NULL");
  if (n < 1 || n > CRU_MAX_PARTS)
    return fail(CRU_EINVAL, "n = %d chunks, must be in [1, %d]", n, CRU_MAX_PARTS);
  if (S < 0 || S > kMaxDim) return fail(CRU_EINVAL, "sequence length %lld out of range", (long long)S);
  if (anything != 0 && anything != 1) return fail(CRU_EINVAL, "anything must be 0 or 1");
  if (!anything && S % n != 0)
    return fail(CRU_ENOTDIV,
                "sequence length %lld is not divisible by ring degree %d "
                "(set anything = 1 for Ring Anything)",
                (long long)S, n);
  const int64_t base = S / n, extra = S % n;
  starts[0] = 0;
  for (int c = 0; c < n; ++c) starts[c + 1] = starts[c] + base + (c < extra ? 1 : 0);
  return CRU_OK;
}

cru_status cru_ring_emulate(const cru_tensor* q_share, const cru_tensor* k, const cru_tensor* v,
                            int n_chunks, int anything, const int64_t* chunk_sizes, int fused,
                            int convert_to_fp32, const cru_tensor* o, const cru_lse* lse,
                            float scale, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  g_err[0] = '\0';
  return cru::ring_emulate_ws(q_share, k, v, n_chunks, anything, chunk_sizes, fused,
                              convert_to_fp32, o, lse, scale, workspace, workspace_bytes, nullptr,
                              stream);
}

}  // extern "C"

namespace cru {

cru_status report(cru_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = '\0'; }

cru_status ring_emulate_ws(const cru_tensor* q_share, const cru_tensor* k, const cru_tensor* v,
                           int n_chunks, int anything, const int64_t* chunk_sizes, int fused,
                           int convert_to_fp32, const cru_tensor* o, const cru_lse* lse,
                           float scale, void* workspace, size_t workspace_bytes,
                           ScratchFn scratch, hipStream_t stream) {
  CRU_TRY(check_qkvo(q_share, k, v, o));
  if (lse != nullptr) CRU_TRY(check_lse(lse, "lse", q_share->B, q_share->H, q_share->S));
  if (n_chunks < 1 || n_chunks > CRU_MAX_PARTS)
    return fail(CRU_EINVAL, "n_chunks = %d, must be in [1, %d]", n_chunks, CRU_MAX_PARTS);
  if (anything != 0 && anything != 1) return fail(CRU_EINVAL, "anything must be 0 or 1");
  if (fused != 0 && fused != 1) return fail(CRU_EINVAL, "fused must be 0 or 1");
  if (convert_to_fp32 != 0 && convert_to_fp32 != 1)
    return fail(CRU_EINVAL, "convert_to_fp32 must be 0 or 1");
  if (!convert_to_fp32 && q_share->dtype != CRU_BF16)
    return fail(CRU_EUNSUPPORTED, "partials in the model dtype need bf16 inputs");
  float scale_log2 = 0.0f;
  CRU_TRY(check_scale(scale, q_share->D, &scale_log2));
  CRU_TRY(check_attn_grid(n_chunks, q_share));
  CRU_TRY(check_merge_grid(q_share));

  const int64_t Skv = k->S;
  int64_t start[CRU_MAX_PARTS + 1];
  start[0] = 0;
  if (chunk_sizes == nullptr) {
    CRU_TRY(cru_ring_chunk_bounds(Skv, n_chunks, anything, start));
  } else {
    for (int c = 0; c < n_chunks; ++c) {
      if (chunk_sizes[c] < 0) return fail(CRU_EINVAL, "chunk_sizes[%d] < 0", c);
      // checked before the add, so the running sum stays in [0, Skv]
      if (chunk_sizes[c] > Skv - start[c])
        return fail(CRU_EINVAL, "chunk sizes pass the %lld K/V rows at chunk %d", (long long)Skv,
                    c);
      start[c + 1] = start[c] + chunk_sizes[c];
    }
    if (start[n_chunks] != Skv)
      return fail(CRU_EINVAL, "chunk sizes sum to %lld, K/V has %lld rows",
                  (long long)start[n_chunks], (long long)Skv);
    if (!anything)
      for (int c = 1; c < n_chunks; ++c)
        if (chunk_sizes[c] != chunk_sizes[0])
          return fail(CRU_ENOTDIV, "unequal chunks need anything = 1 (Ring Anything)");
  }

  size_t need = 0;
  CRU_TRY(cru_ring_workspace_bytes(q_share, n_chunks, &need));
  if (scratch != nullptr) {
    if (need > workspace_bytes)
      return fail(CRU_EWORKSPACE,
                  "the share needs %zu bytes of partials; the library's static scratch holds %zu",
                  need, workspace_bytes);
  } else {
    if (need > 0 && workspace == nullptr) return fail(CRU_EWORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(CRU_EWORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(CRU_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }

  const int64_t rows = q_share->B * q_share->H * q_share->S;
  if (rows == 0) return CRU_OK;
  CRU_TRY(check_device(q_share->data, "q_share"));
  CRU_TRY(check_device(k->data, "k"));
  CRU_TRY(check_device(v->data, "v"));
  CRU_TRY(check_device(o->data, "o"));
  if (lse != nullptr) CRU_TRY(check_device(lse->data, "lse"));
  if (scratch != nullptr)
    CRU_TRY(scratch(&workspace));   // the current device's static array
  else
    CRU_TRY(check_device(workspace, "workspace"));

  // Partials in the workspace: n [B, Sq, H, D] outputs (fp32, or bf16 without
  // convert_to_fp32), then n fp32 [B, H, Sq] LSEs.
  const int64_t B = q_share->B, Sq = q_share->S, H = q_share->H, D = q_share->D;
  const int pes = convert_to_fp32 ? 4 : 2;
  const size_t obytes = align256((size_t)rows * D * pes);
  const size_t lbytes = align256((size_t)rows * 4);
  char* ws = static_cast<char*>(workspace);
  float* o_base = reinterpret_cast<float*>(ws);
  float* l_base = reinterpret_cast<float*>(ws + n_chunks * obytes);

  cru::AttnArgs a = {};
  fill_attn_views(a, q_share, k, v);
  a.o_sb = Sq * H * D; a.o_ss = H * D; a.o_sh = D;
  a.l_sb = H * Sq; a.l_sh = Sq;
  a.o_f32 = convert_to_fp32;
  a.scale_log2 = scale_log2;
  auto launch = q_share->dtype == CRU_BF16 ? cru::launch_attn_bf16 : cru::launch_attn_f32;
  if (fused) {
    a.o = o_base;
    a.lse = l_base;
    a.o_split_stride = (int64_t)(obytes / pes);
    a.l_split_stride = (int64_t)(lbytes / 4);
    a.n_split = n_chunks;
    for (int c = 0; c <= n_chunks; ++c) a.split_start[c] = (int)start[c];
    CRU_TRY(hip_status(launch(a, stream), "fused ring attention launch"));
  } else {
    a.n_split = 1;
    for (int c = 0; c < n_chunks; ++c) {
      a.o = reinterpret_cast<char*>(o_base) + c * obytes;
      a.lse = reinterpret_cast<float*>(reinterpret_cast<char*>(l_base) + c * lbytes);
      a.split_start[0] = (int)start[c];
      a.split_start[1] = (int)start[c + 1];
      CRU_TRY(hip_status(launch(a, stream), "ring step attention launch"));
    }
  }

  cru::MergeArgs m = {};
  m.p_bf16 = !convert_to_fp32;
  for (int c = 0; c < n_chunks; ++c) {
    m.o_part[c] = ws + c * obytes;
    m.l_part[c] = reinterpret_cast<const float*>(reinterpret_cast<char*>(l_base) + c * lbytes);
  }
  m.p_sb = Sq * H * D; m.p_ss = H * D; m.p_sh = D;
  m.pl_sb = H * Sq; m.pl_sh = Sq;
  m.o = o->data;
  m.o_sb = o->sb; m.o_ss = o->ss; m.o_sh = o->sh;
  m.lse = lse ? lse->data : nullptr;
  m.l_sb = lse ? lse->sb : 0;
  m.l_sh = lse ? lse->sh : 0;
  m.B = (int)B; m.S = (int)Sq; m.H = (int)H; m.D = (int)D;
  m.n = n_chunks;
  m.o_f32 = o->dtype == CRU_F32;
  return hip_status(cru::launch_merge(m, stream), "ring merge launch");
}

}  // namespace cru

extern "C" {

static cru_status layout_common(int n, const cru_tensor* x, int P, int anything,
                                const char* what, cru::LayoutArgs* a) {
  if (n < 1 || n > 8) return fail(CRU_EINVAL, "%s: n = %d tensors, must be in [1, 8]", what, n);
  if (x == nullptr) return fail(CRU_EINVAL, "%s: x is NULL", what);
  for (int t = 0; t < n; ++t) {
    CRU_TRY(check_tensor(&x[t], "x[t]"));
    if (!same_shape(&x[t], &x[0]) || x[t].dtype != x[0].dtype)
      return fail(CRU_EINVAL, "%s: x[%d] shape or dtype differs from x[0]", what, t);
    if (x[t].sb != x[0].sb || x[t].ss != x[0].ss || x[t].sh != x[0].sh)
      return fail(CRU_EINVAL, "%s: x[%d] strides differ from x[0]", what, t);
  }
  CRU_TRY(check_head_dim(&x[0], "x[0]"));
  if (P < 1) return fail(CRU_EINVAL, "%s: P = %d must be >= 1", what, P);
  if (anything != 0 && anything != 1) return fail(CRU_EINVAL, "%s: anything must be 0 or 1", what);
  if (!anything && x[0].H % P != 0)
    return fail(CRU_ENOTDIV,
                "%s: head count %lld is not divisible by Ulysses degree %d "
                "(set anything = 1 for Ulysses Anything)",
                what, (long long)x[0].H, P);
  if (!anything && x[0].S % P != 0)
    return fail(CRU_ENOTDIV,
                "%s: sequence length %lld is not divisible by Ulysses degree %d "
                "(set anything = 1 for Ulysses Anything)",
                what, (long long)x[0].S, P);
  CRU_TRY(check_index_range(x[0].B * x[0].S * x[0].H * x[0].D * elem_bytes(x[0].dtype) / 16 + 512,
                            what));
  a->sb = x[0].sb; a->ss = x[0].ss; a->sh = x[0].sh;
  a->B = (int)x[0].B; a->S = (int)x[0].S; a->H = (int)x[0].H; a->D = (int)x[0].D;
  a->P = P;
  a->n = n;
  a->elem_bytes = elem_bytes(x[0].dtype);
  return CRU_OK;
}

cru_status cru_ulysses_head_bounds(int64_t H, int P, int anything, int64_t* starts) {
  g_err[0] = '\0';
  if (starts == nullptr) return fail(CRU_EINVAL, "starts is NULL");
  if (P < 1) return fail(CRU_EINVAL, "P = %d must be >= 1", P);
  if (H < 0 || H > kMaxDim) return fail(CRU_EINVAL, "head count %lld out of range", (long long)H);
  if (anything != 0 && anything != 1) return fail(CRU_EINVAL, "anything must be 0 or 1");
  if (!anything && H % P != 0)
    return fail(CRU_ENOTDIV,
                "head count %lld is not divisible by Ulysses degree %d "
                "(set anything = 1 for Ulysses Anything)",
                (long long)H, P);
  const int64_t base = H / P, extra = H % P;
  starts[0] = 0;
  for (int p = 0; p < P; ++p) starts[p + 1] = starts[p] + base + (p < extra ? 1 : 0);
  return CRU_OK;
}

cru_status cru_ulysses_seq2head(int n, const cru_tensor* x, void* const* y, int P, int anything,
                                hipStream_t stream) {
  g_err[0] = '\0';
  cru::LayoutArgs a = {};
  CRU_TRY(layout_common(n, x, P, anything, "seq2head", &a));
  if (y == nullptr) return fail(CRU_EINVAL, "seq2head: y is NULL");
  const bool empty = (int64_t)a.B * a.S * a.H * a.D == 0;
  for (int t = 0; t < n; ++t) {
    if (!empty && y[t] == nullptr) return fail(CRU_EINVAL, "seq2head: y[%d] is NULL", t);
    if (reinterpret_cast<uintptr_t>(y[t]) % 16 != 0)
      return fail(CRU_EINVAL, "seq2head: y[%d] is not 16-byte aligned", t);
  }
  if (empty) return CRU_OK;
  for (int t = 0; t < n; ++t) {
    CRU_TRY(check_device(x[t].data, "x[t]"));
    CRU_TRY(check_device(y[t], "y[t]"));
    a.src[t] = x[t].data;
    a.dst[t] = y[t];
  }
  a.dir = 0;
  return hip_status(cru::launch_layout(a, stream), "seq2head launch");
}

cru_status cru_ulysses_head2seq(int n, const void* const* y, const cru_tensor* x, int P,
                                int anything, hipStream_t stream) {
  g_err[0] = '\0';
  cru::LayoutArgs a = {};
  CRU_TRY(layout_common(n, x, P, anything, "head2seq", &a));
  if (y == nullptr) return fail(CRU_EINVAL, "head2seq: y is NULL");
  const bool empty = (int64_t)a.B * a.S * a.H * a.D == 0;
  for (int t = 0; t < n; ++t) {
    if (!empty && y[t] == nullptr) return fail(CRU_EINVAL, "head2seq: y[%d] is NULL", t);
    if (reinterpret_cast<uintptr_t>(y[t]) % 16 != 0)
      return fail(CRU_EINVAL, "head2seq: y[%d] is not 16-byte aligned", t);
  }
  for (int t = 0; t < n; ++t) CRU_TRY(check_output_tensor(&x[t], "x[t]"));
  if (empty) return CRU_OK;
  for (int t = 0; t < n; ++t) {
    CRU_TRY(check_device(y[t], "y[t]"));
    CRU_TRY(check_device(x[t].data, "x[t]"));
    a.src[t] = y[t];
    a.dst[t] = x[t].data;
  }
  a.dir = 1;
  return hip_status(cru::launch_layout(a, stream), "head2seq launch");
}

// Unified (USP) attention over a 2-D mesh of ulysses_degree x ring_degree
// devices, every device's share computed on this one:
//   1. seq2head of Q, K and V with P = ulysses_degree (the Ulysses
//      all-to-all's net effect);
//   2. per head group u, the ring over ring_degree sequence chunks: every
//      query row of the group against every chunk, fp32 partials folded in
//      ascending chunk order (rows of chunk r are ring rank r's share);
//   3. the reverse all-to-all: each group's folded output is stored straight
//      into its heads of o (head2seq fused into the fold's store).
// The workspace holds the three regrouped inputs and one ring workspace,
// reused by every group.
static size_t usp_parts(const cru_tensor* q, int Pu, int Pr, size_t* y_bytes,
                        size_t* ring_bytes) {
  const size_t elems = (size_t)q->B * q->S * q->H * q->D;
  const size_t rows_g = (size_t)q->B * q->S * (q->H / Pu);
  *y_bytes = align256(elems * elem_bytes(q->dtype));
  *ring_bytes = (size_t)Pr * (align256(rows_g * q->D * 4) + align256(rows_g * 4));
  return 3 * *y_bytes + *ring_bytes;
}

static cru_status usp_degrees(const cru_tensor* q, int Pu, int Pr) {
  if (Pu < 1) return fail(CRU_EINVAL, "ulysses_degree = %d must be >= 1", Pu);
  if (Pr < 1 || Pr > CRU_MAX_PARTS)
    return fail(CRU_EINVAL, "ring_degree = %d, must be in [1, %d]", Pr, CRU_MAX_PARTS);
  if (q->H % Pu != 0)
    return fail(CRU_ENOTDIV, "head count %lld is not divisible by ulysses_degree %d",
                (long long)q->H, Pu);
  if (q->S % ((int64_t)Pu * Pr) != 0)
    return fail(CRU_ENOTDIV,
                "sequence length %lld is not divisible by ulysses_degree * ring_degree = %lld",
                (long long)q->S, (long long)Pu * Pr);
  return CRU_OK;
}

cru_status cru_usp_workspace_bytes(const cru_tensor* q, int ulysses_degree, int ring_degree,
                                   size_t* bytes) {
  g_err[0] = '\0';
  if (bytes == nullptr) return fail(CRU_EINVAL, "bytes is NULL");
  CRU_TRY(check_tensor(q, "q"));
  CRU_TRY(usp_degrees(q, ulysses_degree, ring_degree));
  size_t y, ring;
  *bytes = usp_parts(q, ulysses_degree, ring_degree, &y, &ring);
  return CRU_OK;
}

cru_status cru_usp_emulate(const cru_tensor* q, const cru_tensor* k, const cru_tensor* v,
                           int ulysses_degree, int ring_degree, int fused, int convert_to_fp32,
                           const cru_tensor* o, const cru_lse* lse, float scale,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  CRU_TRY(check_qkvo(q, k, v, o));
  if (k->S != q->S)
    return fail(CRU_EINVAL, "USP shards one sequence: k has %lld rows, q %lld",
                (long long)k->S, (long long)q->S);
  if (lse != nullptr) CRU_TRY(check_lse(lse, "lse", q->B, q->H, q->S));
  if (fused != 0 && fused != 1) return fail(CRU_EINVAL, "fused must be 0 or 1");
  if (convert_to_fp32 != 0 && convert_to_fp32 != 1)
    return fail(CRU_EINVAL, "convert_to_fp32 must be 0 or 1");
  if (!convert_to_fp32 && q->dtype != CRU_BF16)
    return fail(CRU_EUNSUPPORTED, "partials in the model dtype need bf16 inputs");
  const int Pu = ulysses_degree, Pr = ring_degree;
  CRU_TRY(usp_degrees(q, Pu, Pr));
  float scale_log2 = 0.0f;
  CRU_TRY(check_scale(scale, q->D, &scale_log2));
  size_t y_bytes, ring_bytes;
  const size_t need = usp_parts(q, Pu, Pr, &y_bytes, &ring_bytes);
  if (need > 0 && workspace == nullptr) return fail(CRU_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(CRU_EWORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(CRU_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if (q->B * q->S * q->H == 0) return CRU_OK;

  const int64_t B = q->B, S = q->S, H = q->H, D = q->D, Hp = H / Pu;
  char* ws = static_cast<char*>(workspace);
  void* y[3] = {ws, ws + y_bytes, ws + 2 * y_bytes};
  void* ring_ws = ws + 3 * y_bytes;

  const cru_tensor x3[3] = {*q, *k, *v};
  CRU_TRY(cru_ulysses_seq2head(3, x3, y, Pu, 0, stream));

  const int64_t group = B * S * Hp * D;    // elements of one head group
  const int o_es = elem_bytes(o->dtype), in_es = elem_bytes(q->dtype);
  for (int u = 0; u < Pu; ++u) {
    cru_tensor t[3];
    for (int i = 0; i < 3; ++i) {
      t[i] = *q;
      t[i].data = static_cast<char*>(y[i]) + u * group * in_es;
      t[i].H = Hp;
      t[i].sb = S * Hp * D; t[i].ss = Hp * D; t[i].sh = D;
    }
    // the group's heads of o: the fold stores there directly
    cru_tensor o_u = *o;
    o_u.data = static_cast<char*>(o->data) + u * Hp * o->sh * o_es;
    o_u.H = Hp;
    cru_lse lse_u;
    if (lse != nullptr) {
      lse_u = *lse;
      lse_u.data = lse->data + u * Hp * lse->sh;
      lse_u.H = Hp;
    }
    CRU_TRY(cru_ring_emulate(&t[0], &t[1], &t[2], Pr, 0, nullptr, fused, convert_to_fp32, &o_u,
                             lse ? &lse_u : nullptr, scale, ring_ws, ring_bytes, stream));
  }
  return CRU_OK;
}

}  // extern "C"
