// fa_api.hip - the C ABI of libfa.so (declared in include/fa.h).
//
// Every argument is validated on the host before any HIP call, so a
// rejected call touches neither the device nor the outputs and returns a
// negative FA_E* code. Accepted calls launch on the caller's stream and
// return hipGetLastError() of the launch (0 on success).
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_kernels.h"

namespace {

constexpr long kMaxIndex = 0x7fffffffL;  // 32-bit element offsets per head
constexpr int kMaxRanges = 65536;        // decode page ranges per KV head
constexpr int kMaxPrefillPages = 8192;   // pages per request, paged prefill

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool mul_ok(long a, long b, long* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Element count of a 4-d tensor, or -1 on overflow.
long numel4(long a, long b, long c, long d) {
  long x;
  if (!mul_ok(a, b, &x) || !mul_ok(x, c, &x) || !mul_ok(x, d, &x)) return -1;
  return x;
}

}  // namespace

extern "C" {

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_EINVAL_NULL: return "a required pointer is NULL";
    case FA_EINVAL_DIM: return "a size is not positive, or a tensor is too large";
    case FA_EUNSUPPORTED_D: return "head dimension must be 64 or 128";
    case FA_EGQA: return "Hq must be a multiple of Hkv (and Hq/Hkv <= 16 for decode)";
    case FA_EDTYPE: return "unknown dtype";
    case FA_EDESCALE: return "qkv_descale must be three positive finite floats for fp8 and NULL otherwise";
    case FA_ESCALE: return "softmax scale must be finite and > 0";
    case FA_EPAGE: return "page_size must be 16 and num_pages >= 1";
    case FA_EWORKSPACE: return "workspace missing, misaligned or too small";
    case FA_ESPLITS: return "num_splits is negative or above 65536";
    case FA_EALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ESCRATCH: return "the decode needs more than the library's built-in 16 MiB workspace for these sizes";
    default: break;
  }
  if (code > 0) return "HIP launch error (the value is a hipError_t)";
  return "unknown error code";
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
           int causal, int dtype, const float* qkv_descale, void* stream) {
  if (!q || !k || !v || !o) return FA_EINVAL_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return FA_EINVAL_DIM;
  if (d != 64 && d != 128) return FA_EUNSUPPORTED_D;
  if (Hq % Hkv != 0) return FA_EGQA;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 &&
      dtype != FA_DTYPE_FP8_E4M3)
    return FA_EDTYPE;
  float sq = 1.f, sk = 1.f, sv = 1.f;
  if (dtype == FA_DTYPE_FP8_E4M3) {
    if (!qkv_descale) return FA_EDESCALE;
    sq = qkv_descale[0];
    sk = qkv_descale[1];
    sv = qkv_descale[2];
    if (!(isfinite(sq) && isfinite(sk) && isfinite(sv) && sq > 0.f &&
          sk > 0.f && sv > 0.f))
      return FA_EDESCALE;
  } else if (qkv_descale) {
    return FA_EDESCALE;
  }
  if (!(isfinite(scale) && scale > 0.f)) return FA_ESCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      ((uintptr_t)lse & 3u) != 0)
    return FA_EALIGN;
  // sizes: per-head offsets are 32-bit, whole tensors 64-bit, grid 31-bit
  if ((long)Nq * d > kMaxIndex || (long)Nk * d > kMaxIndex) return FA_EINVAL_DIM;
  if (numel4(B, Hq, Nq, d) < 0 || numel4(B, Hkv, Nk, d) < 0) return FA_EINVAL_DIM;
  const long n_qt = (Nq + 127) / 128;
  long blocks;
  if (!mul_ok(n_qt, (long)Hq * B, &blocks) || blocks > kMaxIndex)
    return FA_EINVAL_DIM;
  if ((long)B * Hq > kMaxIndex || (long)B * Hkv > kMaxIndex) return FA_EINVAL_DIM;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.s_q = sq;
  a.s_k = sk;
  a.s_v = sv;
  a.stream = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == FA_DTYPE_F32) e = fa::launch_fwd_f32(a);
  else if (dtype == FA_DTYPE_BF16) e = fa::launch_fwd_bf16(a);
  else e = fa::launch_fwd_fp8(a);
  return (int)e;
}

size_t fa_bwd_workspace_size(int B, int Hq, int Nq) {
  if (B <= 0 || Hq <= 0 || Nq <= 0) return 0;
  if (numel4(B, Hq, Nq, 1) < 0 || (long)B * Hq * Nq > kMaxIndex * 64L) return 0;
  return fa::bwd_workspace_bytes(B, Hq, Nq);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
           int causal, int dtype, void* workspace, size_t workspace_bytes,
           void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return FA_EINVAL_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return FA_EINVAL_DIM;
  if (d != 64 && d != 128) return FA_EUNSUPPORTED_D;
  if (Hq % Hkv != 0) return FA_EGQA;
  if (dtype != FA_DTYPE_BF16) return FA_EDTYPE;
  if (!(isfinite(scale) && scale > 0.f)) return FA_ESCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      ((uintptr_t)lse & 3u) != 0)
    return FA_EALIGN;
  if ((long)Nq * d > kMaxIndex || (long)Nk * d > kMaxIndex) return FA_EINVAL_DIM;
  if (numel4(B, Hq, Nq, d) < 0 || numel4(B, Hkv, Nk, d) < 0) return FA_EINVAL_DIM;
  long blocks;
  if (!mul_ok((Nq + 127) / 128, (long)Hq * B, &blocks) || blocks > kMaxIndex)
    return FA_EINVAL_DIM;
  if (!mul_ok((Nk + 127) / 128, (long)Hkv * B, &blocks) || blocks > kMaxIndex)
    return FA_EINVAL_DIM;
  if ((long)B * Hq * Nq * (d / 8) / 256 > kMaxIndex) return FA_EINVAL_DIM;
  const size_t need = fa_bwd_workspace_size(B, Hq, Nq);
  if (need == 0) return FA_EINVAL_DIM;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return FA_EWORKSPACE;

  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.ws = workspace;
  a.stream = static_cast<hipStream_t>(stream);
  return (int)fa::launch_bwd_bf16(a);
}

size_t fa_naive_workspace_size(int B, int Hq, int Nq, int Nk) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || Nk <= 0) return 0;
  if (numel4(B, Hq, Nq, Nk) < 0 || numel4(B, Hq, Nq, Nk) > INT64_MAX / 4) return 0;
  return fa::naive_workspace_bytes(B, Hq, Nq, Nk);
}

int fa_naive_attention(const void* q, const void* k, const void* v, void* o,
                       float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                       int d, float scale, int causal, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return FA_EINVAL_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return FA_EINVAL_DIM;
  if (d != 64 && d != 128) return FA_EUNSUPPORTED_D;
  if (Hq % Hkv != 0) return FA_EGQA;
  if (!(isfinite(scale) && scale > 0.f)) return FA_ESCALE;
  if (Nk % 8 != 0 || Nk > 16384) return FA_EINVAL_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      ((uintptr_t)lse & 3u) != 0)
    return FA_EALIGN;
  if ((long)Nq * d > kMaxIndex || (long)Nk * d > kMaxIndex) return FA_EINVAL_DIM;
  if (numel4(B, Hq, Nq, d) < 0 || numel4(B, Hkv, Nk, d) < 0) return FA_EINVAL_DIM;
  if ((long)B * Hq * Nq > kMaxIndex) return FA_EINVAL_DIM;
  const size_t need = fa_naive_workspace_size(B, Hq, Nq, Nk);
  if (need == 0) return FA_EINVAL_DIM;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return FA_EWORKSPACE;
  fa::NaiveArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.ws = workspace;
  a.stream = static_cast<hipStream_t>(stream);
  return (int)fa::launch_naive_bf16(a);
}

int fa_paged_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens,
                     int page_size, int num_pages, int B, int Hq, int Hkv,
                     int Nq, int d, int max_pages_per_seq, float scale,
                     int causal, void* o, float* lse, void* stream) {
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !o)
    return FA_EINVAL_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || max_pages_per_seq <= 0)
    return FA_EINVAL_DIM;
  if (d != 64 && d != 128) return FA_EUNSUPPORTED_D;
  if (Hq % Hkv != 0) return FA_EGQA;
  if (page_size != 16 || num_pages <= 0) return FA_EPAGE;
  if (max_pages_per_seq > kMaxPrefillPages) return FA_EINVAL_DIM;
  if (!(isfinite(scale) && scale > 0.f)) return FA_ESCALE;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned16(o) || ((uintptr_t)lse & 3u) != 0 ||
      ((uintptr_t)block_table & 3u) != 0 || ((uintptr_t)seq_lens & 3u) != 0)
    return FA_EALIGN;
  if ((long)Nq * d > kMaxIndex || numel4(B, Hq, Nq, d) < 0) return FA_EINVAL_DIM;
  if (numel4(num_pages, page_size, Hkv, d) < 0) return FA_EINVAL_DIM;
  if ((long)B * max_pages_per_seq > kMaxIndex) return FA_EINVAL_DIM;
  long blocks;
  if (!mul_ok((Nq + 127) / 128, (long)Hq * B, &blocks) || blocks > kMaxIndex)
    return FA_EINVAL_DIM;
  fa::FwdArgs a;
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = 0;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.s_q = a.s_k = a.s_v = 1.f;
  a.stream = static_cast<hipStream_t>(stream);
  return (int)fa::launch_paged_prefill_bf16(a, block_table, seq_lens,
                                            max_pages_per_seq, num_pages);
}

static int decode_check(int B, int Hq, int Hkv, int d, int max_pages,
                        int page_size, int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_pages <= 0) return FA_EINVAL_DIM;
  if (d != 64 && d != 128) return FA_EUNSUPPORTED_D;
  if (Hq % Hkv != 0 || Hq / Hkv > 16) return FA_EGQA;
  if (page_size != 16) return FA_EPAGE;
  if (num_splits < 0 || num_splits > kMaxRanges) return FA_ESPLITS;
  if ((long)max_pages * page_size > kMaxIndex) return FA_EINVAL_DIM;
  if ((long)B * Hq > kMaxIndex / 256) return FA_EINVAL_DIM;
  if ((long)B * max_pages > kMaxIndex) return FA_EINVAL_DIM;
  return FA_OK;
}

size_t fa_paged_decode_workspace_size(int B, int Hq, int Hkv, int d,
                                      int max_pages_per_seq, int page_size,
                                      int num_splits) {
  if (decode_check(B, Hq, Hkv, d, max_pages_per_seq, page_size, num_splits) !=
      FA_OK)
    return 0;
  fa::DecodePlan plan;
  if (!fa::plan_decode(B, Hq, Hkv, d, max_pages_per_seq, num_splits, &plan))
    return 0;
  return plan.workspace_bytes;
}

static int paged_decode_common(const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, int page_size,
                               int num_pages, int B, int Hq, int Hkv, int d,
                               int max_pages_per_seq, float scale, void* o,
                               float* lse, void* workspace,
                               size_t workspace_bytes, int num_splits,
                               bool kv_fp8, float s_k, float s_v,
                               void* stream, bool use_scratch = false) {
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !o)
    return FA_EINVAL_NULL;
  const int c = decode_check(B, Hq, Hkv, d, max_pages_per_seq, page_size,
                             num_splits);
  if (c != FA_OK) return c;
  if (num_pages <= 0) return FA_EPAGE;
  if (numel4(num_pages, page_size, Hkv, d) < 0) return FA_EINVAL_DIM;
  if (!(isfinite(scale) && scale > 0.f)) return FA_ESCALE;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned16(o) || ((uintptr_t)lse & 3u) != 0 ||
      ((uintptr_t)block_table & 3u) != 0 || ((uintptr_t)seq_lens & 3u) != 0)
    return FA_EALIGN;
  fa::DecodePlan plan;
  if (!fa::plan_decode(B, Hq, Hkv, d, max_pages_per_seq, num_splits, &plan))
    return FA_ESPLITS;
  if (use_scratch) {
    // the built-in workspace: an automatic range count is lowered until the
    // plan fits it; a count the caller chose must fit as it is
    if (plan.workspace_bytes > fa::kDecodeScratchBytes) {
      if (num_splits != 0) return FA_ESCRATCH;
      const long rows = ((long)(fa::kDecodeScratchBytes / 4) - plan.off_o) /
                        ((long)Hq * (d + 1));
      const long r_max = (rows - B) / plan.waves_per_head * plan.waves_per_head;
      if (r_max < plan.waves_per_head) return FA_ESCRATCH;
      if (!fa::plan_decode(B, Hq, Hkv, d, max_pages_per_seq, (int)r_max, &plan) ||
          plan.workspace_bytes > fa::kDecodeScratchBytes)
        return FA_ESCRATCH;
    }
    const hipError_t e = fa::decode_scratch(&workspace);
    if (e != hipSuccess) return (int)e;
  } else if (!workspace || workspace_bytes < plan.workspace_bytes ||
             ((uintptr_t)workspace & 255u) != 0) {
    return FA_EWORKSPACE;
  }

  fa::DecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.num_pages = num_pages;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.max_pages = max_pages_per_seq;
  a.scale = scale;
  a.o = o;
  a.lse = lse;
  a.ws = workspace;
  a.kv_fp8 = kv_fp8;
  a.s_k = s_k;
  a.s_v = s_v;
  a.stream = static_cast<hipStream_t>(stream);
  return (int)fa::launch_paged_decode(a, plan);
}

int fa_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int page_size, int num_pages, int B, int Hq, int Hkv,
                    int d, int max_pages_per_seq, float scale, void* o,
                    float* lse, void* workspace, size_t workspace_bytes,
                    int num_splits, void* stream) {
  return paged_decode_common(q, k_pool, v_pool, block_table, seq_lens,
                             page_size, num_pages, B, Hq, Hkv, d,
                             max_pages_per_seq, scale, o, lse, workspace,
                             workspace_bytes, num_splits, false, 1.f, 1.f,
                             stream);
}

int fa_paged_decode_noalloc(const void* q, const void* k_pool,
                            const void* v_pool, const int32_t* block_table,
                            const int32_t* seq_lens, int page_size,
                            int num_pages, int B, int Hq, int Hkv, int d,
                            int max_pages_per_seq, float scale, void* o,
                            float* lse, int num_splits, void* stream) {
  return paged_decode_common(q, k_pool, v_pool, block_table, seq_lens,
                             page_size, num_pages, B, Hq, Hkv, d,
                             max_pages_per_seq, scale, o, lse, nullptr, 0,
                             num_splits, false, 1.f, 1.f, stream, true);
}

int fa_paged_decode_fp8kv(const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_lens, int page_size,
                          int num_pages, int B, int Hq, int Hkv, int d,
                          int max_pages_per_seq, float scale,
                          const float* kv_descale, void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          int num_splits, void* stream) {
  if (!kv_descale) return FA_EDESCALE;
  const float s_k = kv_descale[0], s_v = kv_descale[1];
  if (!(isfinite(s_k) && isfinite(s_v) && s_k > 0.f && s_v > 0.f))
    return FA_EDESCALE;
  return paged_decode_common(q, k_pool, v_pool, block_table, seq_lens,
                             page_size, num_pages, B, Hq, Hkv, d,
                             max_pages_per_seq, scale, o, lse, workspace,
                             workspace_bytes, num_splits, true, s_k, s_v,
                             stream);
}

}  // extern "C"
