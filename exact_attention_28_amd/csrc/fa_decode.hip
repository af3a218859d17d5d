// fa_decode.hip - paged-KV-cache decode (one query token per request), gfx950.
//
// The cache of each request lives in 16-token pages mapped by a block table
// ([FA3-paged §3.2]). This kernel is bandwidth bound: every K/V byte is read
// once from HBM and used by the Hq/Hkv query heads of its group together.
//
// Work split (balanced split-KV). The pages of the whole batch, request
// after request, form one list of T pages; it is cut into R ranges of equal
// length (R about the number of waves the GPU holds at once, divided by
// Hkv). One wave owns one (range, KV head): it walks the range's pages in
// order, with K/V loads two pages ahead of the page it computes, and every
// time it leaves a request (or the range ends) it emits that request's
// piece. A piece that is a whole request is written as the final output; a
// piece of a request cut by a range border is written as a normalised
// partial with its log-sum-exp, and a small second kernel merges those with
// the log-sum-exp form of the two-block merge ([Capstone §2.2 step 4],
// appendix A Q1): one wave per (request, query head), or, when a call
// cuts each request into many pieces (few, long requests), a workgroup of
// eight waves per (request, query head). Ranges never depend on request lengths, so long and short
// requests cost the same per page and the grid finishes together.
//
// The waves of one workgroup hold different KV heads of the same range, so
// a workgroup of Hkv waves walks the same pages in lockstep and reads each
// page (all heads of 16 tokens, contiguous in the pool) as one block.
//
// The cache may also be stored as OCP e4m3 codes with per-tensor scales
// (s_k, s_v), which halves the bytes to stream: the codes of K and V are
// widened exactly to bf16 in registers for the two products, s_k is folded
// into the exp2 multiplier and s_v into the final 1/l, so the arithmetic
// is that of the bf16 cache on the dequantised
// values ([FA3-guide] fp8 listing for the per-tensor scales, [FA3-paged
// §3.2] for the pages).
//
// Per wave and page (16 tokens of one KV head, rows of d elements at a
// stride of Hkv*d):
//   * S^T[token, head] = K . Q^T on v_mfma_f32_16x16x32_bf16, with K
//     fragments loaded straight from HBM into the A operand (lane: token
//     l%16, 16 B of d) and the group's query heads as the B operand
//     (lane: head l%16; heads past the group are zero);
//   * online softmax per head (column): lane-local over 4 tokens, then two
//     cross-row steps, with the lazy rescale of the prefill kernels;
//   * O[head, d] += P V on v_mfma_f32_16x16x16_bf16, P rounded to bf16
//     (the A operand is the score step's output layout, so P never moves
//     between lanes); a lane reads the V rows of its 4 tokens, D/16
//     contiguous d each, straight from HBM, and byte permutes pair the rows
//     into the B operand (an e4m3 pair is then widened exactly to bf16).
//     O is divided by the sum of the rounded P, the log-sum-exp takes the
//     sum of the unrounded P.
#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

// Built-in workspace of the decode for callers that cannot allocate device
// memory (fa_paged_decode_noalloc): every device the library runs on holds
// one copy of this array for the life of the process. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// for the symbol); it uses the device address that decode_scratch() looks
// up once per device.
static __device__ __align__(256) unsigned char scratch[fa::kDecodeScratchBytes];

namespace fa {
namespace {

constexpr int kPage = 16;
constexpr int kSlots8 = 2;  // pages in flight per wave, e4m3 cache

// Workspace layout, in 4-byte words: T at word 0; the first and the last
// range that touch request b at kFirstWord + b and kFirstWord + B + b; then
// the partial outputs [(B + R) * Hq][D] fp32 and their log-sum-exps
// [(B + R) * Hq]. A piece of request b in range r has slot b + r: along the
// page list (request, range) pairs only grow, so slots never collide.
constexpr int kFirstWord = 64;

// Sizes and plan; the pointers are kernel arguments of their own, declared
// __restrict__, so the block table and lengths are read with scalar loads.
struct KParams {
  int num_pages, B, Hq, Hkv, G, Hh, WPH, ngroups, max_pages, R;
  float c;   // scale * log2(e) (* s_k for an e4m3 cache)
  float sv;  // s_v for an e4m3 cache, else 1
};

// Register images of one page slot's K and V for a lane: bf16 as stored,
// or the e4m3 codes (8 of d per K step, DL per V token row).
template <int D, bool KV8>
struct PageRegs;
template <int D>
struct PageRegs<D, false> {
  typedef uint32_t vrow_t __attribute__((ext_vector_type(D / 32)));
  bf16x8 k[D / 32];
  vrow_t v[4];
};
template <int D>
struct PageRegs<D, true> {
  // K: the lane's D/4 contiguous codes, d = (D/4) * row16 + 8s + (0..7)
  // for MFMA step s (the same permutation of d is applied to Q)
  u32x4 k[D / 64];
  // V: DL codes of each of the lane's 4 token rows
  typedef uint32_t vrow_t __attribute__((ext_vector_type(D / 64)));
  vrow_t v[4];
};
__device__ __forceinline__ int pages_of(int len, int max_len) {
  len = max(0, min(len, max_len));
  return (len + kPage - 1) / kPage;
}
__device__ __forceinline__ int clamp_len(int len, int max_len) {
  return max(0, min(len, max_len));
}
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}
__device__ __forceinline__ int uniform(int x) {
  return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
// O[head, d] += P[head, token] V[token, d] over one page's 16 tokens on
// v_mfma_f32_16x16x16_bf16: A = P (lane: head l%16, tokens 4*(l/16)+0..3,
// as the score step leaves them), B = V (lane: column l%16, the same four
// tokens). Product j takes d = DL*(l%16) + j for column l%16, so a lane's
// V rows, DL contiguous d each, feed the products without crossing lanes,
// and the result of product j for head 4*(l/16)+v at d = DL*(l%16)+j sits
// in element v of accumulator j of lane l.
__device__ __forceinline__ f32x4 mfma_16x16x16_bf16(uint32_t a01, uint32_t a23,
                                                    uint32_t b01, uint32_t b23,
                                                    f32x4 c) {
  const i16x4 a = __builtin_bit_cast(i16x4, u32x2{a01, a23});
  const i16x4 b = __builtin_bit_cast(i16x4, u32x2{b01, b23});
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// bf16 pairs: the low (or high) halves of two rows' words, row x first
__device__ __forceinline__ uint32_t lo_halves(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}
// e4m3 codes of two rows interleaved: bytes (x0, y0, x1, y1) (or of
// bytes 2 and 3), each pair then widened exactly to a bf16 pair
__device__ __forceinline__ uint32_t codes_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05010400u);
}
__device__ __forceinline__ uint32_t codes_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07030602u);
}
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair_bf16(uint32_t w) {
  return __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.f, HI));
}

template <int D, int NW, bool KV8>
__global__ __launch_bounds__(NW * 64) void decode_kernel(
    KParams a, const __bf16* __restrict__ Qp, const void* __restrict__ KPv,
    const void* __restrict__ VPv, const int32_t* __restrict__ BT,
    const int32_t* __restrict__ SL, int* __restrict__ wsi,
    float* __restrict__ ws_o, float* __restrict__ ws_l,
    __bf16* __restrict__ O, float* __restrict__ LSE) {
  constexpr int DL = D / 16;  // d columns per lane in the PV step
  typedef typename std::conditional<KV8, uint8_t, __bf16>::type kv_t;
  using Regs = PageRegs<D, KV8>;
  typedef uint32_t vload_t __attribute__((ext_vector_type(DL / 2)));  // DL bf16
  const kv_t* __restrict__ KP = static_cast<const kv_t*>(KPv);
  const kv_t* __restrict__ VP = static_cast<const kv_t*>(VPv);
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int row16 = lane >> 4;
  const int col = lane & 15;
  const int hg = blockIdx.x % a.ngroups;
  const int slot = blockIdx.x / a.ngroups;
  const int hl = w % a.Hh;
  const int sub = w / a.Hh;
  if (sub >= a.WPH) return;
  const int r = slot * a.WPH + sub;
  if (r >= a.R) return;
  const int hkv = hg * a.Hh + hl;
  const int G = a.G;
  const int max_len = a.max_pages * kPage;
  const long tok_stride = (long)a.Hkv * D;  // elements between tokens

  // ---- this wave's range [x0, x1) of the batch's page list
  int T = 0;
  for (int c0 = 0; c0 < a.B; c0 += 64) {
    const int i = c0 + lane;
    T += wave_sum(i < a.B ? pages_of(SL[i], max_len) : 0);
  }
  T = uniform(T);
  if (blockIdx.x == 0 && w == 0 && lane == 0) wsi[0] = T;
  const int x0 = (int)((long)r * T / a.R);
  const int x1 = (int)((long)(r + 1) * T / a.R);
  if (x0 >= x1) return;

  // request holding page x0 and the list index of its first page
  int b0 = 0, s0 = 0;
  {
    int S = 0;
    for (int c0 = 0; c0 < a.B; c0 += 64) {
      const int i = c0 + lane;
      const int n = i < a.B ? pages_of(SL[i], max_len) : 0;
      const int incl = S + wave_incl_scan(n, lane);
      const unsigned long long hit = __ballot(incl > x0);
      if (hit != 0ull) {
        const int f = uniform(__builtin_ctzll(hit));
        b0 = c0 + f;
        s0 = __builtin_amdgcn_readlane(incl - n, f);
        break;
      }
      S = __builtin_amdgcn_readlane(incl, 63);
    }
  }

  auto page_base = [&](int id, bool& bad) -> long {
    bad = id < 0 || id >= a.num_pages;  // never dereferenced: piece -> NaN
    if (bad) id = 0;
    return ((long)id * kPage * a.Hkv + hkv) * D;
  };
  // K and V are read exactly once: nontemporal loads stream them past the
  // caches instead of evicting lines other waves still use (-10% time).
  auto load_page = [&](long base, Regs& pr) {
    const kv_t* kp = KP + base + (long)col * tok_stride +
                     (KV8 ? (D / 4) * row16 : 8 * row16);
    const kv_t* vp = VP + base + (long)(4 * row16) * tok_stride + DL * col;
    if constexpr (!KV8) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
        pr.k[s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(kp + 32 * s));
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        pr.v[rr] = __builtin_nontemporal_load(
            reinterpret_cast<const typename Regs::vrow_t*>(vp + rr * tok_stride));
    } else {
#pragma unroll
      for (int s = 0; s < D / 64; ++s)
        pr.k[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + 16 * s));
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        pr.v[rr] = __builtin_nontemporal_load(
            reinterpret_cast<const typename Regs::vrow_t*>(vp + rr * tok_stride));
    }
  };

  // query heads of the group as the B operand: head col, d = 32s + 8*row16
  // (e4m3 cache: d = (D/4)*row16 + 8s, the K codes' order)
  bf16x8 qf[D / 32];
  // exponent reference of head `col`; its partial sums of P, unrounded (for
  // the log-sum-exp) and as rounded to bf16 for the products (for O)
  float m, lp, lr;
  f32x4 oacc[DL];
  bool piece_bad;

  auto process = [&](const Regs& pr_in, bool bad, int page, int lim) {
    piece_bad |= bad;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      bf16x8 kf;
      if constexpr (!KV8) {
        kf = pr_in.k[s];
      } else {
        // e4m3 pairs straight to bf16 pairs (exact: scale 1, 3 -> 7
        // mantissa bits)
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const int w0 = (int)pr_in.k[s / 2][2 * (s & 1)];
        const int w1 = (int)pr_in.k[s / 2][2 * (s & 1) + 1];
        const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false);
        const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true);
        const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false);
        const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true);
        kf = bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
      }
      acc = mfma_16x16x32_bf16(kf, qf[s], acc);
    }
    // lane: tokens 4*row16 + v of this page, head col
    const int tok0 = page * kPage + 4 * row16;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (tok0 + v >= lim) acc[v] = kNegInf;
    float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = max_halves(mx);
    const float mxs = mx * a.c;
    const bool need = (col < G) && (mxs > m + kTau);
    if (__any(need)) {
      const float mnew = fmaxf(m, mxs);
      const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - mnew);
      lp *= alpha;
      lr *= alpha;
      m = mnew;
      // heads 4*row16 + v of this lane's accumulators: alpha of lane col = head
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = __shfl(alpha, 4 * row16 + v, 64);
#pragma unroll
        for (int j = 0; j < DL; ++j) oacc[j][v] *= av;
      }
    }
    const float mref = (m == kNegInf) ? 0.f : m;
    float pr[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pr[v] = fast_exp2(__builtin_fmaf(acc[v], a.c, -mref));
      lp += pr[v];
    }
    const uint32_t p01 = pack_bf16x2(pr[0], pr[1]);
    const uint32_t p23 = pack_bf16x2(pr[2], pr[3]);
    lr = add_bf16x2(p23, add_bf16x2(p01, lr));
    // V rows of the lane's four tokens. A token past the piece (the tail of
    // a request's last page) has P = 0, but its V row is a cache slot whose
    // contents are unspecified: it is taken as 0, so that 0 * NaN cannot
    // reach O.
    typename Regs::vrow_t vr[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      vr[rr] = pr_in.v[rr];
      if (tok0 + rr >= lim) vr[rr] = typename Regs::vrow_t{};
    }
    if constexpr (!KV8) {
      // word e of a row holds d = DL*col + 2e (low half) and 2e + 1
#pragma unroll
      for (int e = 0; e < DL / 2; ++e) {
        oacc[2 * e] = mfma_16x16x16_bf16(p01, p23, lo_halves(vr[0][e], vr[1][e]),
                                         lo_halves(vr[2][e], vr[3][e]), oacc[2 * e]);
        oacc[2 * e + 1] = mfma_16x16x16_bf16(p01, p23, hi_halves(vr[0][e], vr[1][e]),
                                             hi_halves(vr[2][e], vr[3][e]), oacc[2 * e + 1]);
      }
    } else {
      // word e of a row holds the codes of d = DL*col + 4e + (0..3)
#pragma unroll
      for (int e = 0; e < DL / 4; ++e) {
        const uint32_t x01 = codes_lo(vr[0][e], vr[1][e]);
        const uint32_t x23 = codes_lo(vr[2][e], vr[3][e]);
        const uint32_t y01 = codes_hi(vr[0][e], vr[1][e]);
        const uint32_t y23 = codes_hi(vr[2][e], vr[3][e]);
        oacc[4 * e] = mfma_16x16x16_bf16(p01, p23, e4m3_pair_bf16<false>(x01),
                                         e4m3_pair_bf16<false>(x23), oacc[4 * e]);
        oacc[4 * e + 1] = mfma_16x16x16_bf16(p01, p23, e4m3_pair_bf16<true>(x01),
                                             e4m3_pair_bf16<true>(x23), oacc[4 * e + 1]);
        oacc[4 * e + 2] = mfma_16x16x16_bf16(p01, p23, e4m3_pair_bf16<false>(y01),
                                             e4m3_pair_bf16<false>(y23), oacc[4 * e + 2]);
        oacc[4 * e + 3] = mfma_16x16x16_bf16(p01, p23, e4m3_pair_bf16<true>(y01),
                                             e4m3_pair_bf16<true>(y23), oacc[4 * e + 3]);
      }
    }
  };

  // Pieces: the part of request b inside this range, pages [p, pe).
  // pages in flight per wave: two for both storages (an e4m3 page is half
  // the bytes, but three or four of them in flight measured slower)
  constexpr int NS = KV8 ? kSlots8 : 2;
  Regs slot_regs[NS];
  bool slot_bad[NS];
  int b = b0, p = x0 - s0, x = x0;
  for (;;) {
    const int L = clamp_len(SL[b], max_len);
    const int n = (L + kPage - 1) / kPage;
    const int pe = min(n, p + (x1 - x));
    if (pe <= p) break;  // only if the lengths changed during the call
    const int lim = min(L, pe * kPage);  // tokens past the piece are masked
    const int32_t* row = BT + (long)b * a.max_pages;
    {
      const bool qv = col < G;
      const __bf16* qrow =
          Qp + ((long)b * a.Hq + (long)hkv * G + (qv ? col : 0)) * D;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const int qd = KV8 ? (D / 4) * row16 + 8 * s : 32 * s + 8 * row16;
        bf16x8 q8 = *reinterpret_cast<const bf16x8*>(qrow + qd);
        if (!qv) q8 = bf16x8{};
        qf[s] = q8;
      }
    }
    m = kNegInf;
    lp = 0.f;
    lr = 0.f;
#pragma unroll
    for (int j = 0; j < DL; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    piece_bad = false;

    // NS page slots, each reloaded right after it is computed. Loads past
    // the piece repeat its last page (cached, never used); the pages a
    // piece's last round computes past its end are fully masked.
    // The prologue issues Q, then slots 0, 1, ... in order (the barriers
    // pin it), the same order the loop leaves behind, so the wait before a
    // slot is computed counts only that slot's loads.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      load_page(page_base(row[min(p + sl, pe - 1)], slot_bad[sl]), slot_regs[sl]);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int q = p; q < pe; q += NS) {
      int ids[NS];
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) ids[sl] = row[min(q + NS + sl, pe - 1)];
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        process(slot_regs[sl], slot_bad[sl], q + sl, lim);
        // keep each reload after the last read of its slot
        __builtin_amdgcn_sched_barrier(0);
        load_page(page_base(ids[sl], slot_bad[sl]), slot_regs[sl]);
      }
    }

    // Emit the piece: final output when it is the whole request, else a
    // partial in slot b + r.
    const bool first = p == 0, req_end = pe == n;
    const bool whole = first && req_end;
    // per head (lane col): sums over the four token rows, the scale of O and
    // the log-sum-exp; then to the lanes that hold the head's outputs
    float ls = lp + xor_lane(lp, 16);
    ls += xor_lane(ls, 32);
    float lrs = lr + xor_lane(lr, 16);
    lrs += xor_lane(lrs, 32);
    const bool live = ls > 0.f;
    float inv = live ? a.sv / lrs : 0.f;
    float lse = live ? (m + fast_log2(ls)) * kLn2 : kNegInf;
    if (piece_bad) {
      inv = __builtin_nanf("");
      lse = __builtin_nanf("");
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int g = 4 * row16 + v;
      const float inv_g = __shfl(inv, g, 64);
      const float lse_g = __shfl(lse, g, 64);
      if (g >= G) continue;
      const long hq = (long)b * a.Hq + (long)hkv * G + g;
      if (whole) {
        vload_t st;
#pragma unroll
        for (int e = 0; e < DL / 2; ++e)
          st[e] = pack_bf16x2(oacc[2 * e][v] * inv_g, oacc[2 * e + 1][v] * inv_g);
        *reinterpret_cast<vload_t*>(O + hq * D + DL * col) = st;
        if (col == 0 && LSE != nullptr) LSE[hq] = lse_g;
      } else {
        const long ph = ((long)b + r) * a.Hq + (long)hkv * G + g;
        float* po = ws_o + ph * D + DL * col;
#pragma unroll
        for (int e = 0; e < DL; e += 4) {
          f32x4 t = {oacc[e][v] * inv_g, oacc[e + 1][v] * inv_g,
                     oacc[e + 2][v] * inv_g, oacc[e + 3][v] * inv_g};
          *reinterpret_cast<f32x4*>(po + e) = t;
        }
        if (col == 0) ws_l[ph] = lse_g;
      }
    }
    if (hkv == 0 && lane == 0) {
      if (first) wsi[kFirstWord + b] = r;
      if (req_end) wsi[kFirstWord + a.B + b] = r;
    }

    x += pe - p;
    if (x >= x1) break;
    do {
      ++b;
    } while (b + 1 < a.B && pages_of(SL[b], max_len) == 0);
    p = 0;
  }
}

// One wave per (request, query head): merge the pieces of requests that a
// range border cut; write O = 0, LSE = -inf for empty requests. A lane owns
// D/64 output columns. The bookkeeping words are read together, then the
// pieces are taken four at a time with all their loads issued before any
// is used (one online merge over the pieces), so the kernel waits for few
// memory round trips.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const int* __restrict__ wsi, const float* __restrict__ ws_o,
    const float* __restrict__ ws_l, const int32_t* __restrict__ SL,
    int max_pages, int R, int Hq, int B, __bf16* __restrict__ O,
    float* __restrict__ LSE) {
  constexpr int DPL = D / 64;
  const long hq = blockIdx.x;  // b * Hq + h
  const int b = (int)(hq / Hq);
  const int h = (int)(hq - (long)b * Hq);
  const int lane = threadIdx.x;
  const int len = SL[b];
  const int r_first = wsi[kFirstWord + b];
  const int r_last = wsi[kFirstWord + B + b];
  const long T = wsi[0];
  __bf16* orow = O + hq * D + DPL * lane;
  if (pages_of(len, max_pages * kPage) == 0) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) orow[e] = (__bf16)0.f;
    if (lane == 0 && LSE != nullptr) LSE[hq] = kNegInf;
    return;
  }
  if (r_first == r_last) return;  // one piece: written as the final output
  // ranges strictly inside [r_first, r_last] may be empty (T < R)
  // (ranges are never empty when the list has at least R pages, which
  // spares the 64-bit divisions)
  auto live = [&](int r) {
    return r <= r_last &&
           (T >= R || (long)r * T / R < (long)(r + 1) * T / R);
  };
  float M = kNegInf, tot = 0.f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  bool nan = false;
  for (int r0 = r_first; r0 <= r_last; r0 += 4) {
    float lj[4], oj[4][DPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = live(r0 + u);
      const long ph = ((long)b + (ok ? r0 + u : r_first)) * Hq + h;
      lj[u] = ok ? ws_l[ph] : kNegInf;
#pragma unroll
      for (int e = 0; e < DPL; ++e) oj[u][e] = ok ? ws_o[ph * D + DPL * lane + e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      nan |= (lj[u] != lj[u]);
      if (!(lj[u] > kNegInf)) continue;  // empty range or NaN: weight 0
      const float mn = fmaxf(M, lj[u]);
      const float fo = (M == kNegInf) ? 0.f : fast_exp2((M - mn) * kLog2e);
      const float fj = fast_exp2((lj[u] - mn) * kLog2e);
      tot = tot * fo + fj;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = acc[e] * fo + fj * oj[u][e];
      M = mn;
    }
  }
  float inv = M != kNegInf ? 1.f / tot : 0.f;
  float L_out = M != kNegInf ? M + fast_log2(tot) * kLn2 : kNegInf;
  if (nan) {
    inv = __builtin_nanf("");
    L_out = __builtin_nanf("");
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) orow[e] = (__bf16)(acc[e] * inv);
  if (lane == 0 && LSE != nullptr) LSE[hq] = L_out;
}

// The same merge for calls with many pieces per request (a few requests,
// long ranges cut into many): one 8-wave workgroup per (request, query
// head). Each wave merges every 8th piece, up to 32 at a time with all
// their loads issued before any is used (an online merge with the wave's
// own running maximum); the eight partial results then meet in LDS with
// the log-sum-exp form of the two-block merge ([Capstone §2.2 step 4]).
template <int D>
__global__ __launch_bounds__(512) void decode_merge_wide_kernel(
    const int* __restrict__ wsi, const float* __restrict__ ws_o,
    const float* __restrict__ ws_l, const int32_t* __restrict__ SL,
    int max_pages, int R, int Hq, int B, __bf16* __restrict__ O,
    float* __restrict__ LSE) {
  constexpr int NWV = 8, DPL = D / 64, U = 32;
  const long hq = blockIdx.x;  // b * Hq + h
  const int b = (int)(hq / Hq);
  const int h = (int)(hq - (long)b * Hq);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int len = SL[b];
  const int r_first = wsi[kFirstWord + b];
  const int r_last = wsi[kFirstWord + B + b];
  const long T = wsi[0];
  __bf16* orow = O + hq * D + DPL * lane;
  // (uniform over the workgroup: the request decides)
  if (pages_of(len, max_pages * kPage) == 0) {
    if (w == 0) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) orow[e] = (__bf16)0.f;
      if (lane == 0 && LSE != nullptr) LSE[hq] = kNegInf;
    }
    return;
  }
  if (r_first == r_last) return;  // one piece: written as the final output
  // (ranges are never empty when the list has at least R pages, which
  // spares the 64-bit divisions)
  auto live = [&](int r) {
    return r <= r_last &&
           (T >= R || (long)r * T / R < (long)(r + 1) * T / R);
  };
  __shared__ float s_m[NWV], s_tot[NWV];
  __shared__ int s_nan[NWV];
  __shared__ float s_acc[NWV][D];
  float M = kNegInf, tot = 0.f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  int nan = 0;
  for (int r0 = r_first + w; r0 <= r_last; r0 += NWV * U) {
    // lane u < U fetches piece u's log-sum-exp (broadcast below); every
    // lane fetches its DPL columns of each piece in one load
    float my_l = kNegInf;
    {
      const int r = r0 + NWV * lane;
      if (lane < U && live(r)) my_l = ws_l[((long)b + r) * Hq + h];
    }
    typedef float fdpl_t __attribute__((ext_vector_type(DPL)));
    fdpl_t oj[U];
    float lj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + NWV * u;
      const bool ok = live(r);
      const long ph = ((long)b + (ok ? r : r_first)) * Hq + h;
      oj[u] = ok ? *reinterpret_cast<const fdpl_t*>(ws_o + ph * D + DPL * lane)
                 : fdpl_t{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) lj[u] = lane_value(my_l, u);
    // the batch's maximum first, so the running sums rescale once a batch
    float mb = M;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      nan |= (lj[u] != lj[u]);
      mb = fmaxf(mb, lj[u]);
    }
    if (mb == kNegInf) continue;  // nothing finite yet
    const float fo = (M == kNegInf) ? 0.f : fast_exp2((M - mb) * kLog2e);
    tot *= fo;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] *= fo;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!(lj[u] > kNegInf)) continue;  // empty range or NaN: weight 0
      const float wt = fast_exp2((lj[u] - mb) * kLog2e);
      tot += wt;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = __builtin_fmaf(wt, oj[u][e], acc[e]);
    }
    M = mb;
  }
  if (lane == 0) {
    s_m[w] = M;
    s_tot[w] = tot;
    s_nan[w] = nan;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) s_acc[w][DPL * lane + e] = acc[e];
  __syncthreads();
  if (w != 0) return;
  float Mx = kNegInf;
  nan = 0;
#pragma unroll
  for (int k = 0; k < NWV; ++k) {
    Mx = fmaxf(Mx, s_m[k]);
    nan |= s_nan[k];
  }
  float t = 0.f, a[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) a[e] = 0.f;
  if (Mx != kNegInf) {
#pragma unroll
    for (int k = 0; k < NWV; ++k) {
      if (s_m[k] == kNegInf) continue;  // a wave with no finite piece
      const float f = fast_exp2((s_m[k] - Mx) * kLog2e);
      t = __builtin_fmaf(s_tot[k], f, t);
#pragma unroll
      for (int e = 0; e < DPL; ++e) a[e] = __builtin_fmaf(s_acc[k][DPL * lane + e], f, a[e]);
    }
  }
  float inv = Mx != kNegInf ? 1.f / t : 0.f;
  float L_out = Mx != kNegInf ? Mx + fast_log2(t) * kLn2 : kNegInf;
  if (nan) {
    inv = __builtin_nanf("");
    L_out = __builtin_nanf("");
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) orow[e] = (__bf16)(a[e] * inv);
  if (lane == 0 && LSE != nullptr) LSE[hq] = L_out;
}

template <int D, int NW, bool KV8>
void* kernel_ptr() {
  return reinterpret_cast<void*>(&decode_kernel<D, NW, KV8>);
}

// Kernel instance for head dim d, waves per workgroup nw and the cache's
// storage (bf16 or e4m3 codes); every group size up to 16 heads shares it
// (the heads are the rows of the products).
template <bool KV8>
void* select_kernel_t(int d, int nw) {
  if (d == 128) return nw == 8 ? kernel_ptr<128, 8, KV8>() : kernel_ptr<128, 4, KV8>();
  return nw == 8 ? kernel_ptr<64, 8, KV8>() : kernel_ptr<64, 4, KV8>();
}
void* select_kernel(int d, int nw, bool kv8) {
  return kv8 ? select_kernel_t<true>(d, nw) : select_kernel_t<false>(d, nw);
}

// Waves the current device holds at once for this kernel instance.
int resident_waves(void* kernel, int nw) {
  int dev = 0, cus = 256, blocks = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &blocks, reinterpret_cast<const void*>(kernel), nw * 64, 0) !=
          hipSuccess ||
      blocks <= 0)
    blocks = 1;
  return cus * blocks * nw;
}

}  // namespace

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices] = {};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

bool plan_decode(int B, int Hq, int Hkv, int d, int max_pages, int num_splits,
                 DecodePlan* p) {
  const int G = Hq / Hkv;
  const int nw = Hkv % 8 == 0 ? 8 : 4;
  // heads per workgroup: the divisor of Hkv <= nw that keeps most waves busy
  int hh = 1;
  for (int c = 1; c <= nw; ++c)
    if (Hkv % c == 0 && c * (nw / c) >= hh * (nw / hh)) hh = c;
  p->nw = nw;
  p->heads_per_wg = hh;
  p->waves_per_head = nw / hh;
  p->head_groups = Hkv / hh;
  long R;
  if (num_splits > 0) {
    R = num_splits;
  } else {
    // sized by the bf16 instance for both storages, so one workspace query
    // serves both entry points
    const int waves = resident_waves(select_kernel(d, nw, false), nw);
    R = waves / Hkv;
  }
  R = ((R + p->waves_per_head - 1) / p->waves_per_head) * p->waves_per_head;
  if (R < 1) R = 1;
  p->ranges = (int)R;
  p->grid = p->head_groups * (long)(R / p->waves_per_head);
  const long first = kFirstWord + 2L * B;
  p->off_o = (first + 63) / 64 * 64;
  p->off_l = p->off_o + ((long)B + R) * Hq * d;
  p->workspace_bytes = (size_t)(p->off_l + ((long)B + R) * Hq) * 4;
  return true;
}

hipError_t launch_paged_decode(const DecodeArgs& a, const DecodePlan& p) {
  KParams k;
  k.num_pages = a.num_pages;
  k.B = a.B;
  k.Hq = a.Hq;
  k.Hkv = a.Hkv;
  k.G = a.Hq / a.Hkv;
  k.Hh = p.heads_per_wg;
  k.WPH = p.waves_per_head;
  k.ngroups = p.head_groups;
  k.max_pages = a.max_pages;
  k.R = p.ranges;
  k.c = a.scale * kLog2e * (a.kv_fp8 ? a.s_k : 1.f);
  k.sv = a.kv_fp8 ? a.s_v : 1.f;
  const __bf16* q = static_cast<const __bf16*>(a.q);
  const void* kp = a.k_pool;
  const void* vp = a.v_pool;
  const int32_t* bt = a.block_table;
  const int32_t* sl = a.seq_lens;
  int* wsi = static_cast<int*>(a.ws);
  float* ws_o = static_cast<float*>(a.ws) + p.off_o;
  float* ws_l = static_cast<float*>(a.ws) + p.off_l;
  __bf16* o = static_cast<__bf16*>(a.o);
  float* lse = a.lse;
  void* fn = select_kernel(a.d, p.nw, a.kv_fp8);
  void* args[] = {&k, &q, &kp, &vp, &bt, &sl, &wsi, &ws_o, &ws_l, &o, &lse};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p.grid),
                                 dim3((unsigned)(p.nw * 64)), args, 0,
                                 a.stream);
  if (e != hipSuccess) return e;
  const dim3 mgrid((unsigned)(a.B * a.Hq));
  // many pieces per request (more than 16 ranges a request, where it
  // measured faster: 3x for one request, even at 16, 6 % slower at 8):
  // the wide merge, whose workgroup spreads a request's pieces over eight
  // waves
  if ((long)p.ranges > 16L * a.B) {
    if (a.d == 128)
      hipLaunchKernelGGL((decode_merge_wide_kernel<128>), mgrid, dim3(512), 0,
                         a.stream, wsi, ws_o, ws_l, sl, a.max_pages, p.ranges,
                         a.Hq, a.B, o, lse);
    else
      hipLaunchKernelGGL((decode_merge_wide_kernel<64>), mgrid, dim3(512), 0,
                         a.stream, wsi, ws_o, ws_l, sl, a.max_pages, p.ranges,
                         a.Hq, a.B, o, lse);
    return hipGetLastError();
  }
  if (a.d == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), mgrid, dim3(64), 0,
                       a.stream, wsi, ws_o, ws_l, sl, a.max_pages, p.ranges,
                       a.Hq, a.B, o, lse);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), mgrid, dim3(64), 0,
                       a.stream, wsi, ws_o, ws_l, sl, a.max_pages, p.ranges,
                       a.Hq, a.B, o, lse);
  return hipGetLastError();
}

}  // namespace fa
