// fa_decode.hip - paged-KV-cache decode (one query token per request), gfx950.
//
// The cache of each request lives in 16-token pages mapped by a block table
// ([FA3-paged §3.2]). The work of one request and one KV head is cut into
// chunks of `pages_per_split` pages; every chunk is a workgroup that
// streams its pages once from HBM (this kernel is bandwidth bound: every
// K/V byte is used once, by the Hq/Hkv query heads of the group together)
// and produces a normalised partial output and its log-sum-exp. A second
// small kernel merges the partials with the log-sum-exp form of the
// two-block merge ([Capstone §2.2 step 4], appendix A Q1).
//
// Per wave and page (16 tokens, one KV head: 16 rows of d bf16 at a
// stride of Hkv*d):
//   * S^T[token, head] = K . Q^T on v_mfma_f32_16x16x32_bf16, with K
//     fragments loaded straight from HBM into the A operand (lane: token
//     l%16, 16 B of d) and the group's query heads as the B operand
//     (lane: head l%16; heads past the group are zero);
//   * online softmax per head (column): lane-local over 4 tokens, then two
//     cross-row steps;
//   * O[head, d] += P V on the VALU: a lane owns 4 tokens and D/16 d
//     columns, P is broadcast inside each 16-lane row with DPP
//     row_newbcast, V is read 16 B per lane from HBM.
// Pages are assigned round-robin to the 4 waves; the next page's K and V
// loads are issued before the current page is computed. The waves' states
// are merged through LDS at the end of the chunk.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kPage = 16;
constexpr int kThreads = 256;
constexpr int kMaxPps = 256;  // pages per split held in LDS

// Lane n of every 16-lane row, broadcast to the whole row (DPP
// row_newbcast): P of head n for the four tokens this row holds.
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      0, __float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}
// o[g][:] += P[token, g] * v[:] for g < G (compile-time unrolled so the
// DPP lane selector is a constant).
template <int G, int GP, int DL>
struct PvAccumulate {
  static __device__ __forceinline__ void run(float (&o)[GP][DL], float p,
                                             const float (&vf)[DL]) {
    PvAccumulate<G - 1, GP, DL>::run(o, p, vf);
    const float pg = row_bcast<G - 1>(p);
#pragma unroll
    for (int e = 0; e < DL; ++e) o[G - 1][e] = __builtin_fmaf(pg, vf[e], o[G - 1][e]);
  }
};
template <int GP, int DL>
struct PvAccumulate<0, GP, DL> {
  static __device__ __forceinline__ void run(float (&)[GP][DL], float,
                                             const float (&)[DL]) {}
};

template <int D, int GP>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const __bf16* __restrict__ Qp, const __bf16* __restrict__ KP,
    const __bf16* __restrict__ VP, const int32_t* __restrict__ BT,
    const int32_t* __restrict__ SL, int num_pages, int Hq, int Hkv,
    int max_pages, int pps, int nsplit, float c, float* __restrict__ ws,
    __bf16* __restrict__ O, float* __restrict__ LSE, int B) {
  constexpr int DL = D / 16;  // d columns per lane in the PV step
  const int G = Hq / Hkv;
  // kv heads fastest: the workgroups that read the head slices of the same
  // pages are dispatched together, so each page (all heads of 16 tokens,
  // contiguous in the pool) is streamed from HBM in one pass
  const int hkv = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int split = rest % nsplit;
  const int b = rest / nsplit;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int row16 = lane >> 4;
  const int col = lane & 15;

  int L = SL[b];
  L = max(0, min(L, max_pages * kPage));
  const int npg = (L + kPage - 1) / kPage;
  const int p0 = split * pps;
  const int p1 = min(p0 + pps, npg);
  if (nsplit > 1 && p0 >= p1) return;  // no pages: the merge skips it

  __shared__ int pid[kMaxPps];
  __shared__ int bad;
  __shared__ float red_m[4][GP];
  __shared__ float red_l[4][GP];
  __shared__ __attribute__((aligned(16))) float red_o[4][GP][D];
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int i = tid; i < p1 - p0; i += kThreads) {
    int id = BT[(long)b * max_pages + p0 + i];
    if (id < 0 || id >= num_pages) {
      bad = 1;  // never dereferenced; the request's output becomes NaN
      id = 0;
    }
    pid[i] = id;
  }
  __syncthreads();

  // query heads of the group as the B operand: head col, d = 32s + 8*row16
  bf16x8 qf[D / 32];
  {
    const bool qv = col < G;
    const __bf16* qrow = Qp + ((long)b * Hq + (long)hkv * G + (qv ? col : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 32 * s + 8 * row16);
      if (!qv) x = bf16x8{};
      qf[s] = x;
    }
  }

  const long tok_stride = (long)Hkv * D;  // elements between tokens
  float m = kNegInf;                       // reference of head `col`
  float lp = 0.f;                          // partial sum: head col, 4 tokens
  float o[GP][DL];
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < DL; ++e) o[g][e] = 0.f;

  typedef uint32_t vload_t __attribute__((ext_vector_type(DL / 2)));
  bf16x8 kf[D / 32], kn[D / 32];
  vload_t vv[4], vn[4];
  auto load_page = [&](int p, bf16x8 (&kd)[D / 32], vload_t (&vd)[4]) {
    const long base = ((long)pid[p - p0] * kPage * Hkv + hkv) * D;
    const __bf16* kp = KP + base + (long)col * tok_stride + 8 * row16;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      kd[s] = *reinterpret_cast<const bf16x8*>(kp + 32 * s);
    const __bf16* vp = VP + base + (long)(4 * row16) * tok_stride + DL * col;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vd[r] = *reinterpret_cast<const vload_t*>(vp + r * tok_stride);
  };

  int p = p0 + w;
  if (p < p1) load_page(p, kn, vn);
  for (; p < p1; p += 4) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) kf[s] = kn[s];
#pragma unroll
    for (int r = 0; r < 4; ++r) vv[r] = vn[r];
    if (p + 4 < p1) load_page(p + 4, kn, vn);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) acc = mfma_16x16x32_bf16(kf[s], qf[s], acc);
    // lane: tokens 4*row16 + v of this page, head col
    const int tok0 = p * kPage + 4 * row16;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (tok0 + v >= L) acc[v] = kNegInf;
    float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float mxs = mx * c;
    const bool need = (col < G) && (mxs > m + kTau);
    if (__any(need)) {
      const float mnew = fmaxf(m, mxs);
      const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - mnew);
      lp *= alpha;
      m = mnew;
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float ag = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(alpha), g));
#pragma unroll
        for (int e = 0; e < DL; ++e) o[g][e] *= ag;
      }
    }
    const float mref = (m == kNegInf) ? 0.f : m;
    float pr[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pr[v] = fast_exp2(__builtin_fmaf(acc[v], c, -mref));
      lp += pr[v];
    }
    // O[g, d] += sum over this lane's 4 tokens of P[token, g] * V[token, d]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float vf[DL];
#pragma unroll
      for (int e = 0; e < DL / 2; ++e) {
        vf[2 * e] = bf16_lo(vv[r][e]);
        vf[2 * e + 1] = bf16_hi(vv[r][e]);
      }
      PvAccumulate<GP, GP, DL>::run(o, pr[r], vf);
    }
  }

  // ---- reduce the four 16-lane rows, then the four waves through LDS
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < DL; ++e) {
      float x = o[g][e];
      x += xor_lane(x, 16);
      x += xor_lane(x, 32);
      o[g][e] = x;
    }
  lp += xor_lane(lp, 16);
  lp += xor_lane(lp, 32);
  if (row16 == 0) {
    if (col < GP) {
      red_m[w][col] = m;
      red_l[w][col] = lp;
    }
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < DL; ++e) red_o[w][g][DL * col + e] = o[g][e];
  }
  __syncthreads();

  const bool poisoned = bad != 0;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx - g * D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, red_m[ww][g]);
    float os = 0.f, ls = kNegInf;
    if (M != kNegInf) {
      float wl = 0.f, wo = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float f = fast_exp2(red_m[ww][g] - M);
        wl += f * red_l[ww][g];
        wo += f * red_o[ww][g][d];
      }
      os = wo / wl;
      ls = (M + fast_log2(wl)) * kLn2;
    }
    if (poisoned) {
      os = __builtin_nanf("");
      ls = __builtin_nanf("");
    }
    const long hq = (long)b * Hq + (long)hkv * G + g;
    if (nsplit > 1) {
      ws[(hq * nsplit + split) * D + d] = os;
      if (d == 0) ws[(long)B * Hq * nsplit * D + hq * nsplit + split] = ls;
    } else {
      O[hq * D + d] = (__bf16)os;
      if (d == 0 && LSE != nullptr) LSE[hq] = ls;
    }
  }
}

// One workgroup per (request, query head): merge the live splits.
template <int D>
__global__ __launch_bounds__(128) void decode_merge_kernel(
    const float* __restrict__ ws, const int32_t* __restrict__ SL,
    int max_pages, int pps, int nsplit, int Hq, int B,
    __bf16* __restrict__ O, float* __restrict__ LSE) {
  const int hq = blockIdx.x;  // b * Hq + h
  const int b = hq / Hq;
  int L = SL[b];
  L = max(0, min(L, max_pages * kPage));
  const int npg = (L + kPage - 1) / kPage;
  const int ns = (npg + pps - 1) / pps;
  const float* lse_p = ws + (long)B * Hq * nsplit * D + (long)hq * nsplit;
  const float* o_p = ws + (long)hq * nsplit * D;
  float M = kNegInf;
  bool nan = false;
  for (int s = 0; s < ns; ++s) {
    const float x = lse_p[s];
    nan |= (x != x);
    M = fmaxf(M, x);
  }
  const int d = threadIdx.x;
  float od = 0.f, L_out = kNegInf;
  if (M != kNegInf) {
    float tot = 0.f, acc = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float f = fast_exp2((lse_p[s] - M) * kLog2e);
      tot += f;
      if (d < D) acc += f * o_p[(long)s * D + d];
    }
    od = acc / tot;
    L_out = M + fast_log2(tot) * kLn2;
  }
  if (nan) {
    od = __builtin_nanf("");
    L_out = __builtin_nanf("");
  }
  if (d < D) O[(long)hq * D + d] = (__bf16)od;
  if (d == 0 && LSE != nullptr) LSE[hq] = L_out;
}

template <int D, int GP>
hipError_t launch_split(const DecodeArgs& a) {
  const long blocks = (long)a.B * a.Hkv * a.num_splits;
  hipLaunchKernelGGL((decode_split_kernel<D, GP>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, a.stream,
                     static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k_pool),
                     static_cast<const __bf16*>(a.v_pool), a.block_table,
                     a.seq_lens, a.num_pages, a.Hq, a.Hkv, a.max_pages,
                     a.pages_per_split, a.num_splits, a.scale * kLog2e, a.ws,
                     static_cast<__bf16*>(a.o), a.lse, a.B);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  hipError_t e;
  if (G <= 1) e = launch_split<D, 1>(a);
  else if (G <= 2) e = launch_split<D, 2>(a);
  else if (G <= 4) e = launch_split<D, 4>(a);
  else if (G <= 8) e = launch_split<D, 8>(a);
  else e = launch_split<D, 16>(a);
  if (e != hipSuccess || a.num_splits == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(a.B * a.Hq)),
                     dim3(128), 0, a.stream, a.ws, a.seq_lens, a.max_pages,
                     a.pages_per_split, a.num_splits, a.Hq, a.B,
                     static_cast<__bf16*>(a.o), a.lse);
  return hipGetLastError();
}

}  // namespace

bool plan_decode(int B, int Hq, int Hkv, int d, int max_pages, int num_splits,
                 DecodePlan* plan) {
  int pps;
  if (num_splits > 0) {
    pps = (max_pages + num_splits - 1) / num_splits;
    if (pps > kMaxPps) return false;
  } else {
    // Enough workgroups to keep every CU streaming (>= 8192 chunks incl.
    // the empty tails of short requests), pages per chunk a power of two.
    pps = 4;
    for (int cand = 64; cand >= 4; cand >>= 1) {
      const long units = (long)B * Hkv * ((max_pages + cand - 1) / cand);
      if (units >= 8192) {
        pps = cand;
        break;
      }
    }
  }
  if (pps < 1) pps = 1;
  if (pps > max_pages) pps = max_pages;
  const int ns = (max_pages + pps - 1) / pps;
  plan->pages_per_split = pps;
  plan->num_splits = ns;
  plan->workspace_bytes =
      ns > 1 ? (size_t)B * Hq * ns * ((size_t)d + 1) * sizeof(float) : 0;
  return true;
}

hipError_t launch_paged_decode(const DecodeArgs& a) {
  if (a.d == 128) return launch_d<128>(a);
  return launch_d<64>(a);
}

}  // namespace fa
