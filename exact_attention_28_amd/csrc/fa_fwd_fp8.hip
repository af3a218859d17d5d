// fa_fwd_fp8.hip - exact attention forward on OCP e4m3 inputs, gfx950.
//
// The fp8 recipe of the [FA3-guide] fp8 listing: Q, K, V as e4m3, Q K^T
// and P V as fp8 products with fp32 accumulation, the softmax in fp32, P
// rounded to e4m3 before the second product, output in bf16 (instead of
// the listing's fp16). Inputs carry per-tensor fp32 scales s_q, s_k, s_v:
// s_q*s_k is folded with scale*log2(e) into the single multiply that turns
// raw scores into exp2 arguments, and s_v into the final 1/l.
// P is the unnormalised exp2(s - m_ref) <= 2^kTau = 256 < 448, so it fits
// e4m3 without a scale. O is normalised by the sum of the rounded P (an
// exact convex combination of V rows), LSE uses the sum of the fp32 P.
//
// Structure as the bf16 kernel (128-row Q tile, 64-key K/V tiles,
// double-buffered swizzled LDS, S^T / O^T register layout) on
// v_mfma_f32_32x32x64_f8f6f4: one MFMA contracts 64 elements, so Q K^T
// takes D/64 steps per 32-key block and one P V step covers the whole
// 64-key tile.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;

template <int D>
struct Fp8Tile {
  static constexpr int CPR = D / 16;                    // 16 B chunks / K row
  static constexpr int K_BYTES = kBN * D;
  static constexpr int VT_ROW = kBN;                    // 64 keys, 4 chunks
  static constexpr int VT_BYTES = D * VT_ROW;
  static constexpr int STAGE = K_BYTES + VT_BYTES;
  static constexpr int KLOADS = kBN * CPR / kThreads;   // 2 (D=128), 1 (D=64)
  static constexpr int VUNITS = (kBN / 4) * (D / 8);    // 4 keys x 8 d
};

template <int D>
__device__ __forceinline__ int k_chunk(int key, int c) {
  if constexpr (D == 128) return c ^ ((key >> 1) & 7);   // 2 rows / 256 B
  else return c ^ ((key >> 2) & 3);                      // 4 rows / 256 B
}
__device__ __forceinline__ int vt_chunk(int d, int c) {
  return c ^ ((d >> 2) & 3);  // 4 V^T rows per 256 B
}
// Position of key k of the tile inside a V^T row: with k = 32*kb + 8*g +
// 4*h + r, pos = 32*h + 16*kb + 4*g + r, so MFMA lane half h reads its 32
// keys as one contiguous 32 B run in the order of the S^T accumulator
// elements (block kb, element 4g + r).

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
    const uint8_t* __restrict__ V, __bf16* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk, float c,
    float s_v) {
  using T = Fp8Tile<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int r32 = lane & 31;

  const int n_qt = (Nq + kBM - 1) / kBM;
  const TileIdx ti = map_tile(blockIdx.x, n_qt, Hq, Hkv, B, CAUSAL);
  const int hk = ti.hq / (Hq / Hkv);
  const int q0 = ti.qt * kBM;
  const long qbase = (long)(ti.b * Hq + ti.hq) * Nq * D;
  const long kvbase = (long)(ti.b * Hkv + hk) * Nk * D;
  const int off = Nk - Nq;
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(q0 + kBM, Nq) + off);
  const int nt = kend > 0 ? (kend + kBN - 1) / kBN : 0;

  const int wrow0 = q0 + w * 32;
  const int row = wrow0 + r32;
  const int rowc = min(row, Nq - 1);
  // Q fragments: row r32, d = 64*s + 32*h + t (t = 0..31)
  i32x8 qf[D / 64];
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    const u32x4* p = reinterpret_cast<const u32x4*>(Q + qbase + (long)rowc * D +
                                                    64 * s + 32 * h);
    const u32x4 x0 = p[0], x1 = p[1];
    qf[s] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                  (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[mb][v] = 0.f;
  RowState st{kNegInf, 0.f, 0.f};

  u32x4 kr[T::KLOADS];
  u32x2 vr[4];
  constexpr int VDC = D / 8;
  const int vkg = tid / VDC, vdc = tid % VDC;
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < T::KLOADS; ++i) {
      const int u = tid + kThreads * i;
      const int key = u / T::CPR, cc = u % T::CPR;
      const int gk = n0 + key;
      u32x4 z = {0u, 0u, 0u, 0u};
      kr[i] = gk < Nk ? *reinterpret_cast<const u32x4*>(K + kvbase +
                                                        (long)gk * D + 16 * cc)
                      : z;
    }
    if (tid < T::VUNITS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gk = n0 + 4 * vkg + r;
        u32x2 z = {0u, 0u};
        vr[r] = gk < Nk ? *reinterpret_cast<const u32x2*>(
                              V + kvbase + (long)gk * D + 8 * vdc)
                        : z;
      }
    }
  };
  auto store_tile = [&](int stage) {
    char* ks = smem + stage * T::STAGE;
    char* vs = ks + T::K_BYTES;
#pragma unroll
    for (int i = 0; i < T::KLOADS; ++i) {
      const int u = tid + kThreads * i;
      const int key = u / T::CPR, cc = u % T::CPR;
      *reinterpret_cast<u32x4*>(ks + key * D + k_chunk<D>(key, cc) * 16) = kr[i];
    }
    if (tid < T::VUNITS) {
      const int cpos = 2 * (vkg & 1) + (vkg >> 3);
      const int dw = (vkg >> 1) & 3;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * vdc + e;
        const int b = e & 3;
        const uint32_t w0 = vr[0][e >> 2], w1 = vr[1][e >> 2];
        const uint32_t w2 = vr[2][e >> 2], w3 = vr[3][e >> 2];
        // byte b of keys 0..3 -> bytes 0..3 of one word
        const uint32_t sel = (uint32_t)b | ((uint32_t)(b + 4) << 8);
        const uint32_t lo = __builtin_amdgcn_perm(w1, w0, sel);   // k0, k1
        const uint32_t hi = __builtin_amdgcn_perm(w3, w2, sel);   // k2, k3
        const uint32_t word = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        *reinterpret_cast<uint32_t*>(vs + d * T::VT_ROW +
                                     vt_chunk(d, cpos) * 16 + dw * 4) = word;
      }
    }
  };

  if (nt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int n0 = t * kBN;
    const bool has_next = t + 1 < nt;
    if (has_next) load_tile(n0 + kBN);
    const bool skip = CAUSAL && (n0 > wrow0 + 31 + off);
    if (!skip) {
      const char* ks = smem + (t & 1) * T::STAGE;
      const char* vs = ks + T::K_BYTES;
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
        const int key = 32 * kb + r32;
#pragma unroll
        for (int sd = 0; sd < D / 64; ++sd) {
          const int c0 = 4 * sd + 2 * h;
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(
              ks + key * D + k_chunk<D>(key, c0) * 16);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(
              ks + key * D + k_chunk<D>(key, c0 + 1) * 16);
          const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                           (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          s[kb] = mfma_32x32x64_e4m3(a, qf[sd], s[kb]);
        }
      }
      const bool need_mask =
          (n0 + kBN > Nk) || (CAUSAL && n0 + kBN - 1 > wrow0 + off);
      if (need_mask) {
        const int lim = CAUSAL ? min(Nk - 1, row + off) : Nk - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = n0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
            if (key > lim) s[kb][v] = kNegInf;
          }
      }
      online_softmax_tile<2, D / 32>(s, o, st, c);
      // P^T as e4m3: byte t = 16*kb + v of this lane's 32 keys
      i32x8 pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kb = j >> 2, v0 = 4 * (j & 3);
        const uint32_t w8 = pack_e4m3x4(s[kb][v0], s[kb][v0 + 1],
                                        s[kb][v0 + 2], s[kb][v0 + 3]);
        st.lr = add_e4m3x4(w8, st.lr);
        pb[j] = (int)w8;
      }
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
        const int dd = 32 * mb + r32;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(
            vs + dd * T::VT_ROW + vt_chunk(dd, 2 * h) * 16);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(
            vs + dd * T::VT_ROW + vt_chunk(dd, 2 * h + 1) * 16);
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                         (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        o[mb] = mfma_32x32x64_e4m3(a, pb, o[mb]);
      }
    }
    if (has_next) store_tile((t + 1) & 1);
    __syncthreads();
  }

  const float ltot = st.l + xor_lane(st.l, 32);
  const float lrtot = st.lr + xor_lane(st.lr, 32);
  if (row < Nq) {
    const bool live = ltot > 0.f;
    const float inv = live ? s_v / lrtot : 0.f;
    __bf16* orow = O + qbase + (long)row * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pr;
        pr[0] = pack_bf16x2(o[mb][4 * g] * inv, o[mb][4 * g + 1] * inv);
        pr[1] = pack_bf16x2(o[mb][4 * g + 2] * inv, o[mb][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * mb + 8 * g + 4 * h) = pr;
      }
    if (h == 0 && LSE != nullptr)
      LSE[(long)(ti.b * Hq + ti.hq) * Nq + row] =
          live ? (st.m + fast_log2(ltot)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long blocks = (long)n_qt * a.Hq * a.B;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, a.stream,
                     static_cast<const uint8_t*>(a.q),
                     static_cast<const uint8_t*>(a.k),
                     static_cast<const uint8_t*>(a.v),
                     static_cast<__bf16*>(a.o), a.lse, a.B, a.Hq, a.Hkv, a.Nq,
                     a.Nk, a.scale * kLog2e * a.s_q * a.s_k, a.s_v);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

}  // namespace fa
