// fa_fwd_f32.hip - exact attention forward, fp32 in / fp32 out, gfx950.
//
// Same algorithm and register layout as the bf16 kernel (Q-outer tiles of
// 128 rows, 4 waves x 32 rows, online softmax with deferred 1/l,
// [Capstone §4.1-4.2]) on v_mfma_f32_32x32x2f32, so products and sums are
// fp32 throughout. 32-key tiles, single-buffered LDS: this path exists for
// full-precision parity, not for throughput.
//
// MFMA operand split of the head dimension: lane half h = l/32 contracts
// d in [h*D/2, (h+1)*D/2), one element per step, for both K and Q.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 32;
constexpr int kThreads = 256;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K,
    const float* __restrict__ V, float* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk,
    float c) {
  // K rows padded by one word: 32 lanes reading one column of 32 rows hit
  // 32 banks. V rows padded by 8 words: the two lane halves read rows four
  // apart, which then land 32 banks apart.
  __shared__ float ks[kBN][D + 1];
  __shared__ __attribute__((aligned(16))) float vs[kBN][D + 8];

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
  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; s += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(
        Q + qbase + (long)rowc * D + h * (D / 2) + s);
    qf[s] = x[0];
    qf[s + 1] = x[1];
    qf[s + 2] = x[2];
    qf[s + 3] = x[3];
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[mb][v] = 0.f;
  RowState st{kNegInf, 0.f, 0.f};  // fp32 P.V: lr unused (equals l)

  constexpr int C4 = D / 4;  // float4 chunks per row
  for (int t = 0; t < nt; ++t) {
    const int n0 = t * kBN;
    __syncthreads();  // previous tile fully consumed
    for (int u = tid; u < kBN * C4; u += kThreads) {
      const int key = u / C4, cc = u % C4;
      const int gk = n0 + key;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (gk < Nk) {
        kx = *reinterpret_cast<const f32x4*>(K + kvbase + (long)gk * D + 4 * cc);
        vx = *reinterpret_cast<const f32x4*>(V + kvbase + (long)gk * D + 4 * cc);
      }
      ks[key][4 * cc] = kx[0];
      ks[key][4 * cc + 1] = kx[1];
      ks[key][4 * cc + 2] = kx[2];
      ks[key][4 * cc + 3] = kx[3];
      *reinterpret_cast<f32x4*>(&vs[key][4 * cc]) = vx;
    }
    __syncthreads();
    if (CAUSAL && n0 > wrow0 + 31 + off) continue;

    f32x16 s[1];
#pragma unroll
    for (int v = 0; v < 16; ++v) s[0][v] = 0.f;
#pragma unroll
    for (int sd = 0; sd < D / 2; ++sd)
      s[0] = mfma_32x32x2_f32(ks[r32][h * (D / 2) + sd], qf[sd], s[0]);

    const bool need_mask =
        (n0 + kBN > Nk) || (CAUSAL && n0 + kBN - 1 > wrow0 + off);
    if (need_mask) {
      const int lim = CAUSAL ? min(Nk - 1, row + off) : Nk - 1;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = n0 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (key > lim) s[0][v] = kNegInf;
      }
    }
    online_softmax_tile<1, D / 32>(s, o, st, c);
    // O^T += V^T P^T: step v contracts key 8(v/4) + 4h + v%4 in lane half h
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = 8 * (v >> 2) + 4 * h + (v & 3);
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
        o[mb] = mfma_32x32x2_f32(vs[key][32 * mb + r32], s[0][v], o[mb]);
    }
  }

  const float ltot = st.l + xor_lane(st.l, 32);
  if (row < Nq) {
    const bool live = ltot > 0.f;
    const float inv = live ? 1.f / ltot : 0.f;
    float* orow = O + qbase + (long)row * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {o[mb][4 * g] * inv, o[mb][4 * g + 1] * inv,
                   o[mb][4 * g + 2] * inv, o[mb][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + 32 * mb + 8 * g + 4 * h) = x;
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
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, a.stream,
                     static_cast<const float*>(a.q),
                     static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o),
                     a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

}  // namespace fa
