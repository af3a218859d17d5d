// fa_fwd_bf16.hip - exact attention forward, bf16 in / bf16 out, gfx950.
//
// One workgroup (4 waves) owns a 128-row query tile of one (batch, head)
// and streams the key/value range in 64-key tiles: the Q-outer / KV-inner
// order of [Capstone §4.1] with O, m, l held on chip and O divided by l
// once at the end ([Capstone §4.2]). Q K^T and P V run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; S and P never leave
// registers. Causal tiles above the diagonal are not visited
// ([Capstone §7.3 Q2]); the tiles that cross it are masked per element.
//
// Data flow per key tile (double-buffered LDS, one barrier per tile):
//   global K, V (16 B per lane, coalesced 256 B rows) -> VGPRs (prefetched
//   one tile ahead, overlapping the MFMA work of the current tile)
//   -> LDS: K row-major with an XOR swizzle of its 16 B chunks;
//           V transposed to V^T (d-major) so the PV operand is a single
//           16 B read, also XOR-swizzled.
//   -> per wave: S^T = K Q^T (Q lives in VGPRs for the whole tile),
//      online softmax, P^T packed to bf16 in registers, O^T += V^T P^T.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kBM = 128;       // query rows per workgroup (32 per wave)
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 waves

template <int D>
struct Bf16Tile {
  static constexpr int CPR = D / 8;                        // 16 B chunks/row
  static constexpr int K_BYTES = kBN * D * 2;              // K tile
  static constexpr int VT_ROW = kBN * 2;                   // V^T row bytes
  static constexpr int VT_BYTES = D * VT_ROW;              // V^T tile
  static constexpr int STAGE = K_BYTES + VT_BYTES;
  static constexpr int KLOADS = kBN * CPR / kThreads;      // 16 B per lane
  static constexpr int VUNITS = (kBN / 4) * CPR;           // 4 keys x 8 d
};

// Physical 16 B chunk of K row `key` that holds logical chunk c: 16
// consecutive keys reading one logical chunk, and 16 lanes writing one
// row, both hit 16 distinct 16 B bank groups.
template <int D>
__device__ __forceinline__ int k_chunk(int key, int c) {
  if constexpr (D == 128) return c ^ (key & 15);
  else return c ^ ((key >> 1) & 7);
}
// V^T row d holds 64 keys (8 chunks of 16 B). Reads (16 consecutive d, one
// chunk) are conflict free; the transposing writes see at most 4-way.
__device__ __forceinline__ int vt_chunk(int d, int c) {
  return c ^ (((d >> 1) ^ (d >> 4)) & 7);
}
// Inside a V^T row, key k of the tile is stored at position pi(k) = k with
// bits 2 and 3 swapped: the 8 keys one MFMA lane needs for the PV step
// (4h + {0..3} and 8 + 4h + {0..3} within a 16-key step) become one 16 B
// chunk, ordered like the P^T operand taken from the S^T accumulator.

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, __bf16* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk,
    float c) {
  using T = Bf16Tile<D>;
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
  const int off = Nk - Nq;  // bottom-right causal alignment
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(q0 + kBM, Nq) + off);
  const int nt = kend > 0 ? (kend + kBN - 1) / kBN : 0;

  // Q fragments (B operand of S^T = K Q^T): row r32 of this wave's 32
  // rows, d = 16*s + 8*h + t.
  const int wrow0 = q0 + w * 32;
  const int row = wrow0 + r32;
  const int rowc = min(row, Nq - 1);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(Q + qbase + (long)rowc * D +
                                             16 * s + 8 * h);

  f32x16 o[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[mb][v] = 0.f;
  RowState st{kNegInf, 0.f, 0.f};

  // ---- register staging of one K/V tile
  u32x4 kr[T::KLOADS];
  u32x4 vr[4];
  const int vkg = tid / T::CPR;  // 4-key group of this lane's V unit
  const int vdc = tid % T::CPR;  // 8-element d chunk of this lane's V unit
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < T::KLOADS; ++i) {
      const int u = tid + kThreads * i;
      const int key = u / T::CPR, cc = u % T::CPR;
      const int gk = n0 + key;
      u32x4 z = {0u, 0u, 0u, 0u};
      kr[i] = gk < Nk ? *reinterpret_cast<const u32x4*>(K + kvbase +
                                                        (long)gk * D + 8 * cc)
                      : z;
    }
    if (tid < T::VUNITS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gk = n0 + 4 * vkg + r;
        u32x4 z = {0u, 0u, 0u, 0u};
        vr[r] = gk < Nk ? *reinterpret_cast<const u32x4*>(
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
      *reinterpret_cast<u32x4*>(ks + key * (D * 2) + k_chunk<D>(key, cc) * 16) =
          kr[i];
    }
    if (tid < T::VUNITS) {
      // keys 4*vkg .. +3 sit at V^T positions pi(4*vkg) .. +3
      const int cpos = 2 * (vkg >> 2) + (vkg & 1);
      const int half = (vkg >> 1) & 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * vdc + e;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 pr;
        pr[0] = __builtin_amdgcn_perm(vr[1][e >> 1], vr[0][e >> 1], sel);
        pr[1] = __builtin_amdgcn_perm(vr[3][e >> 1], vr[2][e >> 1], sel);
        *reinterpret_cast<u32x2*>(vs + d * T::VT_ROW + vt_chunk(d, cpos) * 16 +
                                  half * 8) = pr;
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
      // S^T = K Q^T for two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
        const int key = 32 * kb + r32;
#pragma unroll
        for (int sd = 0; sd < D / 16; ++sd) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              ks + key * (D * 2) + k_chunk<D>(key, 2 * sd + h) * 16);
          s[kb] = mfma_32x32x16_bf16(a, qf[sd], s[kb]);
        }
      }
      // mask the ragged end of the key range and the causal diagonal
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
      // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t pw[4];
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) {
            pw[t2] = pack_bf16x2(s[kb][8 * j + 2 * t2], s[kb][8 * j + 2 * t2 + 1]);
            st.lr = add_bf16x2(pw[t2], st.lr);
          }
          u32x4 pv = {pw[0], pw[1], pw[2], pw[3]};
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pv);
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb) {
            const int dd = 32 * mb + r32;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                vs + dd * T::VT_ROW + vt_chunk(dd, 4 * kb + 2 * j + h) * 16);
            o[mb] = mfma_32x32x16_bf16(a, pb, o[mb]);
          }
        }
    }
    if (has_next) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / lr, LSE = ln 2 * (m + log2 l)
  const float ltot = st.l + xor_lane(st.l, 32);
  const float lrtot = st.lr + xor_lane(st.lr, 32);
  if (row < Nq) {
    const bool live = ltot > 0.f;
    const float inv = live ? 1.f / lrtot : 0.f;
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
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, a.stream,
                     static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v),
                     static_cast<__bf16*>(a.o), a.lse, a.B, a.Hq, a.Hkv, a.Nq,
                     a.Nk, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

}  // namespace fa
