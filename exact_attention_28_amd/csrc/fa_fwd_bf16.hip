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
//   global K, V (16 B per lane) -> VGPRs (prefetched one tile ahead,
//   overlapping the MFMA work of the current tile) -> LDS, both row-major
//   with padded rows
//   -> per wave: S^T = K Q^T (Q lives in VGPRs for the whole tile),
//      online softmax, P^T packed to bf16 in registers, O^T += V^T P^T with
//      the V^T operand produced by gfx950's LDS transpose read.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kBM = 128;       // query rows per workgroup (32 per wave)
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 waves

template <int D>
struct Bf16Tile {
  static constexpr int CPR = D / 8;                   // 16 B chunks per row
  static constexpr int K_ROW = D * 2 + 16;            // padded K row
  static constexpr int V_ROW = D * 2 + 64;            // padded V row
  static constexpr int K_BYTES = kBN * K_ROW;
  static constexpr int V_BYTES = kBN * V_ROW;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int LOADS = kBN * CPR / kThreads;  // 16 B per lane, each of K, V
  static constexpr int ROWS_PER_LOAD = kThreads / CPR;
};

// LDS layouts (both row-major, rows padded so every fragment address is a
// per-lane base plus a compile-time offset, and no access conflicts):
//  * K rows padded by 16 B (stride = 17 groups of 16 B): the S^T = K Q^T
//    A operand is one 16 B read per lane, 16 consecutive keys at one
//    chunk -> 16 distinct bank groups.
//  * V rows padded by 64 B (stride = 16 mod 64 banks): the O^T = V^T P^T A
//    operand is read with ds_read_b64_tr_b16. In each 16-lane group, lane j
//    fetches 4 consecutive d of key row kbase + j/4 and the transpose hands
//    lane i the 4 keys kbase..kbase+3 at column dbase + i -- the k-major
//    V^T fragment the MFMA needs. A 32-lane half reads 4 rows x 64 B, which
//    the stride spreads over all 64 banks.
//  * Writes: 16 lanes store one 256 B row (D = 128) or two 128 B rows.

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
  const __bf16* Kh = K + (long)(ti.b * Hkv + hk) * Nk * D;
  const __bf16* Vh = V + (long)(ti.b * Hkv + hk) * Nk * D;
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

  // ---- K/V tile staging. Lane tid moves chunk (tid % CPR) of rows
  // tid / CPR + ROWS_PER_LOAD * i. Full tiles use a uniform base plus a
  // loop-invariant lane offset; on the ragged last tile rows past Nk are
  // clamped to the last key (their scores are masked, their P is 0).
  const int lrow = tid / T::CPR;
  const int lcol = (tid % T::CPR) * 8;
  u32x4 kr[T::LOADS], vr[T::LOADS];
  auto load_tile = [&](int n0) {
    const __bf16* kt = Kh + (long)n0 * D;
    const __bf16* vt = Vh + (long)n0 * D;
    if (n0 + kBN <= Nk) {
#pragma unroll
      for (int i = 0; i < T::LOADS; ++i) {
        const int o_ = (lrow + T::ROWS_PER_LOAD * i) * D + lcol;
        kr[i] = *reinterpret_cast<const u32x4*>(kt + o_);
        vr[i] = *reinterpret_cast<const u32x4*>(vt + o_);
      }
    } else {
      const int last = Nk - 1 - n0;
#pragma unroll
      for (int i = 0; i < T::LOADS; ++i) {
        const int o_ = min(lrow + T::ROWS_PER_LOAD * i, last) * D + lcol;
        kr[i] = *reinterpret_cast<const u32x4*>(kt + o_);
        vr[i] = *reinterpret_cast<const u32x4*>(vt + o_);
      }
    }
  };
  auto store_tile = [&](int stage) {
    char* ks = smem + stage * T::STAGE + lrow * T::K_ROW + lcol * 2;
    char* vs = smem + stage * T::STAGE + T::K_BYTES + lrow * T::V_ROW + lcol * 2;
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      *reinterpret_cast<u32x4*>(ks + i * T::ROWS_PER_LOAD * T::K_ROW) = kr[i];
      *reinterpret_cast<u32x4*>(vs + i * T::ROWS_PER_LOAD * T::V_ROW) = vr[i];
    }
  };

  // per-lane LDS bases of the fragment reads
  const int kfrag = (32 * 0 + r32) * T::K_ROW + 16 * h;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int vfrag = (4 * h + (i16 >> 2)) * T::V_ROW + (16 * (g16 & 1) + 4 * (i16 & 3)) * 2;

  if (nt > 0) {
    load_tile(0);
    store_tile(0);
  }
  // Everything loaded so far (Q fragments, first tile) has landed: inside
  // the loop the only outstanding global loads are the next tile's, which
  // nothing reads until it is stored.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int n0 = t * kBN;
    const bool has_next = t + 1 < nt;
    if (has_next) load_tile(n0 + kBN);
    const bool skip = CAUSAL && (n0 > wrow0 + 31 + off);
    if (!skip) {
      const char* ks = smem + (t & 1) * T::STAGE + kfrag;
      const char* vs = smem + (t & 1) * T::STAGE + T::K_BYTES + vfrag;
      // S^T = K Q^T for two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
        for (int sd = 0; sd < D / 16; ++sd) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              ks + 32 * kb * T::K_ROW + 32 * sd);
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
      // O^T += V^T P^T, 16 keys per MFMA: lane half h contracts keys
      // 32kb + 16j + 4h + {0..3} (items 0..3) and +8 (items 4..7)
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
            const char* vp = vs + (32 * kb + 16 * j) * T::V_ROW + 64 * mb;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(vp));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(vp + 8 * T::V_ROW));
            const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[mb] = mfma_32x32x16_bf16(a, pb, o[mb]);
          }
        }
    }
    if (has_next) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / lr, LSE = ln 2 * (m + log2 l)
  const float ltot = sum_halves(st.l);
  const float lrtot = sum_halves(st.lr);
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
