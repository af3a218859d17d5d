// fa_fwd_fp8.hip - exact attention forward on OCP e4m3 inputs, gfx950.
//
// The fp8 recipe of the [FA3-guide] fp8 listing: Q, K, V as e4m3, Q K^T
// and P V as fp8 products with fp32 accumulation, the softmax in fp32, P
// rounded to e4m3 before the second product, output in bf16 (instead of
// the listing's fp16). Inputs carry per-tensor fp32 scales s_q, s_k, s_v:
// s_q*s_k is folded with scale*log2(e) into the single multiply that turns
// raw scores into exp2 arguments, and s_v into the final 1/l.
// P is the unnormalised exp2(s - m_ref), rounded to e4m3 without a scale:
// with the first pass's fixed reference it stays below 448 unless later
// scores rise about 2^9 above the first key tile (then its conversion gives
// NaN and the lazy second pass, P <= 2^kTau = 256, takes over). O is
// normalised by the sum of the rounded P (an exact convex combination of V
// rows), LSE uses the sum of the fp32 P.
//
// Structure as the bf16 kernel: one workgroup (4 waves, 32 rows each) per
// 128-row query tile, 64-key K/V tiles arriving by direct global->LDS loads
// into a double-buffered LDS stage, S^T / O^T register layout, tiles taken
// in pairs so that S(t+1) is computed while P(t) is formed. The products
// run on v_mfma_f32_32x32x64_f8f6f4: Q K^T takes D/64 steps per 32-key
// block, and one P V step covers the whole 64-key tile. The V^T operand
// comes from gfx950's 8-bit LDS transpose read. The sum of the rounded P
// comes from one more MFMA per tile against an all-ones operand: every
// output row of ones . P^T is the row sum of P, accumulated exactly. The
// ones are given as fp4 (e2m1), which takes four registers instead of eight.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;

// ------------------------------------------------------------ LDS layout
// A tile is 64 rows of D bytes, stored as 1 KB blocks (one direct load
// instruction: 64 lanes x 16 B) at a pitch of 1 KB + 16 B, so the 16-byte
// units of equal block-relative offset rotate through the sixteen 16-byte
// bank groups (256 bytes of banks) from block to block.
//  * K: block b holds rows b, b + NB, b + 2NB, ... The S^T = K Q^T A
//    operand (32 bytes per lane: key 32kb + r32, bytes 64sd + 32h ..) is
//    read as two 16-byte reads; the sixteen lanes served together hold
//    sixteen consecutive keys, which sit in eight blocks at two slots 128 B
//    apart (D = 128) or four blocks at four slots 64 B apart (D = 64):
//    conflict free.
//  * V: read with ds_read_b64_tr_b8, which in each 16-lane group takes
//    eight rows of 16 bytes (lane j names half j%2 of row j/2) and hands
//    lane i byte i of every row. One read gives a lane 8 keys of its d
//    column; the 8 keys of a read are k0..k0+3 and k0+8..k0+11 (the S^T
//    accumulator order), in eight different blocks at one slot:
//      D = 128: block (r%4) + 4((r/8)%2), slot (r/4)%2 + 2(r/16)
//      D = 64:  block r%4, slot 8((r/4)%2) + r/8
//    The two 16-lane groups of a 32-lane half read the same rows at the
//    column chunks 2m and 2m + 1, so those must sit 128 B apart: the rows
//    at slots s and s ^ S (S = 128 / D, the same block) trade pieces, and
//    chunk 2m + q of the row whose slot is s is stored at slot s ^ (q S),
//    16-byte position 2m + ((s / S) & 1) of that slot's row space.
template <int D>
struct Lay8 {
  static constexpr int RPB = 1024 / D;   // rows per 1 KB block
  static constexpr int NB = kBN / RPB;   // blocks per tile
  static constexpr int CPR = D / 16;     // 16-byte chunks per row
  static constexpr int PITCH = 1040;
  static constexpr int BYTES = NB * PITCH;
  static constexpr int BPW = NB / 4;     // blocks each wave loads
};
template <int D>
__device__ __forceinline__ int v_block(int r) {
  if constexpr (D == 128) return (r & 3) + 4 * ((r >> 3) & 1);
  else return r & 3;
}
template <int D>
__device__ __forceinline__ int v_slot(int r) {
  if constexpr (D == 128) return ((r >> 2) & 1) + 2 * (r >> 4);
  else return 8 * ((r >> 2) & 1) + (r >> 3);
}
// inverse: the row stored at (block, slot)
template <int D>
__device__ __forceinline__ int v_row(int b, int s) {
  if constexpr (D == 128) return 16 * (s >> 1) + 8 * (b >> 2) + 4 * (s & 1) + (b & 3);
  else return 8 * (s & 7) + 4 * (s >> 3) + b;
}


template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
    const uint8_t* __restrict__ V, __bf16* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk, float c,
    float s_v) {
  using T = Lay8<D>;
  __shared__ __attribute__((aligned(16))) char k_lds0[T::BYTES];
  __shared__ __attribute__((aligned(16))) char k_lds1[T::BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds0[T::BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds1[T::BYTES];
  auto kbuf = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)k_lds0;
    else return (lds_char*)k_lds1;
  };
  auto vbuf = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)v_lds0;
    else return (lds_char*)v_lds1;
  };

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
  const uint8_t* Kh = K + (long)(ti.b * Hkv + hk) * Nk * D;
  const uint8_t* Vh = V + (long)(ti.b * Hkv + hk) * Nk * D;
  const int off = Nk - Nq;
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(q0 + kBM, Nq) + off);
  const int nt = kend > 0 ? (kend + kBN - 1) / kBN : 0;

  const int wrow0 = q0 + w * 32;
  const int row = wrow0 + r32;
  const int rowc = min(row, Nq - 1);
  // Q fragments (B operand of S^T = K Q^T): row r32, d = 64*s + 32*h + t
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
  // row sums of the rounded P (every element holds this lane's row sum;
  // only element 0 is kept up to date under rescaling)
  f32x16 lsum;
#pragma unroll
  for (int v = 0; v < 16; ++v) lsum[v] = 0.f;
  RowState st{kNegInf, 0.f, 0.f};
  // e2m1 1.0 (0b0010) in every nibble; an fp4 operand uses dwords 0-3
  const i32x8 ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222,
                      0x22222222, 0x22222222, 0x22222222, 0x22222222};

  // ---- direct loads. Wave w fills blocks w, w+4, ...; lane l moves chunk
  // l % CPR of the block's slot l / CPR. On the ragged last tile rows past
  // Nk are clamped to the last key (their scores are masked, P is 0).
  const int slot = lane / T::CPR, chunk = lane % T::CPR;
  auto k_row = [&](int b) { return b + T::NB * slot; };
  auto issue_k = [&](int tile, auto buf) {
    const int n0 = tile * kBN;
    const uint8_t* src = Kh + (long)n0 * D + 16 * chunk;
    lds_char* dst = kbuf(buf) + w * T::PITCH;
    const int last = min(kBN, Nk - n0) - 1;
#pragma unroll
    for (int i = 0; i < T::BPW; ++i)
      g2lds_16B_own(src + (long)min(k_row(w + 4 * i), last) * D,
                dst + 4 * i * T::PITCH);
  };
  // V: the piece this lane moves (see the layout above)
  constexpr int kS = 128 / D;
  const int vq = ((slot / kS) & 1) ^ (chunk & 1);
  const int vslot = slot ^ (vq * kS);
  const int vchunk = 2 * (chunk >> 1) + vq;
  auto issue_v = [&](int tile, auto buf) {
    const int n0 = tile * kBN;
    const uint8_t* src = Vh + (long)n0 * D + 16 * vchunk;
    lds_char* dst = vbuf(buf) + w * T::PITCH;
    const int last = min(kBN, Nk - n0) - 1;
#pragma unroll
    for (int i = 0; i < T::BPW; ++i)
      g2lds_16B_own(src + (long)min(v_row<D>(w + 4 * i, vslot), last) * D,
                dst + 4 * i * T::PITCH);
  };

  // ---- per-lane fragment bases
  // K: row 32kb + r32 is in block r32 % NB (NB divides 32), slot
  // (32kb + r32) / NB; bytes 64sd + 32h (+16).
  const int kfrag = (r32 % T::NB) * T::PITCH + (r32 / T::NB) * D + 32 * h;
  auto qk = [&](auto buf, f32x16 (&s)[2]) {
    const lds_char* kp = kbuf(buf) + kfrag;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
    for (int sd = 0; sd < D / 64; ++sd)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const lds_char* p = kp + kb * (32 / T::NB) * D + 64 * sd;
        const u32x4 a0 = *(const __attribute__((address_space(3))) u32x4*)(p);
        const u32x4 a1 = *(const __attribute__((address_space(3))) u32x4*)(p + 16);
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                         (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        s[kb] = mfma_32x32x64_e4m3(a, qf[sd], s[kb]);
      }
  };
  // V^T: lane (r32, h) needs, for d = 32mb + r32, the keys of P's byte
  // order: byte t of 32 = key 32(t/16) + 8((t%16)/4) + 4h + t%4. Read j
  // (t = 8j..8j+7): this lane names row u = (r32%16)/2 of the read, i.e.
  // key 32(j/2) + 16(j%2) + 8(u/4) + 4h + u%4, bytes 16(r32/16) + 8(r32%2)
  // of the 32-column block mb (chunk 2mb + r32/16, placed as above).
  int vaddr[4];
  {
    const int u = (r32 & 15) >> 1;
    const int q = r32 >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 32 * (j >> 1) + 16 * (j & 1) + 8 * (u >> 2) + 4 * h + (u & 3);
      const int vs = v_slot<D>(key);
      vaddr[j] = v_block<D>(key) * T::PITCH + (vs ^ (q * kS)) * D +
                 16 * ((vs / kS) & 1) + 8 * (r32 & 1);
    }
  }
  auto skip_tile = [&](int tile) {
    return CAUSAL && (tile * kBN > wrow0 + 31 + off);
  };

  // Two passes, the second almost never run (as in the bf16 kernel): the
  // first fixes the exponent reference at the first key tile's row
  // maximum and never moves it, so a tile needs no row maximum, reference
  // test or O rescale. P then stays at most 2^(later max - first max);
  // once that passes the e4m3 range, its conversion gives NaN codes (no
  // saturation), which reach O and the rounded sum; the workgroup then
  // runs its tiles again with the lazy reference (P <= 2^8 = 256 < 448).
  constexpr std::integral_constant<int, 0> B0{};
  constexpr std::integral_constant<int, 1> B1{};
  __shared__ int redo;
  auto run = [&](auto fixed_ref) {
    constexpr bool FIXED = decltype(fixed_ref)::value;
    // ---- prologue: K(0), V(0), K(1) in flight; S(0)
    if (nt > 0) {
      issue_k(0, B0);
      issue_v(0, B0);
      if (nt > 1) issue_k(1, B1);
    }
    wait_vm0();
    __syncthreads();
    f32x16 sc[2];
    // row max of the next tile's scores, taken beside the previous tile's P.V
    // products; a tile that needs masking takes its max again after the mask
    float mx_next = kNegInf;
    if (nt > 0 && !skip_tile(0)) {
      qk(B0, sc);
      mx_next = tile_max<2>(sc);
    }
    __syncthreads();  // K buffer 0 is refilled below

    // One key tile t (parity P): S(t) arrives in sc, S(t+1) is computed into
    // sn while P(t) is formed. K runs two tiles ahead and V one: both target
    // buffers were last read before the previous barrier. Tiles are taken in
    // pairs with the score buffers swapping roles (no register copies).
    auto step = [&](int t, auto par, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      constexpr int P = decltype(par)::value;
      constexpr std::integral_constant<int, P> cur{};
      constexpr std::integral_constant<int, 1 - P> nxt{};
      const int n0 = t * kBN;
      if (t + 2 < nt) issue_k(t + 2, cur);
      if (t + 1 < nt) issue_v(t + 1, nxt);
      if (!skip_tile(t)) {
        const bool need_mask =
            (n0 + kBN > Nk) || (CAUSAL && n0 + kBN - 1 > wrow0 + off);
        if (need_mask) {
          const int lim = CAUSAL ? min(Nk - 1, row + off) : Nk - 1;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int key = n0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
              if (key > lim) sc[kb][v] = kNegInf;
            }
        }
        if (!FIXED || t == 0) {
          const float mx = need_mask ? tile_max<2>(sc) : mx_next;
          const float alpha = move_reference(mx, st, c);
          if (!FIXED && __any(alpha != 1.f)) {
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
              for (int v = 0; v < 16; ++v) o[mb][v] *= alpha;
            lsum[0] *= alpha;
          }
        }
        // S(t+1) on the matrix cores while P(t) is formed on the VALU (past
        // the last tile, or beyond this wave's causal rows, the product is
        // never read and its buffer is not being written)
        // raised issue priority while this wave feeds the matrix cores: the
        // other wave of the SIMD fills in with its VALU work
        __builtin_amdgcn_s_setprio(1);
        qk(nxt, sn);
        const float mref = (st.m == kNegInf) ? 0.f : st.m;
        float sum = 0.f;
        i32x8 pb;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int kb = jj >> 2, v0 = 4 * (jj & 3);
          float p4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p4[e] = fast_exp2(__builtin_fmaf(sc[kb][v0 + e], c, -mref));
            sum += p4[e];
          }
          pb[jj] = (int)pack_e4m3x4(p4[0], p4[1], p4[2], p4[3]);
        }
        st.l += sum;
        lsum = mfma_32x32x64_fp4_e4m3(ones, pb, lsum);
        const lds_char* vp = vbuf(cur);
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
          i32x8 a;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            typedef int v2i __attribute__((ext_vector_type(2)));
            const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i*)(vp + vaddr[j] + 32 * mb));
            a[2 * j] = r[0];
            a[2 * j + 1] = r[1];
          }
          o[mb] = mfma_32x32x64_e4m3(a, pb, o[mb]);
        }
        if (!FIXED) mx_next = tile_max<2>(sn);
        __builtin_amdgcn_s_setprio(0);
      }
      wait_vm0();
      __syncthreads();
    };
    f32x16 sb[2];
    for (int t = 0; t < nt; t += 2) {
      step(t, B0, sc, sb);
      if (t + 1 < nt) step(t + 1, B1, sb, sc);
    }

  };
  if (tid == 0) redo = 0;
  run(std::true_type{});
  {
    // inf or NaN anywhere in this lane's l, rounded sum or O
    float chk = st.l + lsum[0];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) chk += o[mb][v] * 0.f;
    if (__any(!__builtin_isfinite(chk)) && lane == 0) redo = 1;
  }
  __syncthreads();
  if (redo) {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[mb][v] = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) lsum[v] = 0.f;
    st = RowState{kNegInf, 0.f, 0.f};
    run(std::false_type{});
  }

  // ---- epilogue: O = s_v * O^T / lr, LSE = ln 2 * (m + log2 l)
  const float ltot = sum_halves(st.l);
  const float lrtot = lsum[0];
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
