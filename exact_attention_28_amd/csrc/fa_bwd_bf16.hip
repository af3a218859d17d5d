// fa_bwd_bf16.hip - exact attention backward, bf16 in / bf16 gradients, gfx950.
//
// The forward keeps no P: the backward re-computes it on chip from Q, K and
// the saved row statistics (LSE), as the pages prescribe for the backward
// pass ([Capstone §6.1], the row about writing P to HBM; §7.3 question 1).
// With P_ij = exp(scale * q_i.k_j - LSE_i) and D_i = rowsum(dO_i * O_i)
// (= rowsum(P_i * dP_i), the softmax Jacobian's correction term):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// with dK, dV of a KV head summed over the query heads of its group.
//
// Three kernels, no atomics (the result does not depend on scheduling):
//  * bwd_prep_kernel: -D_i and LSE_i * log2(e) (+inf for a row that saw no
//    key, so its P evaluates to 0) into the workspace; -D_i is the starting
//    value of the dP products, which then leave dP - D directly.
//  * bwd_dkdv_kernel (key-outer): a workgroup owns 128 keys of one (batch,
//    KV head), 32 per wave, with the wave's K and V rows held as MFMA
//    operands in registers; it streams 32-row tiles of Q and dO (and their
//    D, LSE) of every query head of the group through LDS and accumulates
//    dK^T and dV^T in registers. Per tile and wave, on
//    v_mfma_f32_32x32x16_bf16: S = Q K^T and dP = dO V^T (lane = key, so
//    the accumulators become the B operands below without leaving
//    registers), then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T
//    read from row-major LDS by the gfx950 transpose read.
//  * bwd_dq_kernel (query-outer, the forward's order): a workgroup owns a
//    128-row query tile, 32 rows per wave, with Q and dO held as operands;
//    it streams 64-key K/V tiles through LDS: S^T = K Q^T, dP^T = V dO^T,
//    dS^T, then dQ^T += K^T dS^T with K^T from the transpose read.
// Causal: key j is visible to row i iff j <= i + (Nk - Nq); tiles that no
// row of a wave can see are skipped, tiles crossing the diagonal masked.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = kThreads / 64;

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;


// A row-major tile of ROWS rows x D bf16 in LDS, as 1 KB blocks (one direct
// load instruction: 64 lanes x 16 B) at a pitch of 1 KB + 16 B. RowTile
// below and IlvTile (the interleaved layout, fa_device.h) share one
// interface: row_off(r) + chunk_off(k) is the byte offset of the
// 16-byte chunk k of row r, row_off(r) + col_off(x) that of byte x of row r,
// and the direct load of block b moves chunk lane_chunk(lane) of row
// block_row(b, lane) to byte 16 * lane of the block.
//
// RowTile: row r in block r % NB at slot r / NB. Sixteen consecutive rows
// read at one chunk (the A operand of a row-major product) fall in sixteen
// different blocks when NB >= 16, whose pitch spreads them over the banks;
// reads of the transpose (4 consecutive rows x 64 B per 32-lane half) meet
// up to 4-way conflicts. Used where a tile is only read by rows, and at
// d = 64.
template <int D, int ROWS>
struct RowTile {
  static constexpr int RPB = 1024 / (2 * D);  // rows per block
  static constexpr int NB = ROWS / RPB;       // blocks
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int PITCH = 1040;
  static constexpr int BYTES = NB * PITCH;
  static constexpr int BPW = NB / kWaves;     // blocks each wave loads
  static __device__ __forceinline__ constexpr int row_off(int r) {
    return (r % NB) * PITCH + (r / NB) * (2 * D);
  }
  static __device__ __forceinline__ constexpr int chunk_off(int k) { return 16 * k; }
  static __device__ __forceinline__ constexpr int col_off(int x) { return x; }
  static __device__ __forceinline__ int block_row(int b, int lane) {
    return b + NB * (lane / CPR);
  }
  static __device__ __forceinline__ int lane_chunk(int lane) { return lane % CPR; }
};

// The layout of a tile that is read both ways.
template <int D, int ROWS>
using TrTile = std::conditional_t<D == 128, IlvTile<ROWS, kWaves>, RowTile<D, ROWS>>;

// Issues the direct loads of one tile of layout T: rows [r0, r0 + rows) of
// a row-major [n, D] matrix, rows at or past n clamped to the last one
// (never used).
template <int D, class T>
__device__ __forceinline__ void load_tile(const __bf16* src, int r0, int n,
                                          lds_char* dst, int w, int lane) {
  const int chunk = T::lane_chunk(lane);
#pragma unroll
  for (int i = 0; i < T::BPW; ++i) {
    const int b = w + kWaves * i;
    const int r = min(r0 + T::block_row(b, lane), n - 1);
    g2lds_16B_own(src + (long)r * D + 8 * chunk, dst + b * T::PITCH);
  }
}

// 16 bytes of a row (A operand of a row-major product: row, d = 8h + 16s).
__device__ __forceinline__ bf16x8 lds_row16(const lds_char* p) {
  return *(const lds_bf16x8*)p;
}
// Transposed A operand (columns d of the tile as rows of the operand): two
// ds_read_b64_tr_b16, each handing the lane 4 consecutive tile rows of its
// column; the caller's offsets name rows base + 4h + (lane%16)/4 and + 8.
__device__ __forceinline__ bf16x8 lds_tr16(const lds_char* lo,
                                           const lds_char* hi) {
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lo);
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)hi);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ------------------------------------------------------------------ prep
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const __bf16* __restrict__ O, const __bf16* __restrict__ dO,
    const float* __restrict__ LSE, float* __restrict__ Dv,
    float* __restrict__ L2, long rows, long rows_padded) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long r = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int cc = threadIdx.x % LPR;
  // the padding rows after the last head are read by the last query tile
  // of the dK/dV kernel (for rows that do not exist, so masked): they get
  // D = 0 and L2 = +inf (P = 0) here, whatever the workspace held before
  if (r >= rows) {
    if (r < rows_padded && cc == 0) {
      Dv[r] = 0.f;
      L2[r] = __builtin_inff();
    }
    return;
  }
  float acc = 0.f;
  {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(O + r * D + 8 * cc);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dO + r * D + 8 * cc);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (cc == 0) {
    Dv[r] = -acc;  // stored negated: the dP products start from it
    const float l = LSE[r];
    L2[r] = (l == kNegInf) ? __builtin_inff() : l * kLog2e;
  }
}

// -------------------------------------------------------------- dK, dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
    const float* __restrict__ Dv, const float* __restrict__ L2,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int B, int Hq, int Hkv,
    int Nq, int Nk, float c, float scale, int slots) {
  constexpr int BR = 32;  // query rows per tile
  using T = TrTile<D, BR>;      // Q, dO: read by rows and transposed
  using TV = RowTile<D, 128>;   // V: read by rows only
  // the workgroup's 128 V rows, read as B operands every tile (holding
  // them in registers as well as K would leave one wave per SIMD)
  __shared__ __attribute__((aligned(16))) char v_lds[TV::BYTES];
  __shared__ __attribute__((aligned(16))) char q_lds0[T::BYTES];
  __shared__ __attribute__((aligned(16))) char q_lds1[T::BYTES];
  __shared__ __attribute__((aligned(16))) char o_lds0[T::BYTES];
  __shared__ __attribute__((aligned(16))) char o_lds1[T::BYTES];
  __shared__ __attribute__((aligned(16))) float s_lds0[2 * BR];  // L2, D
  __shared__ __attribute__((aligned(16))) float s_lds1[2 * BR];
  auto qbuf = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)q_lds0;
    else return (lds_char*)q_lds1;
  };
  auto obuf = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)o_lds0;
    else return (lds_char*)o_lds1;
  };
  auto sbuf = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)s_lds0;
    else return (lds_char*)s_lds1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int h = lane >> 5;
  const int r32 = lane & 31;
  const int i16 = lane & 15;

  // key tiles of 128 in ascending order (for causal the heaviest first),
  // KV heads of one batch XCD-contiguous
  const int n_kt = (Nk + 127) / 128;
  const TileIdx ti = map_tile(blockIdx.x, n_kt, Hkv, Hkv, B, false);
  const int hk = ti.hq;
  const int G = Hq / Hkv;
  const int k0 = ti.qt * 128;
  const int wk0 = k0 + 32 * w;
  const int key = wk0 + r32;
  const int keyc = min(key, Nk - 1);
  const int off = Nk - Nq;

  // this wave's 32 keys of K as B operands (lane: key r32, d = 16s + 8h +
  // t); the workgroup's 128 V rows go to LDS
  const long kvbase = (long)(ti.b * Hkv + hk) * Nk * D;
  bf16x8 kf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    kf[s] = *reinterpret_cast<const bf16x8*>(K + kvbase + (long)keyc * D + 16 * s + 8 * h);
  load_tile<D, TV>(V + kvbase, k0, Nk, (lds_char*)v_lds, w, lane);
  const lds_char* vrow = (const lds_char*)v_lds + TV::row_off(32 * w + r32) + TV::chunk_off(h);
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) dk[mb][v] = dv[mb][v] = 0.f;

  // query tiles [32t, 32t + 32) that can see a key of this workgroup,
  // taken in order along the query range (direction below), the group's
  // heads inner: the workgroups of a KV head that run together move
  // through Q and dO abreast, so a tile fetched once serves them from L2
  const int nqt = (Nq + BR - 1) / BR;
  const int t0 = CAUSAL ? min(nqt, max(0, k0 - off) / BR) : 0;
  const int per_head = nqt - t0;
  const int n_it = G * per_head;
  // Walk direction. The workgroups of an XCD run `slots` at a time, in
  // dispatch order, heaviest first. Those of the first round start
  // together at the last query tile and walk down abreast. Each slot then
  // takes the next workgroup as its previous one ends, and the earlier a
  // slot frees, the longer its next workgroup: walking up from its first
  // visible tile, that round moves abreast as well (every slot reaches a
  // given tile at about the same time), so one fetch of a tile serves the
  // whole round from L2. Rounds alternate; without the causal mask all
  // workgroups are equally long and walk down.
  const int round = __builtin_amdgcn_readfirstlane((int)(blockIdx.x >> 3) / slots);
  const bool up = CAUSAL && (round & 1);
  const int tstart = up ? t0 : nqt - 1, tstep = up ? 1 : -1;

  // iteration it takes head g = it % G of the group and query tile
  // t = tstart + tstep * (it / G); (g, t) are carried from one iteration
  // to the next instead of divided out
  auto issue = [&](int g, int t, auto buf) {
    const long qb = (long)(ti.b * Hq + hk * G + g) * Nq;
    load_tile<D, T>(Q + qb * D, BR * t, Nq, qbuf(buf), w, lane);
    load_tile<D, T>(dO + qb * D, BR * t, Nq, obuf(buf), w, lane);
    if (w == 0) {
      // the tile's 32 L2 values (lanes 0-31) then its 32 D values, one
      // dword per lane; rows past Nq read the next head's values or the
      // padding the prep kernel fills (masked either way, and finite or
      // +inf L2 with finite D, so P and dS come out exactly 0)
      const float* src = (lane < 32 ? L2 : Dv) + qb + BR * t + (lane & 31);
      g2lds_4B_own(src, sbuf(buf));
    }
  };

  // per-lane fragment offsets in a tile: row r32, chunk h (+ the step's
  // chunks 2 sd); the transposed operand's rows 16j + 8e + 4h + i16/4 at
  // column bytes 2 * (16 * ((lane >> 4) & 1) + 4 * (i16 & 3)) (+ 64 mb).
  // Each is one base register plus compile-time offsets (the layouts are
  // additive over the splits used here).
  const int rfrag = T::row_off(r32) + T::chunk_off(h);
  const int tbase = T::row_off(4 * h + (i16 >> 2)) +
                    T::col_off(2 * (16 * ((lane >> 4) & 1) + 4 * (i16 & 3)));
  auto tfrag = [&](int j, int e) { return tbase + T::row_off(16 * j + 8 * e); };

  constexpr std::integral_constant<int, 0> B0{};
  constexpr std::integral_constant<int, 1> B1{};
  if (n_it > 0) issue(0, tstart, B0);
  int cg = 0, ct = tstart;  // (g, t) of the current iteration

  auto step = [&](int it, auto par) {
    constexpr int P = decltype(par)::value;
    constexpr std::integral_constant<int, P> cur{};
    constexpr std::integral_constant<int, 1 - P> nxt{};
    // this tile in LDS (own loads, then everyone's); the other buffer was
    // last read before the previous barrier
    wait_vm0();
    __syncthreads();
    int ng = cg + 1, nt = ct;
    if (ng == G) { ng = 0; nt += tstep; }
    if (it + 1 < n_it) issue(ng, nt, nxt);
    const int t = ct;
    cg = ng;
    ct = nt;
    const int i0 = BR * t;
    if (CAUSAL && i0 + BR - 1 + off < wk0) return;  // no row sees these keys
    const lds_char* qp = qbuf(cur);
    const lds_char* op = obuf(cur);
    // S = Q K^T and dP = dO V^T: lane = key r32, rows 8(v/4) + 4h + v%4.
    // The MFMA phases run at raised issue priority, so while one wave
    // feeds the matrix cores the other wave of the SIMD fills in with its
    // VALU work.
    // S starts at 0; dP starts at -D of its row (element v: row 8(v/4) +
    // 4h + v%4), so the products leave dP - D and dS = P (dP - D) needs no
    // subtraction
    const lds_char* sp = sbuf(cur);
    f32x16 s, p;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4 nd = *(const lds_f32x4*)(sp + 4 * BR + 4 * (8 * gq + 4 * h));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[4 * gq + e] = 0.f;
        p[4 * gq + e] = nd[e];
      }
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int sd = 0; sd < D / 16; ++sd) {
      s = mfma_32x32x16_bf16(lds_row16(qp + rfrag + T::chunk_off(2 * sd)), kf[sd], s);
      p = mfma_32x32x16_bf16(lds_row16(op + rfrag + T::chunk_off(2 * sd)),
                             lds_row16(vrow + TV::chunk_off(2 * sd)), p);
    }
    __builtin_amdgcn_s_setprio(0);
    // P and dS per element; rows past Nq and causally hidden pairs get 0
    // (the test is uniform over the wave: tiles wholly inside the visible
    // region take the copy of the loop without the per-element test)
    const bool need_mask = (i0 + BR > Nq) || (CAUSAL && i0 + off < wk0 + 31);
    uint32_t pp[2][4], dd[2][4];
    auto elementwise = [&](auto masked) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 l2 = *(const lds_f32x4*)(sp + 4 * (8 * gq + 4 * h));
        float pv[4], dv4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * gq + e;
          float sv = s[v];
          if constexpr (decltype(masked)::value) {
            const int i = i0 + 8 * gq + 4 * h + e;
            const bool vis = (i < Nq) & (!CAUSAL | (key <= i + off));
            sv = vis ? sv : kNegInf;
          }
          pv[e] = fast_exp2(__builtin_fmaf(sv, c, -l2[e]));
          dv4[e] = pv[e] * p[v];
        }
        // element pairs of rows 16j + {4h.., 8 + 4h..}: j = gq / 2
        const int j = gq >> 1, t2 = 2 * (gq & 1);
        pp[j][t2] = pack_bf16x2(pv[0], pv[1]);
        pp[j][t2 + 1] = pack_bf16x2(pv[2], pv[3]);
        dd[j][t2] = pack_bf16x2(dv4[0], dv4[1]);
        dd[j][t2 + 1] = pack_bf16x2(dv4[2], dv4[3]);
      }
    };
    if (need_mask) elementwise(std::true_type{});
    else elementwise(std::false_type{});
    // dV^T += dO^T P and dK^T += Q^T dS, 16 rows per MFMA
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pp[j][0], pp[j][1], pp[j][2], pp[j][3]});
      const bf16x8 db = __builtin_bit_cast(bf16x8, u32x4{dd[j][0], dd[j][1], dd[j][2], dd[j][3]});
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
        dv[mb] = mfma_32x32x16_bf16(
            lds_tr16(op + tfrag(j, 0) + T::col_off(64 * mb),
                     op + tfrag(j, 1) + T::col_off(64 * mb)), pb, dv[mb]);
        dk[mb] = mfma_32x32x16_bf16(
            lds_tr16(qp + tfrag(j, 0) + T::col_off(64 * mb),
                     qp + tfrag(j, 1) + T::col_off(64 * mb)), db, dk[mb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  for (int it = 0; it < n_it; it += 2) {
    step(it, B0);
    if (it + 1 < n_it) step(it + 1, B1);
  }

  // ---- epilogue: dK = scale * dK^T, dV = dV^T (lane: key, d = 32mb + 8g + 4h + e)
  if (key < Nk) {
    __bf16* krow = dK + kvbase + (long)key * D;
    __bf16* vrow = dV + kvbase + (long)key * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 a, b;
        a[0] = pack_bf16x2(dk[mb][4 * gq] * scale, dk[mb][4 * gq + 1] * scale);
        a[1] = pack_bf16x2(dk[mb][4 * gq + 2] * scale, dk[mb][4 * gq + 3] * scale);
        b[0] = pack_bf16x2(dv[mb][4 * gq], dv[mb][4 * gq + 1]);
        b[1] = pack_bf16x2(dv[mb][4 * gq + 2], dv[mb][4 * gq + 3]);
        *reinterpret_cast<u32x2*>(krow + 32 * mb + 8 * gq + 4 * h) = a;
        *reinterpret_cast<u32x2*>(vrow + 32 * mb + 8 * gq + 4 * h) = b;
      }
  }
}

// ------------------------------------------------------------------- dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
    const float* __restrict__ Dv, const float* __restrict__ L2,
    __bf16* __restrict__ dQ, int B, int Hq, int Hkv, int Nq, int Nk, float c,
    float scale, int slots) {
  constexpr int BN = 64;  // keys per tile
  using T = TrTile<D, BN>;  // K read by rows and transposed; V by rows
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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int h = lane >> 5;
  const int r32 = lane & 31;
  const int i16 = lane & 15;

  const int n_qt = (Nq + 127) / 128;
  const TileIdx ti = map_tile(blockIdx.x, n_qt, Hq, Hkv, B, CAUSAL);
  const int hk = ti.hq / (Hq / Hkv);
  const int q0 = ti.qt * 128;
  const long qbase = (long)(ti.b * Hq + ti.hq) * Nq;
  const __bf16* Kh = K + (long)(ti.b * Hkv + hk) * Nk * D;
  const __bf16* Vh = V + (long)(ti.b * Hkv + hk) * Nk * D;
  const int off = Nk - Nq;
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(q0 + 128, Nq) + off);
  const int nt = kend > 0 ? (kend + BN - 1) / BN : 0;

  const int wrow0 = q0 + w * 32;
  const int row = wrow0 + r32;
  const int rowc = min(row, Nq - 1);
  // this wave's rows of Q and dO as B operands (row r32, d = 16s + 8h + t)
  bf16x8 qf[D / 16], of[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = *reinterpret_cast<const bf16x8*>(Q + (qbase + rowc) * D + 16 * s + 8 * h);
    of[s] = *reinterpret_cast<const bf16x8*>(dO + (qbase + rowc) * D + 16 * s + 8 * h);
  }
  const float l2 = L2[qbase + rowc];
  // -D of this lane's row in every element: the accumulator input of the
  // first dP product of each tile, so the products leave dP - D
  f32x16 negd;
  {
    const float nd = Dv[qbase + rowc];
#pragma unroll
    for (int v = 0; v < 16; ++v) negd[v] = nd;
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[mb][v] = 0.f;

  // fragment offsets: K/V rows 32kb + r32, chunk h (+ the step's chunks
  // 2 sd); K^T rows 32kb + 16j + 8e + 4h + i16/4 at column bytes
  // 2*(16*((lane>>4)&1) + 4*(i16&3)) (+ 64 mb). Each is one base register
  // plus a compile-time constant (the layouts are additive over the splits
  // used here).
  const int rbase = T::row_off(r32) + T::chunk_off(h);
  const int tbase = T::row_off(4 * h + (i16 >> 2)) +
                    T::col_off(2 * (16 * ((lane >> 4) & 1) + 4 * (i16 & 3)));
  auto rfrag = [&](int kb) { return rbase + T::row_off(32 * kb); };
  auto tfrag = [&](int kb, int j, int e) {
    return tbase + T::row_off(32 * kb + 16 * j + 8 * e);
  };

  auto issue = [&](int tile, auto buf) {
    load_tile<D, T>(Kh, BN * tile, Nk, kbuf(buf), w, lane);
    load_tile<D, T>(Vh, BN * tile, Nk, vbuf(buf), w, lane);
  };
  auto skip_tile = [&](int tile) {
    return CAUSAL && (tile * BN > wrow0 + 31 + off);
  };
  // Walk direction over the key tiles (see the dK/dV kernel): the first
  // round of an XCD's workgroups starts together and walks up from key 0;
  // the next round, whose workgroups start one by one as the longest
  // before them end, walks down from its last visible tile and so stays
  // abreast; rounds alternate.
  const int round = __builtin_amdgcn_readfirstlane((int)(blockIdx.x >> 3) / slots);
  const bool down = CAUSAL && (round & 1);
  auto tile_at = [&](int it) { return down ? nt - 1 - it : it; };

  constexpr std::integral_constant<int, 0> B0{};
  constexpr std::integral_constant<int, 1> B1{};
  if (nt > 0) issue(tile_at(0), B0);

  auto step = [&](int t, auto par) {
    constexpr int P = decltype(par)::value;
    constexpr std::integral_constant<int, P> cur{};
    constexpr std::integral_constant<int, 1 - P> nxt{};
    wait_vm0();
    __syncthreads();
    if (t + 1 < nt) issue(tile_at(t + 1), nxt);
    const int tl = tile_at(t);
    if (skip_tile(tl)) return;
    const int n0 = tl * BN;
    const lds_char* kp = kbuf(cur);
    const lds_char* vp = vbuf(cur);
    // S^T = K Q^T, dP^T = V dO^T: lane = row r32, keys 32kb + 8(v/4) + 4h + v%4
    // (dP^T starts from -D of the lane's row: the first product takes negd
    // as its accumulator input)
    f32x16 s[2], p[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int sd = 0; sd < D / 16; ++sd)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = mfma_32x32x16_bf16(lds_row16(kp + rfrag(kb) + T::chunk_off(2 * sd)), qf[sd], s[kb]);
        p[kb] = mfma_32x32x16_bf16(lds_row16(vp + rfrag(kb) + T::chunk_off(2 * sd)), of[sd],
                                   sd == 0 ? negd : p[kb]);
      }
    __builtin_amdgcn_s_setprio(0);
    // (uniform over the wave: tiles wholly inside the visible region take
    // the copy of the loop without the per-element test)
    const bool need_mask = (n0 + BN > Nk) || (CAUSAL && n0 + BN - 1 > wrow0 + off);
    const int lim = CAUSAL ? min(Nk - 1, row + off) : Nk - 1;
    uint32_t dd[2][2][4];
    auto elementwise = [&](auto masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float ds[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float sv = s[kb][v];
          if constexpr (decltype(masked)::value) {
            const int kk = n0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
            if (kk > lim) sv = kNegInf;
          }
          const float pv = fast_exp2(__builtin_fmaf(sv, c, -l2));
          ds[v] = pv * p[kb][v];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2)
            dd[kb][j][t2] = pack_bf16x2(ds[8 * j + 2 * t2], ds[8 * j + 2 * t2 + 1]);
      }
    };
    if (need_mask) elementwise(std::true_type{});
    else elementwise(std::false_type{});
    // dQ^T += K^T dS^T, 16 keys per MFMA
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 db = __builtin_bit_cast(
            bf16x8, u32x4{dd[kb][j][0], dd[kb][j][1], dd[kb][j][2], dd[kb][j][3]});
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
          acc[mb] = mfma_32x32x16_bf16(
              lds_tr16(kp + tfrag(kb, j, 0) + T::col_off(64 * mb),
                       kp + tfrag(kb, j, 1) + T::col_off(64 * mb)),
              db, acc[mb]);
      }
    __builtin_amdgcn_s_setprio(0);
  };
  for (int t = 0; t < nt; t += 2) {
    step(t, B0);
    if (t + 1 < nt) step(t + 1, B1);
  }

  if (row < Nq) {
    __bf16* orow = dQ + (qbase + row) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pr;
        pr[0] = pack_bf16x2(acc[mb][4 * g] * scale, acc[mb][4 * g + 1] * scale);
        pr[1] = pack_bf16x2(acc[mb][4 * g + 2] * scale, acc[mb][4 * g + 3] * scale);
        *reinterpret_cast<u32x2*>(orow + 32 * mb + 8 * g + 4 * h) = pr;
      }
  }
}

// Workspace: D then L2, each [B*Hq*Nq] fp32 followed by at least one tile
// (32 rows) of padding that the last tile of the last head may read.
long bwd_rows_padded(long rows) { return (rows + 32 + 63) / 64 * 64; }

// Workgroups of the dK/dV or dQ kernel that one XCD of the current device
// runs at once: both kernels fit two workgroups on a CU (two waves per
// SIMD by their launch bounds, 66 KB of LDS each), and the tile maps
// spread the grid over the 8 XCDs.
int slots_per_xcd() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess)
    cus = 256;
  return max(1, cus * 2 / 8);
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  const long rows = (long)a.B * a.Hq * a.Nq;
  float* Dv = static_cast<float*>(a.ws);
  float* L2 = Dv + bwd_rows_padded(rows);  // both arrays rows_padded long
  const float c = a.scale * kLog2e;
  const long rows_padded = bwd_rows_padded(rows);
  const long prep_blocks = (rows_padded * (D / 8) + 255) / 256;
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)prep_blocks),
                     dim3(256), 0, a.stream, static_cast<const __bf16*>(a.o),
                     static_cast<const __bf16*>(a.dout), a.lse, Dv, L2, rows,
                     rows_padded);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long kv_blocks = (long)((a.Nk + 127) / 128) * a.Hkv * a.B;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)kv_blocks),
                     dim3(kThreads), 0, a.stream,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dout),
                     Dv, L2, static_cast<__bf16*>(a.dk), static_cast<__bf16*>(a.dv),
                     a.B, a.Hq, a.Hkv, a.Nq, a.Nk, c, a.scale,
                     slots_per_xcd());
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long q_blocks = (long)((a.Nq + 127) / 128) * a.Hq * a.B;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)q_blocks),
                     dim3(kThreads), 0, a.stream,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dout),
                     Dv, L2, static_cast<__bf16*>(a.dq), a.B, a.Hq, a.Hkv, a.Nq,
                     a.Nk, c, a.scale,
                     slots_per_xcd());
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int Hq, int Nq) {
  return (size_t)(2 * bwd_rows_padded((long)B * Hq * Nq)) * 4;
}

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

}  // namespace fa
