// fa_naive.hip - the three-kernel attention the pages use as the contrast
// to the fused kernel ([Capstone §0] and §1.1): the score matrix S and the
// probabilities P are materialised in device memory, every kernel a round
// trip through HBM:
//   naive_scores_kernel   S = scale * Q K^T          (write S: 2 bytes/score)
//   naive_softmax_kernel  P = softmax(S) row by row  (read S, write P)
//   naive_pv_kernel       O = P V                    (read P and V, write O)
// which moves 8Nd + 8N^2 bytes per head at 2 bytes per element ([Capstone
// §1.1], the traffic ledger) against the fused kernel's 8Nd. S is stored as
// fp16 (the pages' element type, which keeps the scores' precision) and P
// as bf16 (the PV operand type) in the same buffer, each row of P written
// over its row of S. The masking (bottom-right causal) is applied in the
// softmax kernel, as a plain implementation would; the product kernels do
// not skip masked tiles.
//
// The two products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation
// (Q K^T with K tiles staged in LDS; P V with V tiles staged in LDS and read
// transposed); they are written to be reasonable, not slow, so that what the
// measurement shows is the traffic.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));


// 64-row tile of D bf16 in LDS, 1 KB blocks at a 1040 B pitch, row r in
// block r % NB, slot r / NB (16-byte row reads conflict free).
template <int D>
struct Tile64 {
  static constexpr int RPB = 1024 / (2 * D);
  static constexpr int NB = 64 / RPB;
  static constexpr int CPR = D / 8;
  static constexpr int PITCH = 1040;
  static constexpr int BYTES = NB * PITCH;
  static constexpr int BPW = NB / 4;
  static __device__ __forceinline__ constexpr int row_off(int r) {
    return (r % NB) * PITCH + (r / NB) * (2 * D);
  }
  static __device__ __forceinline__ constexpr int col_off(int x) { return x; }
  static __device__ __forceinline__ int block_row(int b, int lane) {
    return b + NB * (lane / CPR);
  }
  static __device__ __forceinline__ int lane_chunk(int lane) { return lane % CPR; }
};
// V tiles are only read transposed: at d = 128 the interleaved layout keeps
// those reads conflict free (four consecutive rows 64 B apart)
template <int D>
using VTile64 = std::conditional_t<D == 128, IlvTile<64, 4>, Tile64<D>>;
// Direct loads of rows [r0, r0 + 64) of a row-major [n, D] matrix into a
// tile of layout T (rows past n clamped to the last one, never used).
template <int D, class T = Tile64<D>>
__device__ __forceinline__ void load64(const __bf16* src, int r0, int n,
                                       lds_char* dst, int w, int lane) {
  const int chunk = T::lane_chunk(lane);
#pragma unroll
  for (int i = 0; i < T::BPW; ++i) {
    const int b = w + 4 * i;
    const int r = min(r0 + T::block_row(b, lane), n - 1);
    g2lds_16B(src + (long)r * D + 8 * chunk, dst + b * T::PITCH);
  }
}

// ----------------------------------------------------------- S = Q K^T
// Workgroup: 128 query rows (32 per wave) of one (batch, head) against
// every key, 64 keys per tile. S = Q K^T with Q as the A operand (rows in
// registers) and K^T as the B operand (key rows from LDS), so a lane holds
// one key column. Each wave's 32 x 64 tile of S goes through a small LDS
// buffer (row pitch 136 B) and leaves as 16-byte pieces, eight lanes per
// 128-byte row segment, so the stores of S are whole segments.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void naive_scores_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    _Float16* __restrict__ S, int B, int Hq, int Hkv, int Nq, int Nk,
    float scale) {
  using T = Tile64<D>;
  __shared__ __attribute__((aligned(16))) char kl0[T::BYTES];
  __shared__ __attribute__((aligned(16))) char kl1[T::BYTES];
  constexpr int kSPitch = 136;  // bytes per staged row of 64 fp16 scores
  __shared__ __attribute__((aligned(16))) char sl[4][32 * kSPitch];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int n_qt = (Nq + 127) / 128;
  const TileIdx ti = map_tile(blockIdx.x, n_qt, Hq, Hkv, B, false);
  const int hk = ti.hq / (Hq / Hkv);
  const long bh = (long)ti.b * Hq + ti.hq;
  const __bf16* Kh = K + ((long)ti.b * Hkv + hk) * Nk * D;
  const int row0 = ti.qt * 128 + 32 * w;
  const int rowc = min(row0 + r32, Nq - 1);
  bf16x8 qa[D / 16];  // A operand: row r32, d = 16s + 8h
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qa[s] = *reinterpret_cast<const bf16x8*>(Q + (bh * Nq + rowc) * D + 16 * s + 8 * h);
  const int nt = (Nk + 63) / 64;
  const int kfrag = T::row_off(r32) + 16 * h;
  auto buf = [&](int i) -> lds_char* { return (lds_char*)(i ? kl1 : kl0); };
  load64<D>(Kh, 0, Nk, buf(0), w, lane);
  for (int t = 0; t < nt; ++t) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (t + 1 < nt) load64<D>(Kh, 64 * (t + 1), Nk, buf((t + 1) & 1), w, lane);
    const lds_char* kp = buf(t & 1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        acc = mfma_32x32x16_bf16(
            qa[s], *(const lds_bf16x8*)(kp + kfrag + T::row_off(32 * kb) + 32 * s), acc);
      // lane: key 32kb + r32 of the tile, rows 8(v/4) + 4h + v%4
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * h + (v & 3);
        *(__attribute__((address_space(3))) _Float16*)(
            (lds_char*)sl[w] + r * kSPitch + 2 * (32 * kb + r32)) =
            (_Float16)(acc[v] * scale);
      }
    }
    // the wave's tile back out: lane l takes 8 keys (16 B) of row l/8 + 8i
    const int chunk = lane & 7, key = 64 * t + 8 * chunk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (lane >> 3) + 8 * i;
      const u32x4 piece = *(const __attribute__((address_space(3))) u32x4*)(
          (lds_char*)sl[w] + r * kSPitch + 16 * chunk);
      if (key < Nk && row0 + r < Nq)
        *reinterpret_cast<u32x4*>(S + (bh * Nq + row0 + r) * Nk + key) = piece;
    }
  }
}

// -------------------------------------------------------- P = softmax(S)
// One workgroup per row (rows of more than 4096 keys): the row's scores
// are read once into registers as 16-byte pieces of 8 (Nk is a multiple of
// 8, so rows are 16-byte aligned; NP pieces per thread), the three passes
// of the safe softmax ([Capstone §2.1]) run on them with workgroup
// reductions, and P (bf16) is written over the row as 16-byte pieces, with
// the row's LSE. Bottom-right causal mask: key j visible to row i iff
// j <= i + Nk - Nq.
template <int NP>  // 8-score pieces per thread: NP * 8 * kThreads >= Nk
__global__ __launch_bounds__(kThreads) void naive_softmax_kernel(
    _Float16* __restrict__ S, float* __restrict__ LSE, int Nq, int Nk,
    bool causal) {
  __shared__ float red[kThreads / 64];
  const long rowid = blockIdx.x;  // (b * Hq + h) * Nq + i
  const int i = (int)(rowid % Nq);
  const int lim = causal ? min(Nk, i + (Nk - Nq) + 1) : Nk;  // visible keys
  _Float16* srow = S + rowid * Nk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float x[NP][8];
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    const int j0 = 8 * (tid + kThreads * c);
    f16x8 v8 = {};
    if (j0 < Nk) v8 = *reinterpret_cast<const f16x8*>(srow + j0);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[c][e] = (j0 + e < lim) ? (float)v8[e] : kNegInf;
  }
  auto block_reduce = [&](float v, bool is_max) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float u = __shfl_xor(v, o, 64);
      v = is_max ? fmaxf(v, u) : v + u;
    }
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int k = 1; k < kThreads / 64; ++k) r = is_max ? fmaxf(r, red[k]) : r + red[k];
    return r;
  };
  float m = kNegInf;
#pragma unroll
  for (int c = 0; c < NP; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, x[c][e]);
  m = block_reduce(m, true);
  const float mref = (m == kNegInf) ? 0.f : m;
  float l = 0.f;
#pragma unroll
  for (int c = 0; c < NP; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[c][e] = fast_exp2((x[c][e] - mref) * kLog2e);
      l += x[c][e];
    }
  l = block_reduce(l, false);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  __bf16* prow = reinterpret_cast<__bf16*>(srow);
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    const int j0 = 8 * (tid + kThreads * c);
    if (j0 < Nk) {
      bf16x8 p8;
#pragma unroll
      for (int e = 0; e < 8; ++e) p8[e] = (__bf16)(x[c][e] * inv);
      *reinterpret_cast<bf16x8*>(prow + j0) = p8;
    }
  }
  if (tid == 0 && LSE != nullptr) LSE[rowid] = l > 0.f ? m + __logf(l) : kNegInf;
}

// The same softmax with one wave per row (rows of up to 4096 keys): the
// row is read as 16-byte pieces of 8 scores (Nk is a multiple of 8, so rows
// are 16-byte aligned), max and sum are reduced inside the wave by lane
// exchanges (no barrier), and P goes back as 16-byte pieces. This keeps the
// kernel a plain stream of S in and P out.
template <int NC>  // 8-score pieces per lane: NC * 512 >= Nk
__global__ __launch_bounds__(kThreads) void naive_softmax_wave_kernel(
    _Float16* __restrict__ S, float* __restrict__ LSE, long rows, int Nq,
    int Nk, bool causal) {
  const int lane = threadIdx.x & 63;
  const long rowid = (long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (rowid >= rows) return;
  const int i = (int)(rowid % Nq);
  const int lim = causal ? min(Nk, i + (Nk - Nq) + 1) : Nk;  // visible keys
  _Float16* srow = S + rowid * Nk;
  float x[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j0 = 8 * (lane + 64 * c);
    f16x8 v8 = {};
    if (j0 < Nk) v8 = *reinterpret_cast<const f16x8*>(srow + j0);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[c][e] = (j0 + e < lim) ? (float)v8[e] : kNegInf;
  }
  float m = kNegInf;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, x[c][e]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float mref = (m == kNegInf) ? 0.f : m;
  float l = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[c][e] = fast_exp2((x[c][e] - mref) * kLog2e);
      l += x[c][e];
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  __bf16* prow = reinterpret_cast<__bf16*>(srow);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j0 = 8 * (lane + 64 * c);
    if (j0 < Nk) {
      bf16x8 p8;
#pragma unroll
      for (int e = 0; e < 8; ++e) p8[e] = (__bf16)(x[c][e] * inv);
      *reinterpret_cast<bf16x8*>(prow + j0) = p8;
    }
  }
  if (lane == 0 && LSE != nullptr) LSE[rowid] = l > 0.f ? m + __logf(l) : kNegInf;
}

// ----------------------------------------------------------- O = P V
// Workgroup: 128 rows (32 per wave) of one (batch, head); V streams through
// LDS in 64-key tiles and is read transposed (ds_read_b64_tr_b16) as the A
// operand of O^T = V^T P^T. Each wave's 32 x 64 tile of P comes in by
// direct loads too (whole 128-byte row segments), into four 1 KB blocks at
// a 1032-byte pitch: block b holds rows 8b .. 8b + 7, the 8-byte unit u of
// row 8b + j at unit 32 (u / 4) + 4 j + u % 4 of the block, so the P^T B
// operand (lane: row r32, keys 16j + 4h + 0..3 and + 8, the order the
// transposed V read delivers) is two 8-byte reads that meet no bank
// conflict.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void naive_pv_kernel(
    const __bf16* __restrict__ P, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, int B, int Hq, int Hkv, int Nq, int Nk) {
  using T = VTile64<D>;
  constexpr int kPPitch = 1032;
  __shared__ __attribute__((aligned(16))) char vl0[T::BYTES];
  __shared__ __attribute__((aligned(16))) char vl1[T::BYTES];
  __shared__ __attribute__((aligned(16))) char pl0[4][4 * kPPitch];
  __shared__ __attribute__((aligned(16))) char pl1[4][4 * kPPitch];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = lane >> 5, r32 = lane & 31, i16 = lane & 15;
  const int n_qt = (Nq + 127) / 128;
  const TileIdx ti = map_tile(blockIdx.x, n_qt, Hq, Hkv, B, false);
  const int hk = ti.hq / (Hq / Hkv);
  const long bh = (long)ti.b * Hq + ti.hq;
  const __bf16* Vh = V + ((long)ti.b * Hkv + hk) * Nk * D;
  const int row0 = ti.qt * 128 + 32 * w;
  const int row = row0 + r32;
  f32x16 o[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[mb][v] = 0.f;
  // transposed read offsets: rows 16j + 8e + 4h + i16/4 of the tile,
  // columns 2*(16*((lane>>4)&1) + 4*(i16&3)) bytes (+64 per 32 columns)
  const int tbase = T::row_off(4 * h + (i16 >> 2)) +
                    T::col_off(2 * (16 * ((lane >> 4) & 1) + 4 * (i16 & 3)));
  auto buf = [&](int i) -> lds_char* { return (lds_char*)(i ? vl1 : vl0); };
  auto pbuf = [&](int i) -> lds_char* { return (lds_char*)(i ? pl1[w] : pl0[w]); };
  // this lane's piece of the P tile: row 8b + (lane%16)/2, keys 8c .. 8c+7
  // with c = 2 (lane/16) + lane%2 (rows past Nq and keys past Nk are read
  // from a clamped place; their P is replaced by 0 below)
  const int pj = (lane & 15) >> 1, pc = 2 * (lane >> 4) + (lane & 1);
  auto load_p = [&](int tile, lds_char* dst) {
    const int key = min(64 * tile + 8 * pc, Nk - 8);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = min(row0 + 8 * b + pj, Nq - 1);
      g2lds_16B(P + (bh * Nq + r) * Nk + key, dst + b * kPPitch);
    }
  };
  const int pfrag = (r32 >> 3) * kPPitch + 32 * (r32 & 7) + 8 * h;
  const int nt = (Nk + 63) / 64;
  load64<D, T>(Vh, 0, Nk, buf(0), w, lane);
  load_p(0, pbuf(0));
  for (int t = 0; t < nt; ++t) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (t + 1 < nt) {
      load64<D, T>(Vh, 64 * (t + 1), Nk, buf((t + 1) & 1), w, lane);
      load_p(t + 1, pbuf((t + 1) & 1));
    }
    const lds_char* vp = buf(t & 1);
    const lds_char* pp = pbuf(t & 1) + pfrag;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {  // 16-key steps of the tile
      const int k0 = 64 * t + 16 * j4 + 4 * h;
      u32x2 lo = *(const __attribute__((address_space(3))) u32x2*)(pp + 256 * j4);
      u32x2 hi = *(const __attribute__((address_space(3))) u32x2*)(pp + 256 * j4 + 16);
      // keys past Nk (the ragged last tile; Nk is a multiple of 8) weigh 0
      if (k0 >= Nk) lo = u32x2{0u, 0u};
      if (k0 + 8 >= Nk) hi = u32x2{0u, 0u};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      const int rl = T::row_off(16 * j4), rh = T::row_off(16 * j4 + 8);
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
        const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(vp + tbase + rl + T::col_off(64 * mb)));
        const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(vp + tbase + rh + T::col_off(64 * mb)));
        const bf16x8 av = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        o[mb] = mfma_32x32x16_bf16(av, pb, o[mb]);
      }
    }
  }
  if (row < Nq) {
    __bf16* orow = O + (bh * Nq + row) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pr;
        pr[0] = pack_bf16x2(o[mb][4 * g], o[mb][4 * g + 1]);
        pr[1] = pack_bf16x2(o[mb][4 * g + 2], o[mb][4 * g + 3]);
        *reinterpret_cast<u32x2*>(orow + 32 * mb + 8 * g + 4 * h) = pr;
      }
  }
}

template <int D>
hipError_t launch(const NaiveArgs& a) {
  const long qblocks = (long)((a.Nq + 127) / 128) * a.Hq * a.B;
  _Float16* S = static_cast<_Float16*>(a.ws);
  hipLaunchKernelGGL((naive_scores_kernel<D>), dim3((unsigned)qblocks),
                     dim3(kThreads), 0, a.stream, static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k), S, a.B, a.Hq, a.Hkv, a.Nq,
                     a.Nk, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned rows = (unsigned)((long)a.B * a.Hq * a.Nq);
  const int np = (a.Nk + 8 * kThreads - 1) / (8 * kThreads);  // <= 8: Nk <= 16384
  const int nc = (a.Nk + 511) / 512;
  const unsigned wgrid = (rows + kThreads / 64 - 1) / (kThreads / 64);
  if (nc <= 1)
    hipLaunchKernelGGL((naive_softmax_wave_kernel<1>), dim3(wgrid), dim3(kThreads), 0,
                       a.stream, S, a.lse, (long)rows, a.Nq, a.Nk, a.causal);
  else if (nc <= 2)
    hipLaunchKernelGGL((naive_softmax_wave_kernel<2>), dim3(wgrid), dim3(kThreads), 0,
                       a.stream, S, a.lse, (long)rows, a.Nq, a.Nk, a.causal);
  else if (nc <= 4)
    hipLaunchKernelGGL((naive_softmax_wave_kernel<4>), dim3(wgrid), dim3(kThreads), 0,
                       a.stream, S, a.lse, (long)rows, a.Nq, a.Nk, a.causal);
  else if (nc <= 8)
    hipLaunchKernelGGL((naive_softmax_wave_kernel<8>), dim3(wgrid), dim3(kThreads), 0,
                       a.stream, S, a.lse, (long)rows, a.Nq, a.Nk, a.causal);
  else if (np <= 4)
    hipLaunchKernelGGL((naive_softmax_kernel<4>), dim3(rows), dim3(kThreads), 0,
                       a.stream, S, a.lse, a.Nq, a.Nk, a.causal);
  else
    hipLaunchKernelGGL((naive_softmax_kernel<8>), dim3(rows), dim3(kThreads), 0,
                       a.stream, S, a.lse, a.Nq, a.Nk, a.causal);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((naive_pv_kernel<D>), dim3((unsigned)qblocks), dim3(kThreads),
                     0, a.stream, reinterpret_cast<const __bf16*>(S),
                     static_cast<const __bf16*>(a.v), static_cast<__bf16*>(a.o),
                     a.B, a.Hq, a.Hkv, a.Nq, a.Nk);
  return hipGetLastError();
}

}  // namespace

size_t naive_workspace_bytes(int B, int Hq, int Nq, int Nk) {
  return (size_t)B * Hq * Nq * Nk * 2;
}

hipError_t launch_naive_bf16(const NaiveArgs& a) {
  return a.d == 128 ? launch<128>(a) : launch<64>(a);
}

}  // namespace fa
