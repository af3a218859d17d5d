// fa_device.h - device-side building blocks shared by the gfx950 kernels:
// vector types, MFMA wrappers, wave64 cross-lane helpers and the online
// softmax update on an MFMA score tile.
//
// Layout convention used by every prefill kernel (the "transposed" form):
// a wave computes S^T = K . Q^T with v_mfma_f32_32x32x*, so that in the
// 32x32 accumulator lane l holds the scores of query row (l % 32) against
// 16 of the 32 keys: key = 8*(v/4) + 4*(l/32) + (v%4) for accumulator
// element v. Row statistics (max, sum) are then almost entirely lane-local
// (the other 16 keys of the row sit in lane l ^ 32), and the same
// accumulator feeds the B operand of O^T += V^T . P^T without leaving
// registers. O^T keeps the row in the lane as well, so the per-row rescale
// of the online softmax is a per-lane multiply.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// Lazy rescale threshold in log2 units: the running maximum used as the
// exponent reference is only raised when a new score exceeds it by more
// than this, so exp2 arguments stay <= kTau (P <= 256, fine in fp32, bf16
// and e4m3) while O and l are rescaled only rarely. Exact: O and l always
// share the same reference.
constexpr float kTau = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}
__device__ __forceinline__ float fast_log2(float x) {
  return __builtin_amdgcn_logf(x);
}

// ------------------------------------------------ direct global -> LDS
typedef __attribute__((address_space(3))) char lds_char;

// One 16-byte piece per lane straight from global memory into LDS
// (global_load_lds_dwordx4): the 64 lanes of the instruction fill 1 KB of
// contiguous LDS starting at the wave's address l, with no VGPR staging.
__device__ __forceinline__ void g2lds_16B(const void* g, lds_char* l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l,
                                   16, 0, 0);
}
// The same direct loads (16 or 4 bytes per lane) written out as
// instructions, for loops that read LDS while their next tiles' direct
// loads are in flight: a direct load issued through the compiler's builtin
// counts there as an LDS access of unknown order, and the compiler then
// waits for every outstanding LDS read (lgkmcnt 0) wherever it needs one,
// so no fragment read can run ahead of the products that use it. Issued
// this way the loads are invisible to its wait counting: a kernel using
// them waits for them itself (a vmcnt wait before the barrier that
// publishes a tile), and the waits the compiler computes for its own loads
// can only become more conservative. M0 carries the wave's LDS base; the s_nop is the one
// wait state a direct load needs after M0 is written.
__device__ __forceinline__ void g2lds_16B_own(const void* g, lds_char* l) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)l);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0)
               : "memory");
}
__device__ __forceinline__ void g2lds_4B_own(const void* g, lds_char* l) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)l);
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(m0)
               : "memory");
}

// s_waitcnt vmcnt(0): the direct loads of this wave have reached LDS.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b,
                                                     f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b,
                                                    f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x2_f32(float a, float b,
                                                   f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// e4m3 x e4m3 (format code 0 for both operands), no block scaling.
__device__ __forceinline__ f32x16 mfma_32x32x64_e4m3(i32x8 a, i32x8 b,
                                                     f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0,
                                                         0, 0);
}
// fp4 e2m1 (format code 4, dwords 0-3 of a) x e4m3, no block scaling.
__device__ __forceinline__ f32x16 mfma_32x32x64_fp4_e4m3(i32x8 a, i32x8 b,
                                                         f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 0, 0, 0,
                                                         0, 0);
}

// ------------------------------------------------------- cross-lane ops
__device__ __forceinline__ float xor_lane(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}
// x[l] and x[l ^ 32] in every lane (v_permlane32_swap: lanes 32-63 of one
// copy trade places with lanes 0-31 of the other), reduced with max / add.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------- conversions
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};     // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
// Four fp32 -> four OCP e4m3 bytes, byte i = x_i (round to nearest even).
__device__ __forceinline__ uint32_t pack_e4m3x4(float x0, float x1, float x2,
                                                float x3) {
  // the first conversion fills the low half and keeps the high half of its
  // third operand, which the second conversion replaces: x0's bits serve
  // there, so the register needs no clearing first
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __float_as_int(x0), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}
// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against ones).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones,
                                         acc, false);
}
// acc + the four e4m3 values of a packed word.
__device__ __forceinline__ float add_e4m3x4(uint32_t w, float acc) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return acc + ((lo[0] + lo[1]) + (hi[0] + hi[1]));
}

// ------------------------------------------ interleaved LDS tile layout
// A row-major tile of ROWS rows x 128 bf16 in LDS as 1 KB blocks (one
// direct load instruction: 64 lanes x 16 B) at a pitch of 1 KB + 16 B, for
// tiles read by 16-byte rows and/or by the transpose read: block b holds
// rows 4b .. 4b + 3 with their chunks interleaved in 64-byte groups: chunk
// k = 4a + c of row 4b + j sits at byte 256a + 64j + 16c of the block.
//  * row reads: sixteen consecutive rows at one chunk are four blocks x four
//    rows; block b adds 16 b (mod 256) and row j adds 64 j, so the sixteen
//    16-byte pieces cover the 256 bytes of the banks once;
//  * transpose reads: a 32-lane half reads 64 contiguous bytes of each of
//    four consecutive rows 4b .. 4b + 3, which sit 64 B apart: again each
//    bank once.
// Both offsets stay one per-lane base plus compile-time constants (row_off
// is additive over multiples of 4 rows, chunk_off over the chunk's bit 0
// and col_off over multiples of 64 bytes).
template <int ROWS, int WAVES>
struct IlvTile {
  static constexpr int NB = ROWS / 4;
  static constexpr int PITCH = 1040;
  static constexpr int BYTES = NB * PITCH;
  static constexpr int BPW = NB / WAVES;  // blocks each of WAVES waves loads
  static __device__ __forceinline__ constexpr int row_off(int r) {
    return (r / 4) * PITCH + 64 * (r % 4);
  }
  static __device__ __forceinline__ constexpr int chunk_off(int k) {
    return 256 * (k / 4) + 16 * (k % 4);
  }
  static __device__ __forceinline__ constexpr int col_off(int x) {
    return 256 * (x / 64) + x % 64;
  }
  static __device__ __forceinline__ int block_row(int b, int lane) {
    return 4 * b + ((lane >> 2) & 3);
  }
  static __device__ __forceinline__ int lane_chunk(int lane) {
    return 4 * (lane >> 4) + (lane & 3);
  }
};

// ------------------------------------------------ workgroup -> tile map
// One workgroup computes one BM-row query tile of one (batch, query head).
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2), so the block id is remapped to give every XCD a contiguous range of
// logical tiles; logical order is (kv head, batch) group-major, so the
// query heads that share a KV head, and all their query tiles, run on one
// XCD and hit the same K/V lines in its L2, and the requests of a batch
// (whose key ranges may differ, as in the paged cache) are spread over the
// XCDs by KV head rather than handed out a few whole requests per XCD.
// Within a group, causal tiles go heaviest (longest key range) first.
struct TileIdx {
  int b, hq, qt;
};
__device__ __forceinline__ TileIdx map_tile(int bid, int n_qt, int Hq,
                                            int Hkv, int B, bool causal) {
  const int total = n_qt * Hq * B;
  int lid = bid;
  if ((total & 7) == 0) lid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int G = Hq / Hkv;
  const int per_group = n_qt * G;
  const int grp = lid / per_group;
  const int rem = lid - grp * per_group;
  const int rank = rem / G;
  TileIdx t;
  t.b = grp % B;
  t.hq = (grp / B) * G + (rem - rank * G);
  t.qt = causal ? (n_qt - 1 - rank) : rank;
  return t;
}

// ---------------------------------------------- online softmax on S^T
// State of one query row (one lane, mirrored in lane ^ 32).
struct RowState {
  float m;   // exponent reference in log2 units (-inf until a key is seen)
  float l;   // this lane's partial sum of P (its 16 of every 32 keys), fp32
  float lr;  // the same sum over P as rounded for the P.V product
};
// Why two sums: O is divided by lr, so the weights applied to V are the
// rounded P divided by their own sum, an exact convex combination (the
// rounding of P then only perturbs the weights, it cannot scale O);
// LSE = m + log2(l) uses the unrounded sum. Kernels whose P.V product is
// fp32 keep lr == l.

// Applies one key tile to the running state ([Capstone §2.2 steps 3-4]
// with the deferred normalisation of §4.2): s[] holds the raw scores of
// NKB 32-key blocks in the transposed accumulator layout (masked entries
// already -inf); c = scale * log2(e). On return s[] holds P = exp2(s*c -
// m_ref) and o[] (NMB blocks of O^T) and st.l are rescaled if the
// reference moved.
template <int NKB, int NMB>
__device__ __forceinline__ void online_softmax_tile(f32x16 (&s)[NKB],
                                                    f32x16 (&o)[NMB],
                                                    RowState& st, float c) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
  mx = max_halves(mx);
  const float mxs = mx * c;  // c > 0, so max commutes with the scaling
  const bool need = mxs > st.m + kTau;
  if (__any(need)) {
    const float mnew = fmaxf(st.m, mxs);
    const float alpha = (st.m == kNegInf) ? 0.f : fast_exp2(st.m - mnew);
    st.l *= alpha;
    st.lr *= alpha;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[mb][v] *= alpha;
    st.m = mnew;
  }
  const float mref = (st.m == kNegInf) ? 0.f : st.m;
  float sum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = fast_exp2(__builtin_fmaf(s[kb][v], c, -mref));
      s[kb][v] = p;
      sum += p;
    }
  st.l += sum;
}

// The same update split in parts, so that a caller can put independent MFMA
// work between them. tile_max: row max of a tile (masked entries -inf);
// move_reference: lazy move of the exponent reference for that max, l and
// lr rescaled, returning the factor O must be multiplied by (1 when the
// reference did not move). softmax_exp_pack: P = exp2(s*c - m_ref) summed
// into l, rounded to bf16 and packed in the PV operand order (block kb,
// 16-key step j, pairs), the rounded values summed into lr.
template <int NKB>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[NKB]) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
  return max_halves(mx);
}
__device__ __forceinline__ float move_reference(float mx, RowState& st,
                                                float c) {
  const float mxs = mx * c;  // c > 0, so max commutes with the scaling
  float alpha = 1.f;
  if (__any(mxs > st.m + kTau)) {
    const float mnew = fmaxf(st.m, mxs);
    alpha = (st.m == kNegInf) ? 0.f : fast_exp2(st.m - mnew);
    st.l *= alpha;
    st.lr *= alpha;
    st.m = mnew;
  }
  return alpha;
}

template <int NKB>
__device__ __forceinline__ void softmax_exp_pack(f32x16 (&s)[NKB],
                                                 RowState& st, float c,
                                                 uint32_t (&pw)[NKB][2][4]) {
  const float mref = (st.m == kNegInf) ? 0.f : st.m;
  float sum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = fast_exp2(__builtin_fmaf(s[kb][v], c, -mref));
      s[kb][v] = p;
      sum += p;
    }
  st.l += sum;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        pw[kb][j][t2] = pack_bf16x2(s[kb][8 * j + 2 * t2], s[kb][8 * j + 2 * t2 + 1]);
        st.lr = add_bf16x2(pw[kb][j][t2], st.lr);
      }
}

}  // namespace fa
