// fa_fwd_bf16.hip - exact attention forward, bf16 in / bf16 out, gfx950,
// for d = 64 (contiguous and paged K/V). At d = 128 the launchers below hand
// the call to fwd_bf16_pp_kernel (fa_fwd_bf16_pp.hip), which computes the
// same arithmetic in the same order with the two waves of each SIMD in
// opposite phases; this kernel interleaves each wave's products and vector
// work within one basic block instead.
//
// One workgroup (8 waves, one per CU) owns a 256-row query tile of one
// (batch, head) and streams the key/value range in 64-key tiles: the
// Q-outer / KV-inner order of [Capstone §4.1] with O, m, l held on chip and
// O divided by l once at the end ([Capstone §4.2]). Q K^T and P V run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; S and P never leave
// registers. Causal tiles above the diagonal are not visited
// ([Capstone §7.3 Q2]); the tiles that cross it are masked per element.
//
// Data flow per key tile (one barrier per tile):
//   global K, V -> LDS by direct loads (no VGPR staging), K two tiles ahead
//   in two buffers, V two tiles ahead in three
//   -> per wave (32 rows): S^T = K Q^T (Q lives in VGPRs), online softmax,
//      P^T packed to bf16 in registers, O^T += V^T P^T with the V^T operand
//      produced by gfx950's LDS transpose read. S(t+1) is computed while
//      P(t) is formed.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kBM = 256;       // query rows per workgroup (32 per wave)
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 512;  // 8 waves: one workgroup per CU
constexpr int kWaves = kThreads / 64;
constexpr int kVStages = 3;    // V buffers: V is loaded kVStages-1 tiles ahead

// ------------------------------------------------------------ LDS layout
// K and V tiles (64 rows x d) arrive by direct global->LDS loads
// (global_load_lds_dwordx4): one instruction moves 64 lanes x 16 B into 1 KB
// of contiguous LDS, so a tile is stored as 1 KB blocks of RPB rows, placed
// at a pitch of 1 KB + 16 B (+ 32 B for V at d = 64). Which rows share a
// block is chosen so that every fragment read is conflict free and is one
// per-lane base plus a compile-time offset:
//  * K: block b holds rows b, b + NB, b + 2NB, ... The S^T = K Q^T A operand
//    (16 B per lane, 16 consecutive keys at one chunk) then touches 16
//    different blocks, whose pitch spreads them over the 16 bank groups.
//  * V: block (r % 4) * NB/4 + r / (4 RPB) holds row r at slot (r/4) % RPB.
//    The O^T = V^T P^T A operand is read with ds_read_b64_tr_b16: in each
//    16-lane group lane j fetches 4 consecutive d of key row kbase + j/4 and
//    the transpose hands lane i the keys kbase..kbase+3 at column dbase + i
//    (the k-major V^T fragment the MFMA needs). A 32-lane half reads rows
//    kbase..kbase+3, which sit in blocks 64 B apart modulo 256 B.
template <int D>
struct Lay {
  static constexpr int CPR = D / 8;             // 16 B chunks per row
  static constexpr int RPB = 1024 / (2 * D);    // rows per 1 KB block
  static constexpr int NB = kBN / RPB;          // blocks per tile
  static constexpr int KPITCH = 1040;
  static constexpr int VPITCH = D == 128 ? 1040 : 1056;
  static constexpr int K_BYTES = NB * KPITCH;
  static constexpr int V_BYTES = NB * VPITCH;
  static constexpr int BPW = NB / kWaves;       // blocks each wave loads
};

// Where K and V come from. Contiguous: [B, Hkv, Nk, d]. Paged (the
// chunked prefill of [FA3-paged §3.2]): the cache of request b is
// seq_lens[b] tokens in 16-token pages of a [num_pages, 16, Hkv, d] pool,
// logical page p at physical page block_table[b, p]; the Nq queries are the
// request's last Nq positions (bottom-right causal alignment).
struct PagedKV {
  const int32_t* bt;  // [B, max_pages]
  const int32_t* sl;  // [B]
  int max_pages, num_pages;
};
constexpr int kMaxPagesLds = 8192;  // page-table entries a workgroup stages
constexpr int kMaxRankB = 256;      // batches up to this size run longest first
static_assert(kMaxRankB <= kThreads, "one request length per thread");

template <int D, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kThreads, 512 / kThreads) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, __bf16* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk,
    float c, PagedKV pk) {
  using T = Lay<D>;
  // Four separate arrays, always selected by a compile-time index: the
  // compiler can then tell that reading one buffer does not depend on the
  // direct loads still in flight into another, and waits only where a
  // buffer is actually reused.
  __shared__ __attribute__((aligned(16))) char k_lds0[T::K_BYTES];
  __shared__ __attribute__((aligned(16))) char k_lds1[T::K_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds0[T::V_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds1[T::V_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds2[kVStages > 2 ? T::V_BYTES : 16];
  auto kbuf = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)k_lds0;
    else return (lds_char*)k_lds1;
  };
  auto vbuf = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)v_lds0;
    else if constexpr (decltype(b)::value == 1) return (lds_char*)v_lds1;
    else return (lds_char*)v_lds2;
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
  // The batch index this workgroup serves. For the paged cache, whose
  // requests differ in length, the logical index is a rank: requests are
  // taken longest first (ties by index), so the longest workgroups start
  // first and the grid ends without a ragged tail. Each workgroup ranks the
  // lengths itself (a batch of at most kMaxRankB requests; larger batches
  // keep their order).
  int bq = ti.b;
  if constexpr (PAGED) {
    if (B <= kMaxRankB) {
      __shared__ int lens[kMaxRankB];
      __shared__ int ranked;
      const int cap = pk.max_pages * 16;
      if (tid < B) lens[tid] = max(0, min(pk.sl[tid], cap));
      __syncthreads();
      if (tid < B) {
        const int lr = lens[tid];
        int rank = 0;
        for (int r2 = 0; r2 < B; ++r2) {
          const int l2 = lens[r2];
          rank += (l2 > lr) || (l2 == lr && r2 < tid);
        }
        if (rank == ti.b) ranked = tid;
      }
      __syncthreads();
      bq = ranked;
    }
  }
  const long qbase = (long)(bq * Hq + ti.hq) * Nq * D;
  // keys of this request; for the paged cache its length, and the page
  // table staged in LDS (ids outside the pool are replaced by 0 and turn
  // the request's output to NaN)
  __shared__ int page_ids[PAGED ? kMaxPagesLds : 1];
  __shared__ int page_bad;
  int nk = Nk;
  if constexpr (PAGED) {
    nk = max(0, min(pk.sl[bq], pk.max_pages * 16));
    const int np = (nk + 15) / 16;
    if (tid == 0) page_bad = 0;
    __syncthreads();
    bool bad = false;
    for (int i = tid; i < np; i += kThreads) {
      const int id = pk.bt[(long)bq * pk.max_pages + i];
      const bool ok = id >= 0 && id < pk.num_pages;
      page_ids[i] = ok ? id : 0;
      bad |= !ok;
    }
    if (bad) page_bad = 1;
    __syncthreads();
  }
  // contiguous: the head's K/V; paged: the pool plus this head's offset
  // within a token row (rows of a page are Hkv * d apart)
  const long kv_head = PAGED ? (long)hk * D : (long)(bq * Hkv + hk) * Nk * D;
  const __bf16* Kh = K + kv_head;
  const __bf16* Vh = V + kv_head;
  const long tok_stride = PAGED ? (long)Hkv * D : D;
  const int off = nk - Nq;  // bottom-right causal alignment
  int kend = nk;
  if (CAUSAL) kend = min(nk, min(q0 + kBM, Nq) + off);
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

  // ---- direct loads. Wave w fills blocks w, w + kWaves, ...; lane l moves chunk
  // l % CPR of the block's slot l / CPR. Full tiles use precomputed lane
  // offsets; on the ragged last tile rows past Nk are clamped to the last
  // key (their scores are masked, their P is 0).
  const int slot = lane / T::CPR, chunk = lane % T::CPR;
  auto k_row = [&](int b) { return b + T::NB * slot; };
  auto v_row = [&](int b) {
    return 4 * T::RPB * (b % (T::NB / 4)) + 4 * slot + b / (T::NB / 4);
  };
  int koff[T::BPW], voff[T::BPW];
#pragma unroll
  for (int i = 0; i < T::BPW; ++i) {
    koff[i] = k_row(w + kWaves * i) * D + 8 * chunk;
    voff[i] = v_row(w + kWaves * i) * D + 8 * chunk;
  }
  // Paged cache, full tiles: a tile is 4 whole pages, so each of this
  // lane's rows lies in a fixed page of the tile at a fixed offset inside
  // it; per tile only the page ids change. The page's element offset is
  // one 32 x 32 -> 64-bit multiply (ids are checked non-negative).
  int kpg[T::BPW], kpo[T::BPW], vpg[T::BPW], vpo[T::BPW];
  const uint32_t page_elems = 16u * (uint32_t)tok_stride;
#pragma unroll
  for (int i = 0; i < T::BPW; ++i) {
    const int rk = k_row(w + kWaves * i), rv = v_row(w + kWaves * i);
    kpg[i] = rk >> 4;
    kpo[i] = (rk & 15) * (int)tok_stride + 8 * chunk;
    vpg[i] = rv >> 4;
    vpo[i] = (rv & 15) * (int)tok_stride + 8 * chunk;
  }
  auto page_off = [&](int n0, int pg) -> long {
    return (long)((uint64_t)(uint32_t)page_ids[(n0 >> 4) + pg] * page_elems);
  };
  // element offset of tile-relative row r of tile n0 (rows past the keys
  // clamped to the last key: their scores are masked, their P is 0)
  auto row_elem = [&](int n0, int r) -> long {
    const int t = n0 + min(r, nk - 1 - n0);
    if constexpr (PAGED)
      return ((long)page_ids[t >> 4] * 16 + (t & 15)) * tok_stride;
    else
      return (long)t * D;
  };
  auto issue_k = [&](int tile, auto buf) {
    const int n0 = tile * kBN;
    lds_char* dst = kbuf(buf) + w * T::KPITCH;
    if (PAGED && n0 + kBN <= nk) {
#pragma unroll
      for (int i = 0; i < T::BPW; ++i)
        g2lds_16B_own(Kh + page_off(n0, kpg[i]) + kpo[i], dst + kWaves * i * T::KPITCH);
    } else if (!PAGED && n0 + kBN <= nk) {
      const __bf16* src = Kh + (long)n0 * D;
#pragma unroll
      for (int i = 0; i < T::BPW; ++i)
        g2lds_16B_own(src + koff[i], dst + kWaves * i * T::KPITCH);
    } else {
#pragma unroll
      for (int i = 0; i < T::BPW; ++i)
        g2lds_16B_own(Kh + row_elem(n0, k_row(w + kWaves * i)) + 8 * chunk,
                  dst + kWaves * i * T::KPITCH);
    }
  };
  auto issue_v = [&](int tile, auto buf) {
    const int n0 = tile * kBN;
    lds_char* dst = vbuf(buf) + w * T::VPITCH;
    if (PAGED && n0 + kBN <= nk) {
#pragma unroll
      for (int i = 0; i < T::BPW; ++i)
        g2lds_16B_own(Vh + page_off(n0, vpg[i]) + vpo[i], dst + kWaves * i * T::VPITCH);
    } else if (!PAGED && n0 + kBN <= nk) {
      const __bf16* src = Vh + (long)n0 * D;
#pragma unroll
      for (int i = 0; i < T::BPW; ++i)
        g2lds_16B_own(src + voff[i], dst + kWaves * i * T::VPITCH);
    } else {
#pragma unroll
      for (int i = 0; i < T::BPW; ++i)
        g2lds_16B_own(Vh + row_elem(n0, v_row(w + kWaves * i)) + 8 * chunk,
                  dst + kWaves * i * T::VPITCH);
    }
  };

  // ---- per-lane fragment bases
  const int kfrag = (r32 % T::NB) * T::KPITCH + (r32 / T::NB) * (2 * D) + 16 * h;
  const int i16 = lane & 15, e_l = i16 >> 2;
  const int vfrag = e_l * (T::NB / 4) * T::VPITCH + h * (2 * D) +
                    (16 * ((lane >> 4) & 1) + 4 * (i16 & 3)) * 2;
  // S^T = K Q^T for the two 32-key blocks of a tile (two independent
  // accumulation chains, interleaved)
  auto qk = [&](auto buf, f32x16 (&s)[2]) {
    const lds_char* kp = kbuf(buf) + kfrag;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
    for (int sd = 0; sd < D / 16; ++sd)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *(const __attribute__((address_space(3))) bf16x8*)(
            kp + kb * (32 / T::NB) * (2 * D) + 32 * sd);
        s[kb] = mfma_32x32x16_bf16(a, qf[sd], s[kb]);
      }
  };
  auto skip_tile = [&](int tile) {
    return CAUSAL && (tile * kBN > wrow0 + 31 + off);
  };

  // Two passes over the key tiles, of which the second almost never runs.
  // The exponent reference only keeps P = 2^(S c - m) inside the range of
  // fp32 and bf16: any reference gives the same softmax. The first pass
  // fixes it at the row maximum of the first key tile and never moves it,
  // so a tile needs no row maximum, no reference test and no rescaling of
  // O (about 30 VALU instructions per tile and wave fewer). A row that
  // sees anything sees key 0, so every such row has a finite reference
  // after that tile. Scores that later rise more than ~2^7 above it make
  // P, l or O overflow; the pass then ends with a non-finite l or O in
  // some lane, and the workgroup runs the tiles again with the exact lazy
  // reference of the second pass (moved when a tile's maximum passes it by
  // kTau, O rescaled then), from a clean state.
  constexpr std::integral_constant<int, 0> B0{};
  constexpr std::integral_constant<int, 1> B1{};
  constexpr std::integral_constant<int, 2> B2{};
  __shared__ int redo;
  auto run = [&](auto fixed_ref) {
    constexpr bool FIXED = decltype(fixed_ref)::value;
    // ---- prologue: K(0), V(0), K(1) (and V(1) with three V buffers) in
    // flight; S(0)
    if (nt > 0) {
      issue_k(0, B0);
      issue_v(0, B0);
      if (nt > 1) issue_k(1, B1);
      if (kVStages > 2 && nt > 1) issue_v(1, B1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sc[2];
    // row max of the next tile's scores, taken where S is formed (beside
    // the P.V products of the previous tile); a tile that needs masking
    // takes its max again after the mask
    float mx_next = kNegInf;
    if (nt > 0 && !skip_tile(0)) {
      qk(B0, sc);
      mx_next = tile_max<2>(sc);
    }
    __syncthreads();  // K buffer 0 is refilled below

    // One key tile: S(t) arrives in sc; S(t+1) is computed into sn while
    // P(t) is formed. Tiles are taken in pairs with the two score buffers
    // swapping roles, so no tile ends with a register copy.
    // `par` is t % 2 and `vst` t % kVStages as compile-time indices.
    auto step = [&](int t, auto par, auto vst, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      constexpr int P = decltype(par)::value;
      constexpr int VS = decltype(vst)::value;
      constexpr std::integral_constant<int, P> cur{};
      constexpr std::integral_constant<int, 1 - P> nxt{};
      constexpr std::integral_constant<int, VS> vcur{};
      constexpr std::integral_constant<int, (VS + kVStages - 1) % kVStages> vnew{};
      const int n0 = t * kBN;
      // K runs two tiles ahead, V kVStages - 1: both target buffers were
      // last read before the previous barrier.
      const bool more_k = t + 2 < nt;
      const bool more_v = t + kVStages - 1 < nt;
      if (more_k) issue_k(t + 2, cur);
      if (more_v) issue_v(t + kVStages - 1, vnew);
      const bool do_t = !skip_tile(t);
      if (do_t) {
        // mask the ragged end of the key range and the causal diagonal
        const bool need_mask =
            (n0 + kBN > nk) || (CAUSAL && n0 + kBN - 1 > wrow0 + off);
        if (need_mask) {
          const int lim = CAUSAL ? min(nk - 1, row + off) : nk - 1;
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
          // rescale O before the MFMA work below, so that the S(t+1)
          // product and the P(t) arithmetic share one branch-free block
          if (!FIXED && __any(alpha != 1.f)) {
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
              for (int v = 0; v < 16; ++v) o[mb][v] *= alpha;
          }
        }
        uint32_t pw[2][2][4];
        // S(t+1) on the matrix cores while P(t) is formed on the VALU. Run
        // without a branch (so both sit in one basic block and
        // interleave): past the last tile, or beyond this wave's causal
        // rows, the result is never read, and the K buffer it reads is not
        // being written.
        // raised issue priority while this wave feeds the matrix cores:
        // the other wave on the SIMD (a wave of this workgroup: the 83 KB
        // of LDS leave room for one workgroup per CU) fills in with its
        // VALU work
        __builtin_amdgcn_s_setprio(1);
        qk(nxt, sn);
        softmax_exp_pack<2>(sc, st, c, pw);
        // O^T += V^T P^T, 16 keys per MFMA: lane half h contracts keys
        // 32kb + 16j + 4h + {0..3} (items 0..3) and +8 (items 4..7)
        const lds_char* vp0 = vbuf(vcur) + vfrag;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            u32x4 pv = {pw[kb][j][0], pw[kb][j][1], pw[kb][j][2], pw[kb][j][3]};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pv);
            const int rb = 32 * kb + 16 * j;              // multiple of 16
            const int vimm = (rb / (4 * T::RPB)) * T::VPITCH +
                             ((rb / 4) % T::RPB) * (2 * D);
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb) {
              const lds_char* vp = vp0 + vimm + 64 * mb;
              const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                  (__attribute__((address_space(3))) bf16x4*)(vp));
              const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                  (__attribute__((address_space(3))) bf16x4*)(vp + 2 * (2 * D)));
              const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              o[mb] = mfma_32x32x16_bf16(a, pb, o[mb]);
            }
          }
        if (!FIXED) mx_next = tile_max<2>(sn);
        // LLVM's preset interleave 0 (LDS reads among the products) on
        // this block: -1.4 to -2.1 % on the long causal prefill, neutral
        // without the mask, +3.6 % with the paged loads, so not there
        if constexpr (!PAGED) __builtin_amdgcn_iglp_opt(0);
        __builtin_amdgcn_s_setprio(0);
      }
      // tile t+1 needs K(t+2) and V(t+1), so only the V(t+2) loads just
      // issued (the last BPW in flight) could stay pending; the barrier's
      // workgroup fence then waits for the wave's remaining direct loads
      // as well, so every load has this tile's compute time to land
      if (kVStages > 2 && more_v) __builtin_amdgcn_s_waitcnt(0x0F70 | T::BPW);
      else wait_vm0();
      __syncthreads();
    };
    f32x16 sb[2];
    if constexpr (kVStages == 2) {
      for (int t = 0; t < nt; t += 2) {
        step(t, B0, B0, sc, sb);
        if (t + 1 < nt) step(t + 1, B1, B1, sb, sc);
      }
    } else {
      for (int t = 0; t < nt; t += 6) {
        step(t, B0, B0, sc, sb);
        if (t + 1 < nt) step(t + 1, B1, B1, sb, sc);
        if (t + 2 < nt) step(t + 2, B0, B2, sc, sb);
        if (t + 3 < nt) step(t + 3, B1, B0, sb, sc);
        if (t + 4 < nt) step(t + 4, B0, B1, sc, sb);
        if (t + 5 < nt) step(t + 5, B1, B2, sb, sc);
      }
    }
  };
  if (tid == 0) redo = 0;
  run(std::true_type{});
  {
    // inf or NaN anywhere in this lane's l, lr or O shows up in the sum
    float chk = st.l + st.lr;
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
    st = RowState{kNegInf, 0.f, 0.f};
    run(std::false_type{});
  }

  // ---- epilogue: O = O^T / lr, LSE = ln 2 * (m + log2 l)
  const float ltot = sum_halves(st.l);
  const float lrtot = sum_halves(st.lr);
  if (row < Nq) {
    const bool live = ltot > 0.f;
    float inv = live ? 1.f / lrtot : 0.f;
    bool nan_out = false;
    if constexpr (PAGED) nan_out = page_bad != 0;
    if (nan_out) inv = __builtin_nanf("");
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
      LSE[(long)(bq * Hq + ti.hq) * Nq + row] =
          nan_out ? __builtin_nanf("")
                  : (live ? (st.m + fast_log2(ltot)) * kLn2 : kNegInf);
  }
}

template <int D, bool CAUSAL, bool PAGED>
hipError_t launch(const FwdArgs& a, const PagedKV& pk) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long blocks = (long)n_qt * a.Hq * a.B;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, PAGED>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, a.stream,
                     static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v),
                     static_cast<__bf16*>(a.o), a.lse, a.B, a.Hq, a.Hkv, a.Nq,
                     a.Nk, a.scale * kLog2e, pk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  const PagedKV none{nullptr, nullptr, 0, 0};
  if (a.d == 128) return launch_fwd_bf16_pp(a);
  return a.causal ? launch<64, true, false>(a, none) : launch<64, false, false>(a, none);
}

hipError_t launch_paged_prefill_bf16(const FwdArgs& a, const int32_t* bt,
                                     const int32_t* sl, int max_pages,
                                     int num_pages) {
  if (a.d == 128) return launch_paged_prefill_bf16_pp(a, bt, sl, max_pages, num_pages);
  const PagedKV pk{bt, sl, max_pages, num_pages};
  return a.causal ? launch<64, true, true>(a, pk) : launch<64, false, true>(a, pk);
}

}  // namespace fa
