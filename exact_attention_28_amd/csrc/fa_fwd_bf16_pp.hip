// fa_fwd_bf16_pp.hip - exact attention forward, bf16, d = 128, gfx950: the
// two waves of each SIMD in opposite phases. K/V contiguous, or a paged
// cache (the chunked prefill of [FA3-paged §3.2]).
//
// The method is the bf16 forward's ([Capstone §4.1] Q-outer / KV-inner
// order, online softmax of §2.2 with the deferred 1/l of §4.2, causal tiles
// above the diagonal skipped per §7.3 Q2): one workgroup of 8 waves owns a
// 256-row query tile (32 rows a wave), K and V arrive in 64-key tiles by
// direct global->LDS loads, S^T = K Q^T and O^T += V^T P^T run on
// v_mfma_f32_32x32x16_bf16, P is rounded to bf16 in registers and O is
// divided by the sum of the rounded P at the end (LSE from the fp32 sum).
//
// What differs is the order of the work. Per key tile t a wave has a
// matrix phase M(t) (the 16 products of S(t) and the 16 of P(t-1).V(t-1))
// and a vector phase X(t) (mask, exp2, sums, rounding of S(t) into P(t)).
// Waves 0-3 run M(t), X(t), M(t+1), ... and waves 4-7 the same one phase
// later, with a workgroup barrier between phases, so while one wave of a
// SIMD (waves w and w + 4 share one) keeps the matrix core busy the other
// issues its vector work. The matrix phase is written out as inline asm
// (fa_pp_asm.h): its LDS fragments are read two products ahead of use with
// exact waits, which a compiler schedule does not give, and without which
// a phase made only of products waits on LDS latency at every product.
//
// Slots (one phase between two barriers), for a workgroup with nt tiles:
//   slot 2t:     waves 0-3 M(t),   waves 4-7 X(t-1)
//   slot 2t + 1: waves 0-3 X(t),   waves 4-7 M(t)
// for t = 0 .. nt (M(nt) is the last P.V product only). K(t) is read in
// slots 2t and 2t+1, V(t) in 2t+2 and 2t+3. K sits in two LDS buffers and
// V in three. Each group issues its share of the direct loads just before
// its own vector phase: the following waves K(u+1) at slot 2u, the leading
// waves V(u+1) at slot 2u+1, into buffers freed by the previous barrier;
// K(u+1) has landed by the end of slot 2u+1 and V(u+1) by the end of slot
// 2u+3. A wave raises its issue priority during its vector phase, so that
// the other wave's products fill the gaps between its vector instructions
// (measured faster than raising it for the products, or not at all).
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_pp_asm.h"

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kBM = 256;        // query rows per workgroup (32 per wave)
constexpr int kBN = 64;         // keys per tile
constexpr int kThreads = 512;   // 8 waves: one workgroup per CU
constexpr int kWaves = 8;
constexpr int kPitch = 1040;    // 1 KB direct-load block + 16 B
constexpr int kNB = 16;         // 1 KB blocks per 64 x 128 bf16 tile
constexpr int kRPB = 4;         // tile rows per block
constexpr int kLPW = kNB / 4;   // blocks each loading wave moves per tile
constexpr int kTileBytes = kNB * kPitch;
constexpr int kKBufs = 2, kVBufs = 3;

// Where K and V come from when PAGED: the cache of request b is
// seq_lens[b] tokens in 16-token pages of a [num_pages, 16, Hkv, d] pool,
// logical page p at physical page block_table[b, p]; the Nq queries are the
// request's last Nq positions (bottom-right causal alignment).
struct PagedCache {
  const int32_t* bt;  // [B, max_pages]
  const int32_t* sl;  // [B]
  int max_pages, num_pages;
};
constexpr int kMaxPagesLds = 8192;  // page-table entries a workgroup stages
constexpr int kMaxRankB = 256;      // batches up to this size run longest first
static_assert(kMaxRankB <= kThreads, "one request length per thread");

// LDS layout of a tile (as in the other bf16 forward): K block b holds
// rows b, b + 16, b + 32, b + 48 (conflict-free 16-byte row reads of 16
// consecutive keys); V block (r % 4) * 4 + r / 16 holds row r at slot
// (r / 4) % 4 (conflict-free ds_read_b64_tr_b16 of four consecutive rows).
__device__ __forceinline__ int k_row(int b, int slot) { return b + kNB * slot; }
__device__ __forceinline__ int v_row(int b, int slot) {
  return 4 * kRPB * (b % (kNB / 4)) + 4 * slot + b / (kNB / 4);
}

// A 16-byte direct load (global_load_lds_dwordx4) addressed as a scalar
// base plus a per-lane 32-bit byte offset (the SADDR form): a full tile's
// base is wave-uniform, so with each lane's offset kept in a register the
// loads need no vector address arithmetic. M0 carries the wave's LDS
// destination; the s_nop is the one wait state a direct load needs after
// M0 is written. Issued as an instruction of its own, the load is invisible
// to the compiler's wait counting: the kernel waits for it (vmcnt) before
// the barrier that publishes the tile.
__device__ __forceinline__ void g2lds_16B_sbase(const void* base, uint32_t off,
                                                lds_char* l) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)l);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "{m0}"(m0)
               : "memory");
}

template <bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_pp_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, __bf16* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk,
    float c, PagedCache pk) {
  __shared__ __attribute__((aligned(16))) char lds[(kKBufs + kVBufs) * kTileBytes];
  __shared__ int redo;
  const uint32_t lds0 = (uint32_t)(size_t)(lds_char*)lds;
  const uint32_t kbase = lds0, vbase = lds0 + kKBufs * kTileBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2;  // 0: waves 0-3 lead, 1: waves 4-7 follow
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
  const long qbase = (long)(bq * Hq + ti.hq) * Nq * kD;
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
  const long kv_head = PAGED ? (long)hk * kD : (long)(bq * Hkv + hk) * Nk * kD;
  const __bf16* Kh = K + kv_head;
  const __bf16* Vh = V + kv_head;
  const long tok_stride = PAGED ? (long)Hkv * kD : kD;
  const uint32_t page_elems = 16u * (uint32_t)tok_stride;
  const int off = nk - Nq;  // bottom-right causal alignment
  int kend = nk;
  if (CAUSAL) kend = min(nk, min(q0 + kBM, Nq) + off);
  const int nt = kend > 0 ? (kend + kBN - 1) / kBN : 0;

  // Q fragments (B operand of S^T = K Q^T): row r32 of the wave's rows,
  // d = 16 sd + 8 h + (0..7)
  const int wrow0 = q0 + w * 32;
  const int row = wrow0 + r32;
  const int rowc = min(row, Nq - 1);
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(Q + qbase + (long)rowc * kD + 16 * s + 8 * h);

  auto kbuf = [&](int t) __attribute__((always_inline)) { return kbase + (uint32_t)((t % kKBufs) * kTileBytes); };
  auto vbuf = [&](int t) __attribute__((always_inline)) { return vbase + (uint32_t)((t % kVBufs) * kTileBytes); };

  // ---- direct loads: K by the four following waves, V by the four leading
  // ones (each just before its vector phase); wave w fills blocks w % 4,
  // w % 4 + 4, + 8, + 12 of a tile; lane l moves 16-byte chunk l % 16 of
  // the block's slot l / 16.
  // Full tiles: a scalar tile base plus each lane's fixed byte offset. The
  // ragged last tile clamps rows past the keys to the last key (their
  // scores are masked, their P is 0).
  const int fw = w & 3;
  const int slot = lane >> 4, chunk = lane & 15;
  // The four rows a lane moves are tile rows k_row(fw + 4i, slot) =
  // fw + 16 slot + 4i of K and v_row(fw + 4i, slot) = 16 fw + 4 slot + i of
  // V: one per-lane row plus a step of 4 (K) or 1 (V) rows per load. In a
  // paged cache a full tile is four whole pages, and these rows lie in one
  // of them (K: page `slot` of the tile, V: page `fw`).
  const int krow0 = k_row(fw, slot), vrow0 = v_row(fw, slot);
  constexpr int kStepK = 4, kStepV = 1;  // rows between a lane's loads
  auto issue = [&](const __bf16* src, int row0, int step, int page, int tile,
                   uint32_t buf) __attribute__((always_inline)) {
    const int n0 = tile * kBN;
    if (!PAGED && n0 + kBN <= nk) {
      const __bf16* base = src + (long)n0 * kD;
      const uint32_t ofs = (uint32_t)(row0 * kD + 8 * chunk) * 2u;
#pragma unroll
      for (int i = 0; i < kLPW; ++i)
        g2lds_16B_sbase(base + (long)i * step * kD, ofs,
                        (lds_char*)(size_t)(buf + (fw + 4 * i) * kPitch));
    } else if (PAGED && n0 + kBN <= nk) {
      const __bf16* base =
          src + (long)((uint64_t)(uint32_t)page_ids[(n0 >> 4) + page] * page_elems) +
          (long)(row0 & 15) * tok_stride + 8 * chunk;
#pragma unroll
      for (int i = 0; i < kLPW; ++i)
        g2lds_16B_own(base + (long)i * step * tok_stride,
                      (lds_char*)(size_t)(buf + (fw + 4 * i) * kPitch));
    } else {
      // the ragged last tile: rows past the keys clamped to the last key
      // (their scores are masked, their P is 0); paged: token t of the
      // request sits at row t % 16 of page page_ids[t / 16]
#pragma unroll
      for (int i = 0; i < kLPW; ++i) {
        const int t = n0 + min(row0 + i * step, nk - 1 - n0);
        long e;
        if constexpr (PAGED)
          e = ((long)page_ids[t >> 4] * 16 + (t & 15)) * tok_stride;
        else
          e = (long)t * kD;
        g2lds_16B_own(src + e + 8 * chunk,
                      (lds_char*)(size_t)(buf + (fw + 4 * i) * kPitch));
      }
    }
  };
  auto issue_all = [&](int tile, auto which) __attribute__((always_inline)) {
    // which: 0 both (the prologue), 1 K, 2 V
    constexpr int WH = decltype(which)::value;
    if (WH != 2) issue(Kh, krow0, kStepK, slot, tile, kbuf(tile));
    if (WH != 1) issue(Vh, vrow0, kStepV, fw, tile, vbuf(tile));
  };

  // per-lane fragment bases within a tile
  const uint32_t kfrag = (r32 % kNB) * kPitch + (r32 / kNB) * (2 * kD) + 16 * h;
  const int i16 = lane & 15, e_l = i16 >> 2;
  const uint32_t vfrag = e_l * (kNB / 4) * kPitch + h * (2 * kD) +
                         (16 * ((lane >> 4) & 1) + 4 * (i16 & 3)) * 2;

  auto skip_tile = [&](int t) __attribute__((always_inline)) { return CAUSAL && (t * kBN > wrow0 + 31 + off); };

  f32x16 o[4];
  f32x16 sc[2];
  u32x4 pp[4];  // packed bf16 P of the last X phase, per 16-key step
  RowState st;

  // matrix phase M(t): S(t) if tile t is this wave's, P(t-1).V(t-1) if
  // tile t-1 was. One asm statement for every case, so that O stays in the
  // same registers throughout: at t = 0 P is zero and the V buffer it
  // meets was cleared in the prologue (0 * 0 adds nothing, whatever the
  // inputs hold), and past this wave's last tile the scores are computed
  // from whatever the K buffer holds and never read.
  auto matrix_phase = [&](int t) __attribute__((always_inline)) {
    const bool do_s = t < nt && !skip_tile(t);
    const bool do_pv = t >= 1 && !skip_tile(t - 1);
    if (!(do_s || do_pv)) return;
    const uint32_t ka = kbuf(t) + kfrag;
    const uint32_t va = vbuf(t + kVBufs - 1) + vfrag;  // V(t-1)
    asm volatile(PP_ASM_BOTH
                 : [o0] "+v"(o[0]), [o1] "+v"(o[1]), [o2] "+v"(o[2]), [o3] "+v"(o[3]),
                   [s0] "=&v"(sc[0]), [s1] "=&v"(sc[1])
                 : [q0] "v"(qf[0]), [q1] "v"(qf[1]), [q2] "v"(qf[2]), [q3] "v"(qf[3]),
                   [q4] "v"(qf[4]), [q5] "v"(qf[5]), [q6] "v"(qf[6]), [q7] "v"(qf[7]),
                   [p0] "v"(pp[0]), [p1] "v"(pp[1]), [p2] "v"(pp[2]), [p3] "v"(pp[3]),
                   [ka] "v"(ka), [va] "v"(va)
                 : "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247",
                   "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255",
                   "memory");
  };

  // vector phase X(t): mask, (first tile or exact pass) reference and
  // rescale, P = exp2(S c - m) summed, rounded and packed for M(t+1)
  auto vector_phase = [&](int t, auto fixed_ref) __attribute__((always_inline)) {
    constexpr bool FIXED = decltype(fixed_ref)::value;
    if (t >= nt || skip_tile(t)) return;
    __builtin_amdgcn_s_setprio(1);
    const int n0 = t * kBN;
    // the rest of the phase, written out in both branches below so that
    // the masked scores never need a second set of registers
    auto finish = [&]() __attribute__((always_inline)) {
      if (!FIXED || t == 0) {
        const float alpha = move_reference(tile_max<2>(sc), st, c);
        if (!FIXED && __any(alpha != 1.f)) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[mb][v] *= alpha;
        }
      }
      uint32_t pw[2][2][4];
      softmax_exp_pack<2>(sc, st, c, pw);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          pp[2 * kb + j] = u32x4{pw[kb][j][0], pw[kb][j][1], pw[kb][j][2], pw[kb][j][3]};
    };
    const bool need_mask = (n0 + kBN > nk) || (CAUSAL && n0 + kBN - 1 > wrow0 + off);
    if (need_mask) {
      const int lim = CAUSAL ? min(nk - 1, row + off) : nk - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = n0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
          if (key > lim) sc[kb][v] = kNegInf;
        }
      finish();
    } else {
      finish();
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // The exponent reference (as in the other bf16 forward): a first pass
  // fixes it at the row maximum of the first key tile; if a later score
  // rises far enough above it for P, l or O to overflow, the workgroup
  // runs the tiles again with the exact lazy reference (moved when a
  // tile's maximum passes it by kTau, O rescaled then).
  auto run = [&](auto fixed_ref) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[mb][v] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) pp[i] = u32x4{0u, 0u, 0u, 0u};
    st = RowState{kNegInf, 0.f, 0.f};
    if (nt == 0) return;
    // prologue: K(0) and V(0) in place before slot 0, and the V buffer
    // that the first (P = 0) product reads cleared
    if (grp == 1) issue_all(0, std::integral_constant<int, 0>{});
    {
      typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
      lds_u32x4* z = (lds_u32x4*)(size_t)vbuf(kVBufs - 1);
      for (int i = tid; i < kTileBytes / 16; i += kThreads) z[i] = u32x4{0u, 0u, 0u, 0u};
    }
    wait_vm0();
    __syncthreads();
    // One loop per wave group (the group is uniform per wave), so that
    // neither loop carries the other order's values; both pass the same
    // 2 (nt + 1) barriers.
    auto slots = [&](auto lead) __attribute__((always_inline)) {
      constexpr bool LEAD = decltype(lead)::value;
      for (int u = 0; u <= nt; ++u) {
        // slot 2u: waves 0-3 M(u); waves 4-7 load K(u+1), then X(u-1)
        const bool more = u + 1 < nt;
        if constexpr (!LEAD) {
          if (more) issue_all(u + 1, std::integral_constant<int, 1>{});
        }
        if constexpr (LEAD) matrix_phase(u);
        else if (u >= 1) vector_phase(u - 1, fixed_ref);
        __syncthreads();
        // slot 2u + 1: waves 0-3 load V(u+1), then X(u); waves 4-7 M(u)
        if constexpr (LEAD) {
          if (more) issue_all(u + 1, std::integral_constant<int, 2>{});
          vector_phase(u, fixed_ref);
          // V(u) (issued two slots ago) must have landed; V(u+1) may stay
          if (more) __builtin_amdgcn_s_waitcnt(0x0F70 | kLPW);
          else wait_vm0();
        } else {
          matrix_phase(u);
          wait_vm0();  // K(u+1)
        }
        __syncthreads();
      }
    };
    if (grp == 0) slots(std::true_type{});
    else slots(std::false_type{});
  };

  if (tid == 0) redo = 0;
  run(std::true_type{});
  {
    // inf or NaN anywhere in this lane's l, lr or O shows up in the sum
    float chk = st.l + st.lr;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) chk += o[mb][v] * 0.f;
    if (__any(!__builtin_isfinite(chk)) && lane == 0) redo = 1;
  }
  __syncthreads();
  if (redo) run(std::false_type{});

  // ---- epilogue: O = O^T / lr, LSE = ln 2 * (m + log2 l)
  const float ltot = sum_halves(st.l);
  const float lrtot = sum_halves(st.lr);
  if (row < Nq) {
    const bool live = ltot > 0.f;
    float inv = live ? 1.f / lrtot : 0.f;
    bool nan_out = false;
    if constexpr (PAGED) nan_out = page_bad != 0;
    if (nan_out) inv = __builtin_nanf("");
    __bf16* orow = O + qbase + (long)row * kD;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
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

template <bool CAUSAL, bool PAGED>
hipError_t launch(const FwdArgs& a, const PagedCache& pk) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long blocks = (long)n_qt * a.Hq * a.B;
  hipLaunchKernelGGL((fwd_bf16_pp_kernel<CAUSAL, PAGED>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, a.stream, static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                     static_cast<__bf16*>(a.o), a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                     a.scale * kLog2e, pk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_pp(const FwdArgs& a) {
  const PagedCache none{nullptr, nullptr, 0, 0};
  return a.causal ? launch<true, false>(a, none) : launch<false, false>(a, none);
}

hipError_t launch_paged_prefill_bf16_pp(const FwdArgs& a, const int32_t* bt,
                                        const int32_t* sl, int max_pages,
                                        int num_pages) {
  const PagedCache pk{bt, sl, max_pages, num_pages};
  return a.causal ? launch<true, true>(a, pk) : launch<false, true>(a, pk);
}

}  // namespace fa
