// SLA2 attention for one query block: sparse branch, linear branch and the combine in one
// kernel (steps 2-4 of the computation flow on the summary page "SLA2: Sparse-Linear
// Attention with Learnable Routing and QAT", paper.rainbus.top; "Sparse Branch", "Linear
// Branch" and the mix box of the §3 flowchart, §7 note 2, of "SLA2: Sparse-Linear
// Attention v2 for Diffusion Transformers").
//
// One workgroup per query block i (128 queries, 8 wavefronts). Wavefronts 0-3 run the sparse
// branch and wavefronts 4-7 the linear branch at the same time, so that on each SIMD a
// wavefront bound by vector ALU work (the softmax) shares the unit with one bound by memory
// traffic (the h_j^T gathers). The groups advance independently: each synchronises its four
// wavefronts through its own counter in LDS, and the workgroup barrier is used only to
// start and to hand N_l over at the end.
//
// Sparse branch — wavefront w owns queries 32 w .. 32 w + 31 (lane: query 32 w + lane % 32,
// half g = lane / 32 of each key tile) and all of d_v. For each kept key block j, ascending:
//   S^T = Khat_j Qhat_i^T                 INT8 MFMA 32x32x32, exact int32
//   S   = S_int * s_q * s_k / sqrt(d)     folded into one fp32 multiply (log2 domain)
//   m   = max(m, rowmax S)                running max, raised once per 64-key block
//   P~  = exp(S - m);  l = l e^(m_old-m) + sum P~   (l sums the unquantised P~)
//   Phat = E4M3(448 P~)                   packed from the accumulator registers
//   acc = acc e^(m_old-m) + (Phat Vhat_j) s_v / 448   FP8 MFMA 32x32x64
// O_s = acc / l (0 for a query block with no kept block). The accumulator is kept in units
// of the current block's V scale: acc' <- acc' (f s_v,prev / s_v,j) + Phat Vhat_j.
// With S^T (keys as MFMA rows) every lane owns one query, so row maxima and sums are in-lane
// plus one exchange with lane ^ 32, and the lane's 32 P values are exactly the B operand of
// the FP8 product (V^T tiles are stored in the matching key order, vkey_at); acc[dt] holds
// O^T rows d_v = 32 dt + 8 (i/4) + 4 g + i%4 (register i) of the lane's query. K and V^T
// tiles stream through 6-slot LDS rings (global_load_lds, four blocks ahead); step e issues
// the S product of block e + 1 before the softmax of block e, so the matrix unit works
// while the vector unit computes the exponentials. The ring depth gives the group barrier a
// step of slack: at step e a wavefront waits only for the others to have finished step
// e - 2.
//
// Linear branch — H_i, Z_i over the dropped blocks: the total minus the kept blocks when
// those are fewer (the same list the sparse loop walks), else a direct sum over the dropped
// blocks. Wavefront w gathers rows d_v = 32 w .. +31 of every h_j^T into MFMA accumulators:
// with A = +-I (one nonzero product per output, so each step is one exact fp32 addition) and
// B = 16 columns of the h_j^T rows, 32x32x16 bf16 MFMAs add H tiles (rows d_phi, columns
// d_v); z_j is summed alongside. That accumulator layout is already the A operand (rows d_v,
// 8 d_phi per lane) of N_l^T = H_i^T phi(Q_i)^T, so H_i goes through bf16 hi + lo straight
// from registers; the B operand phi(Q_i) (phi = softmax over d) is shared through LDS with
// its d order permuted to match. den = phi(q) . Z_i with the same bf16 phi values.
//
// Combine — the linear wavefronts leave N_l^T in LDS over the idle rings; the sparse
// wavefronts form O = alpha O_s + (1 - alpha) N_l / den. alpha = 1 or no dropped block skips
// the linear branch (O_l = 0).
#include <algorithm>
#include <type_traits>

#include "sla2_common.h"

namespace sla2 {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.8073549220576041f;  // log2(448)
constexpr float kInvSqrtD = 0.088388347648318440f;
constexpr int kTile = kBK * kD;            // 8 KB: one K tile or one V^T tile
constexpr int kRing = 6;                   // slots of the K and V^T rings
constexpr int kAhead = 4;                  // tiles in flight ahead of the one in use
// LDS map (bytes): K ring, V^T ring; linear branch: phi(Q_i) (128 rows x 272 B), block list
// (< nkb / 2 entries), Z_i, den. N_l is handed over through the idle rings.
constexpr int kOffK = 0;
constexpr int kOffV = kRing * kTile;
constexpr int kPadPhi = 136;               // bf16 row stride of phi(Q_i)
constexpr int kOffPhi = 2 * kRing * kTile; // 98304
constexpr int kOffLst = kOffPhi + 128 * kPadPhi * 2;
constexpr int kOffZ = kOffLst + 4096;
constexpr int kOffDen = kOffZ + 512;       // 2 x 128 floats (by row parity)
constexpr int kOstPad = 36;                // float row stride of the output staging tiles
constexpr int kOffOst = kOffDen + 1024;    // 4 wavefronts x 32 rows x kOstPad floats
constexpr int kLdsBytes = kOffOst + 4 * 32 * kOstPad * 4;   // 157184
constexpr int kOffNl = 0;
static_assert(kOffNl + 4 * 4 * 4 * 64 * 16 <= kOffPhi, "N_l hand-over exceeds the rings");
constexpr int kAttnThreads = 512;

// One key block: 512 chunks of 16 B of K and 512 of V^T. Wavefront w, instruction u copies
// chunks ((u & 1) * 4 + w) * 64 .. +63 of K (u = 0, 1) or of V^T (u = 2, 3), in LDS order: the
// destination of a wavefront's instruction is contiguous.
__device__ inline void issue_tile(int8_t* kdst, int8_t* vdst, const int8_t* kt, const uint8_t* vt,
                                  int w, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c0 = ((u & 1) * 4 + w) * 64;     // chunk of this wavefront within the tile
    const unsigned off = 16u * static_cast<unsigned>(c0 + lane);
    const void* src = u < 2 ? static_cast<const void*>(kt + off) : static_cast<const void*>(vt + off);
    int8_t* dst = (u < 2 ? kdst : vdst) + 16 * c0;
    __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                              reinterpret_cast<uintptr_t>(dst)),
                                     16, 0, 0);
  }
}

// Synchronisation of one group of four wavefronts through LDS (the hardware barrier spans the
// whole workgroup, and the two groups advance at their own pace). Each wavefront counts its
// arrivals in a word of its own: an arrival waits for the wavefront's LDS operations to
// complete, then adds one. A wait polls the group's four words (one 16-byte read) until each
// has reached the target. The poll is bounded (kSpinLimit sleeps of 64 clocks): a miscounted
// wait ends instead of waiting forever, and sets the error word `err` (the host reads it back
// with sla2_workspace_status), since the output is then unreliable. The counter accesses
// are written in asm (the poll waits for its read inside the same asm block): the compiler
// would otherwise treat them as possibly overlapping the loads into LDS still in flight and
// wait for all of them first.
constexpr int kSpinLimit = 1 << 20;
__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ inline void group_arrive(uint32_t group, int w) {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's LDS accesses are done
  // one increment, from lane 0 alone (exec narrowed inside the asm: no branch in the code)
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "ds_add_u32 %1, %2\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(group + 4 * w), "v"(1u)
      : "memory");
}
__device__ inline void group_wait(uint32_t group, uint32_t target, uint32_t* err) {
  for (int it = 0; it < kSpinLimit; ++it) {
    i32x4 v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(group) : "memory");
    const uint32_t lo = min(min(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1])),
                            min(static_cast<uint32_t>(v[2]), static_cast<uint32_t>(v[3])));
    if (__builtin_amdgcn_readfirstlane(lo) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
  if (__builtin_amdgcn_mbcnt_lo(~0u, 0u) == 0u) atomicOr(err, 1u);   // lane 0: gave up
}

__device__ inline int lane_value(int v, int k) { return __builtin_amdgcn_readlane(v, k); }
// A per-lane value the compiler may not hoist out of the row loop: offsets derived from it
// are recomputed per row (hoisted, they would stay live across the rows and, with all
// registers in use, be spilled; reloading a spill waits for every store in flight)
__device__ inline unsigned lane_off(unsigned x) {
  asm volatile("" : "+v"(x));
  return x;
}
// max / sum of a value and its copy in lane ^ 32 (one VALU swap of the two lane halves); the
// two lanes get the same result (the operation is commutative)
__device__ inline int pair_max(int v) {
  const auto r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
  return max(static_cast<int>(r[0]), static_cast<int>(r[1]));
}
__device__ inline float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float lane_value(float v, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}

// Values of one row (query block) for the sparse group, staged in LDS by the linear group.
struct RowStage {
  int n;
  float a, sq;
  int pad;
  int lj[128];
  float lsk[128], lsv[128];
};

// Persistent grid: gridDim.x workgroups (one per CU), each taking rows blockIdx.x + gridDim.x k
// (remapped per XCD); kAttnThreads threads. kTaps: also write O_s and O_l (debug taps).
// kSparse = false: the linear branch alone, O = (1 - alpha) O_l (the unquantised sparse branch
// is then added by its own kernel); the sparse wavefronts only do the combine.
template <typename T, bool kTaps, bool kSparse>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const T* __restrict__ Q, const int8_t* __restrict__ qc, const int8_t* __restrict__ kc,
    const uint8_t* __restrict__ vc, const float* __restrict__ sq, const float* __restrict__ sk,
    const float* __restrict__ sv, const uint16_t* __restrict__ ht_bf16,
    const float* __restrict__ z, const float* __restrict__ htot_t,
    const float* __restrict__ ztot, const uint8_t* __restrict__ mask,
    const int32_t* __restrict__ list, int list_stride, const int32_t* __restrict__ cnt,
    const float* __restrict__ alpha, float* __restrict__ O, float* __restrict__ O_s_tap,
    float* __restrict__ O_l_tap, uint32_t* __restrict__ err, int N, int H, int BH) {
  __shared__ __attribute__((aligned(16))) int8_t smem[kLdsBytes];
  // arrival counters of the sparse (0-3) and linear (4-7) wavefronts: an object of their own
  __shared__ __attribute__((aligned(16))) uint32_t ctr[8];
  // the next row's values for the sparse group, staged by the linear group (by row parity)
  __shared__ RowStage stage[2];
  const int t = threadIdx.x;
  // w is wave-uniform (a scalar): addresses are formed as a uniform row base plus a 32-bit
  // lane offset, so no 64-bit per-lane address stays live across rows
  const int lane = t & 63, w = __builtin_amdgcn_readfirstlane((t >> 6) & 3), g = lane >> 5,
            l32 = lane & 31;
  const bool linear_role = t >= 256;
  const int nqb = N / kBQ, nkb = N / kBK, total = nqb * BH;
  // counters first: the barrier then waits for no memory read
  if (t < 8) ctr[t] = 0;
  lds_barrier();   // counters set
  // Row (query block) k of this workgroup: rows blockIdx.x + gridDim.x k, remapped so that
  // consecutive rows of one head stay on one XCD (workgroups are dealt to the 8 XCDs in turn)
  struct Row {
    int i, bh;
    size_t row, qblk, tile0;
    const int32_t* L;
  };
  auto row_at = [&](int k, Row& r) -> bool {
    int lr = static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) * k;
    if (lr >= total) return false;
    if ((total & 7) == 0 && (gridDim.x & 7) == 0) lr = (lr & 7) * (total >> 3) + (lr >> 3);
    r.i = lr % nqb;
    r.bh = lr / nqb;
    r.row = static_cast<size_t>(r.bh) * nqb + r.i;
    r.qblk = static_cast<size_t>(r.bh) * N + static_cast<size_t>(r.i) * kBQ;   // first query
    r.tile0 = static_cast<size_t>(r.bh) * nkb;
    r.L = list + r.row * list_stride;
    return true;
  };
  // N_l hand-over slot (d_v tile dt, query tile qt, k4) of this lane: 4 floats, lane-contiguous
  auto nl_slot = [&](int dt, int qt, int k4, unsigned ln) {
    return reinterpret_cast<float*>(smem + kOffNl) + (((dt * 4 + qt) * 4 + k4) * 64 + ln) * 4;
  };

  if (!linear_role) {
    // =========================================================== sparse branch
    const uint32_t cs = lds_addr(&ctr[0]);   // arrivals: per wavefront, see the prologue
    const int qo = 32 * w + l32;              // the query this lane scores
    uint32_t narr = 0;                        // this wavefront's arrivals so far (all alike)
    for (int kr = 0;; ++kr) {
    Row rw;
    if (!row_at(kr, rw)) break;
    const size_t row = rw.row, qblk = rw.qblk, tile0 = rw.tile0;
    const int32_t* L = rw.L;
    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
    float lsum = 0.f, svcur = 0.f;
    int n, nuns;
    float a;
    bool do_lin;
    if constexpr (!kSparse) {
      n = cnt[row];
      a = alpha[static_cast<size_t>(rw.bh % H) * nqb + rw.i];
      nuns = nkb - n;
      do_lin = nuns > 0 && (kTaps || a != 1.f);
    } else {
      // block index, s_k and s_v of kept blocks 0 .. 127, one per lane (later ones are read
      // from memory when needed). The first row reads them itself: the list row without
      // waiting for the count n (entries past n are never used, and clamping keeps their
      // reads in range) together with the Q codes, then the first tiles, then the scales. For
      // later rows the linear group has staged them in LDS.
      int lj[2];
      float lsk[2], lsv[2], sqv;
      i32x4 qf[4];
      const int8_t* qrow = qc + qblk * kD;   // Q codes of the row's first query
      const unsigned ln = lane_off(static_cast<unsigned>(lane));
      const unsigned qoff = (32u * w + (ln & 31u)) * kD + 16u * (ln >> 5);   // this lane's
      if (kr == 0) {
#pragma unroll
        for (int c = 0; c < 2; ++c) lj[c] = L[static_cast<unsigned>(min(64 * c + lane, list_stride - 1))];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          qf[tt] = *reinterpret_cast<const i32x4*>(qrow + static_cast<unsigned>(qo * kD + 32 * tt + 16 * g));
        asm volatile("" ::: "memory");
        n = cnt[row];
        a = alpha[static_cast<size_t>(rw.bh % H) * nqb + rw.i];
        sqv = sq[row];
#pragma unroll
        for (int c = 0; c < 2; ++c) lj[c] = min(max(lj[c], 0), nkb - 1);
      } else {
        // every sparse wavefront has read the previous row's hand-over (over the rings)
        group_arrive(cs, w);
        ++narr;
        group_wait(cs, narr, err);
        const RowStage& st = stage[kr & 1];
        n = st.n;
        a = st.a;
        sqv = st.sq;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          lj[c] = st.lj[64 * c + lane];
          lsk[c] = st.lsk[64 * c + lane];
          lsv[c] = st.lsv[64 * c + lane];
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          qf[tt] = *reinterpret_cast<const i32x4*>(qrow + (qoff + 32u * tt));
      }
      nuns = nkb - n;
      do_lin = nuns > 0 && (kTaps || a != 1.f);
      // value of kept block k < 128 from the lanes, without a branch (both reads, one select)
      auto pick = [&](const auto (&v)[2], int k) {
        const auto a0 = lane_value(v[0], k & 63), a1 = lane_value(v[1], k & 63);
        return k < 64 ? a0 : a1;
      };
      // kSmall (n <= 128): every kept block's values come from the lanes; otherwise blocks
      // from 128 on are read from memory
      auto blk_of = [&](int k, auto small) -> int {
        if constexpr (decltype(small)::value) return pick(lj, k);
        else return k < 128 ? pick(lj, k) : L[k];
      };
      auto sk_of = [&](int k, auto small) -> float {
        if constexpr (decltype(small)::value) return pick(lsk, k);
        else return k < 128 ? pick(lsk, k) : sk[tile0 + L[k]];
      };
      auto sv_of = [&](int k, auto small) -> float {
        if constexpr (decltype(small)::value) return pick(lsv, k);
        else return k < 128 ? pick(lsv, k) : sv[tile0 + L[k]];
      };
      const float cq = sqv * (kLog2e * kInvSqrtD);
      float m2 = -INFINITY;
      auto issue = [&](int k, auto small) {
        const size_t o = (tile0 + blk_of(k, small)) * kTile;
        const int slot = k % kRing;
        issue_tile(smem + kOffK + slot * kTile, smem + kOffV + slot * kTile, kc + o, vc + o, w, lane);
      };
      // refill of step e: tile e + kAhead, or past the end of the list the same four
      // instructions copying one 16-byte line (every lane the same address) into that free
      // slot, so that every step has the same number of loads in flight (no branch, one
      // wait count)
      auto refill = [&](int e, auto small) {
        const int k = e + kAhead;
        const bool real = k < n;
        const size_t o = (tile0 + blk_of(real ? k : 0, small)) * kTile;
        const int slot = k % kRing;
        const int8_t* ks = kc + o;
        const uint8_t* vs = vc + o;
        int8_t* kdst = smem + kOffK + slot * kTile;
        int8_t* vdst = smem + kOffV + slot * kTile;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c0 = ((u & 1) * 4 + w) * 64;
          const unsigned src_off = real ? 16u * static_cast<unsigned>(c0 + lane) : 0u;
          const void* src = u < 2 ? static_cast<const void*>(ks + src_off)
                                  : static_cast<const void*>(vs + src_off);
          int8_t* dst = (u < 2 ? kdst : vdst) + 16 * c0;
          __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                                    reinterpret_cast<uintptr_t>(dst)),
                                           16, 0, 0);
        }
      };
      for (int kk = 0; kk < kAhead && kk < n; ++kk) issue(kk, std::true_type{});
      if (kr == 0) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          lsk[c] = (sk + tile0)[static_cast<unsigned>(lj[c])];
          lsv[c] = (sv + tile0)[static_cast<unsigned>(lj[c])];
        }
      }
      // Arrival 0: this wavefront's parts of tiles 0 .. kAhead - 1 (and the Q codes and
      // per-block values) have landed. Arrival e + 1 ends step e: its part of tile
      // e + kAhead - 1 has landed and its LDS reads of the step are done. Step e >= 1 waits
      // for all four arrivals e - 1 (end of step e - 2): tile e + 1 is then complete for its S
      // product, and the slot of tile e - 2 is free for tile e + kAhead.
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      group_arrive(cs, w);
      ++narr;
      const uint32_t base = narr;   // arrivals after the prologue's
      group_wait(cs, base, err);
      // S^T of block k into (s0, s1): key tiles 0-31 and 32-63; the first product takes a
      // literal zero accumulator (the MFMA's inline constant, no register fill)
      auto qk = [&](int k, i32x16& s0, i32x16& s1) {
        const int8_t* kt = smem + kOffK + (k % kRing) * kTile;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int r0 = l32, r1 = 32 + l32;
          const i32x4 a0 = *reinterpret_cast<const i32x4*>(kt + r0 * kD + 16 * kchunk_swz(r0, 2 * tt + g));
          const i32x4 a1 = *reinterpret_cast<const i32x4*>(kt + r1 * kD + 16 * kchunk_swz(r1, 2 * tt + g));
          s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, qf[tt], tt == 0 ? i32x16{} : s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, qf[tt], tt == 0 ? i32x16{} : s1, 0, 0, 0);
        }
      };
      // step e: refill, S of block e + 1, softmax and P V of block e. After the block's scalars
      // and the refill, the step is one straight-line region (the S product is issued also on
      // the last step, on a stale slot, and not used), in which the S products are interleaved
      // with the softmax arithmetic and the P V products with the rescale.
      auto step = [&](int e, const i32x16& c0, const i32x16& c1, i32x16& n0, i32x16& n1,
                      auto small) {
        if (e >= 1) group_wait(cs, base - 1 + e, err);
        refill(e, small);
        const float c = cq * sk_of(e, small);
        const float svj = sv_of(e, small);
        // The region below is written in issue order and fenced (sched_barrier): every pair of
        // S products of block e + 1 is followed by a share of the softmax arithmetic of block
        // e, which runs on the vector unit while the matrix unit works; then the V reads, and
        // each P V product after its rescale. (The S product is issued also on the last step,
        // on a stale slot, and not used.)
        const int8_t* kt = smem + kOffK + ((e + 1) % kRing) * kTile;
        i32x4 ka[4], kb[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int r0 = l32, r1 = 32 + l32;
          ka[tt] = *reinterpret_cast<const i32x4*>(kt + r0 * kD + 16 * kchunk_swz(r0, 2 * tt + g));
          kb[tt] = *reinterpret_cast<const i32x4*>(kt + r1 * kD + 16 * kchunk_swz(r1, 2 * tt + g));
        }
        // S^T of block e + 1 for key tiles 0-31 (n0) and 32-63 (n1), K step tt; the first step
        // takes a literal zero accumulator (the MFMA's inline constant, no register fill)
        auto qk_step = [&](int tt) {
          n0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[tt], qf[tt], tt == 0 ? i32x16{} : n0, 0, 0, 0);
          n1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kb[tt], qf[tt], tt == 0 ? i32x16{} : n1, 0, 0, 0);
        };
        __builtin_amdgcn_sched_barrier(0);
        qk_step(0);
        // ---- online softmax of block e in the log2 domain: row maximum
        int mx = c0[0];
#pragma unroll
        for (int k = 1; k < 16; ++k) mx = max(mx, c0[k]);
#pragma unroll
        for (int k = 0; k < 16; ++k) mx = max(mx, c1[k]);
        mx = pair_max(mx);
        const float m2new = fmaxf(m2, static_cast<float>(mx) * c);
        const float f = __builtin_amdgcn_exp2f(m2 - m2new);  // 0 on the first block
        const float b0 = kLog2_448 - m2new;
        float psum = 0.f;
        i32x8 pk;
        // exponentials, sums and E4M3 packing of the lane's values wv0 .. wv0 + 1 (groups of 4)
        auto soft_part = [&](int wv0) {
#pragma unroll
          for (int wv = wv0; wv < wv0 + 2; ++wv) {
            const i32x16& sT = (wv < 4) ? c0 : c1;
            const int e0 = 4 * (wv & 3);
            const float p0 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sT[e0]), c, b0));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sT[e0 + 1]), c, b0));
            const float p2 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sT[e0 + 2]), c, b0));
            const float p3 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sT[e0 + 3]), c, b0));
            psum += (p0 + p1) + (p2 + p3);
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
            pk[wv] = word;
          }
        };
        __builtin_amdgcn_sched_barrier(0);
        qk_step(1);
        soft_part(0);
        __builtin_amdgcn_sched_barrier(0);
        qk_step(2);
        soft_part(2);
        __builtin_amdgcn_sched_barrier(0);
        qk_step(3);
        soft_part(4);
        __builtin_amdgcn_sched_barrier(0);
        // ---- V^T reads for the P V products
        const int8_t* vt = smem + kOffV + (e % kRing) * kTile;
        i32x8 av[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d = 32 * dt + l32;
          const i32x4 v0 = *reinterpret_cast<const i32x4*>(vt + d * kBK + 16 * vchunk_swz(d, 2 * g));
          const i32x4 v1 = *reinterpret_cast<const i32x4*>(vt + d * kBK + 16 * vchunk_swz(d, 2 * g + 1));
          av[dt] = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        }
        soft_part(6);
        lsum = fmaf(lsum, f, psum);
        m2 = m2new;
        // rescale of the accumulator for this block: f s_v,prev / s_v,j. A block with s_v = 0
        // has all-zero codes, adds nothing and keeps the current units (factor f alone). The
        // ratio uses the hardware reciprocal (a rescale factor; 1 ulp does not matter).
        const float rsv = __builtin_amdgcn_rcpf(svj);   // unused when s_v,j = 0
        const float rr = svcur > 0.f ? f * svcur * rsv : 0.f;
        const float r = svj > 0.f ? rr : f;
        svcur = svj > 0.f ? svj : svcur;
        // ---- acc[dt] <- acc[dt] r + Vhat_dt Phat (d_v tile dt, this lane's query)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          __builtin_amdgcn_sched_barrier(0);
          acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[dt], pk, acc[dt] * r, 0, 0, 0,
                                                                    127, 0, 127);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the step's products stay in this region (the compiler would otherwise move the
        // softmax and the P V products past the arrival, away from the S products they are
        // interleaved with)
        asm volatile("" : : "v"(acc[0]), "v"(acc[1]), "v"(acc[2]), "v"(acc[3]));
        // ---- end of step: this wavefront's part of tile e + kAhead - 1 landed (the refill of
        // this step may still be in flight) and its reads done
        __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
        group_arrive(cs, w);
      };
      auto run = [&](auto small) {
        i32x16 sa0, sa1, sb0, sb1;
        if (n > 0) qk(0, sa0, sa1);
        for (int e = 0; e < n; e += 2) {
          step(e, sa0, sa1, sb0, sb1, small);
          if (e + 1 < n) step(e + 1, sb0, sb1, sa0, sa1, small);
        }
      };
      if (n <= 128) run(std::true_type{});
      else run(std::false_type{});
      narr = base + n;
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the last refills have landed
    }
    lsum = pair_sum(lsum);
    const float os_scale = (n > 0 && lsum > 0.f) ? svcur / lsum : 0.f;
    lds_barrier();   // rings idle
    lds_barrier();   // N_l and den handed over
    // lane's output rows: query qo, d_v = 32 dt + 8 k4 + 4 g + (0..3)
    auto out_ptr = [&](float* base, int dt, int k4) {
      return base + qblk * kD + static_cast<unsigned>(qo * kD + 32 * dt + 8 * k4 + 4 * g);
    };
    // O rows of this wavefront (queries 32 w .. +31: 16 KB, contiguous) leave through LDS one
    // d_v tile at a time: the lane's four groups of 4 go in at row l32, and each store
    // instruction then writes 8 rows x 128 B, whole lines (the registers alone would give
    // 32-byte pieces of 32 rows per instruction). The staging tile is this wavefront's own.
    float* ost = reinterpret_cast<float*>(smem + kOffOst) + w * (32 * kOstPad);
    float* orow = O + (qblk + 32 * w) * kD;   // the wavefront's first output row
    const unsigned ln = lane_off(static_cast<unsigned>(lane));
    auto store_tile = [&](int dt, const f32x4 (&v)[4]) {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
        *reinterpret_cast<f32x4*>(ost + l32 * kOstPad + 8 * k4 + 4 * g) = v[k4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const unsigned r = 8u * u + (ln >> 3), c = 4u * (ln & 7u);
        *reinterpret_cast<f32x4*>(orow + (r * kD + 32u * dt + c)) =
            *reinterpret_cast<const f32x4*>(ost + r * kOstPad + c);
      }
    };
    if (!do_lin) {
      // no dropped block (O_l = 0) or alpha = 1: O = alpha O_s
      const float coef = (nuns == 0 ? a : 1.f) * os_scale;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        f32x4 v[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
          v[k4] = f32x4{acc[dt][4 * k4] * coef, acc[dt][4 * k4 + 1] * coef,
                        acc[dt][4 * k4 + 2] * coef, acc[dt][4 * k4 + 3] * coef};
        store_tile(dt, v);
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          if (kTaps) {
            if (O_s_tap)
              *reinterpret_cast<f32x4*>(out_ptr(O_s_tap, dt, k4)) =
                  f32x4{acc[dt][4 * k4] * os_scale, acc[dt][4 * k4 + 1] * os_scale,
                        acc[dt][4 * k4 + 2] * os_scale, acc[dt][4 * k4 + 3] * os_scale};
            if (O_l_tap) *reinterpret_cast<f32x4*>(out_ptr(O_l_tap, dt, k4)) = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      continue;
    }
    // O = alpha O_s + (1 - alpha) O_l with O_s = acc os_scale, O_l = N_l / den
    const float rden =
        1.0f / (reinterpret_cast<const float*>(smem + kOffDen) + 128 * (kr & 1))[32u * w + (ln & 31u)];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 o[4];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const f32x4 nlv = *reinterpret_cast<const f32x4*>(nl_slot(dt, w, k4, ln));
        f32x4 os, ol;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          os[k] = acc[dt][4 * k4 + k] * os_scale;
          ol[k] = nlv[k] * rden;
          o[k4][k] = fmaf(a, os[k], (1.f - a) * ol[k]);
        }
        if (kTaps) {
          if (O_s_tap) *reinterpret_cast<f32x4*>(out_ptr(O_s_tap, dt, k4)) = os;
          if (O_l_tap) *reinterpret_cast<f32x4*>(out_ptr(O_l_tap, dt, k4)) = ol;
        }
      }
      store_tile(dt, o);
    }
    }
    return;
  }

  // =========================================================== linear branch
  const uint32_t cl = lds_addr(&ctr[4]);
  const int tl = t - 256;
  uint32_t larr = 0;   // this wavefront's arrivals so far (all alike)
  uint16_t* phs = reinterpret_cast<uint16_t*>(smem + kOffPhi);
  uint16_t* lst = reinterpret_cast<uint16_t*>(smem + kOffLst);
  float* zsh = reinterpret_cast<float*>(smem + kOffZ);
  for (int kr = 0;; ++kr) {
  Row rw;
  if (!row_at(kr, rw)) break;
  const size_t row = rw.row, qblk = rw.qblk, tile0 = rw.tile0;
  const int32_t* L = rw.L;
  const int bh = rw.bh;
  const int n = cnt[row];
  const float a = alpha[static_cast<size_t>(rw.bh % H) * nqb + rw.i];
  const int nuns = nkb - n;
  const bool do_lin = nuns > 0 && (kTaps || a != 1.f);
  float* dsh = reinterpret_cast<float*>(smem + kOffDen) + 128 * (kr & 1);
  f32x16 accl[4];
  if (do_lin) {
  const bool sub = n <= nuns;   // total minus kept, else direct sum over dropped
  const int nl = sub ? n : nuns;
  const float sgn = sub ? -1.f : 1.f;
  // ---- block list in LDS: the kept list (total minus kept) or the dropped blocks
  if (w == 0) {
    if (sub) {
      for (int k = lane; k < n; k += 64) lst[k] = static_cast<uint16_t>(L[k]);
    } else {
      int before = 0;
      for (int j0 = 0; j0 < nkb; j0 += 64) {
        const int j = j0 + lane;
        const bool take = j < nkb && (mask + row * nkb)[static_cast<unsigned>(j)] == 0;
        const uint64_t m = __ballot(take);
        if (take)
          lst[before + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0))] =
              static_cast<uint16_t>(j);
        before += __popcll(m);
      }
    }
  }
  // ---- H tiles of this wavefront's d_v rows: hacc[tl4] rows d_phi = 32 tl4 + 8 (i/4) + 4 g +
  // i%4, column d_v = 32 w + l32; start from H_tot^T (fragment order: chunk
  // (16 w + 4 tl4 + k4) * 64 + lane holds d_phi = 32 tl4 + 8 k4 + 4 g .. +3) or zero
  f32x16 hacc[4];
  if (sub) {
    const float* hp = htot_t + static_cast<size_t>(bh) * (kD * kD) + static_cast<unsigned>((1024 * w + lane) * 4);
#pragma unroll
    for (int tl4 = 0; tl4 < 4; ++tl4)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(hp + 256 * (4 * tl4 + k4));
        hacc[tl4][4 * k4] = v[0]; hacc[tl4][4 * k4 + 1] = v[1];
        hacc[tl4][4 * k4 + 2] = v[2]; hacc[tl4][4 * k4 + 3] = v[3];
      }
  } else {
#pragma unroll
    for (int tl4 = 0; tl4 < 4; ++tl4) hacc[tl4] = f32x16{};
  }
  // ---- phi(q) for query tl/2, d = 64 (tl%2) .. +63, rounded to bf16, and to LDS with the d
  // order permuted for the MFMA B operand: slot 16 k + s of a row holds d = 16 k + (s with
  // bits 2 and 3 swapped)
  const int pq = tl >> 1, ph = tl & 1;
  uint16_t* prow = phs + pq * kPadPhi + 64 * ph;
  {
    uint32_t phw[32];   // bf16 pairs, d = 64 ph + 2 e, +1
    const T* qp = Q + qblk * kD + static_cast<unsigned>(pq * kD + 64 * ph);
    float x[64];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8<T>(qp + 8 * u, x + 8 * u);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 64; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      x[e] = __expf(x[e] - mx);
      sum += x[e];
    }
    sum += __shfl_xor(sum, 1);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int e = 0; e < 32; ++e) phw[e] = pack_bf16x2(x[2 * e] * inv, x[2 * e + 1] * inv);
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const uint32_t* hw = phw + 8 * G;   // d = 16 G + 0..15 of this half as 8 bf16 pairs
      *reinterpret_cast<i32x4*>(prow + 16 * G) =
          i32x4{static_cast<int>(hw[0]), static_cast<int>(hw[1]), static_cast<int>(hw[4]),
                static_cast<int>(hw[5])};
      *reinterpret_cast<i32x4*>(prow + 16 * G + 8) =
          i32x4{static_cast<int>(hw[2]), static_cast<int>(hw[3]), static_cast<int>(hw[6]),
                static_cast<int>(hw[7])};
    }
  }
  group_arrive(cl, w);
  ++larr;
  group_wait(cl, larr, err);   // block list and phi(Q_i) visible
  // ---- gathers. A = sgn I: fragment m has lane row l32 = 16 m + 8 g + b set at element b; B
  // fragment f = 2 tl4 + m of block j: row d_v = 32 w + l32 of h_j^T, d_phi = 32 tl4 + 16 m +
  // 8 g .. +7, which in fragment order is chunk (8 w + f) * 64 + lane. Each lane also sums
  // z_j[2 lane], z_j[2 lane + 1].
  bf16x8 idf[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int b = 0; b < 8; ++b) idf[m][b] = to_bf16(l32 == 16 * m + 8 * g + b ? sgn : 0.f);
  // block j of the head: h_j^T at ht_bf16 + (tile0 + j) d^2 (this lane's chunks at hoff +
  // 512 f), z_j at z + (tile0 + j) d (this lane's pair at 2 lane)
  const unsigned hoff = static_cast<unsigned>((512 * w + lane) * 8);
  float zs0 = 0.f, zs1 = 0.f;
  struct Blk {
    i32x4 h[8];
    f32x2 z;
  };
  // Three register buffers used in turn: blocks b + 1 and b + 2 are loading while block b is
  // added. The loads are unconditional (the index is clamped; the extra loads at the end are
  // cache hits), so the wait before each use is an exact count.
  auto gload = [&](Blk& dst, int nn) {
    const int j = __builtin_amdgcn_readfirstlane(lst[min(nn, nl - 1)]);   // the same in every lane
    const uint16_t* hp = ht_bf16 + (tile0 + j) * (kD * kD);
#pragma unroll
    for (int f = 0; f < 8; ++f) dst.h[f] = *reinterpret_cast<const i32x4*>(hp + (hoff + 512u * f));
    dst.z = *reinterpret_cast<const f32x2*>(z + (tile0 + j) * kD + static_cast<unsigned>(2 * lane));
    asm volatile("" ::: "memory");   // keeps the loads here (not moved down to their use)
  };
  auto gadd = [&](const Blk& src) {
#pragma unroll
    for (int f = 0; f < 8; ++f)   // f = 2 tl4 + m
      hacc[f >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          idf[f & 1], __builtin_bit_cast(bf16x8, src.h[f]), hacc[f >> 1], 0, 0, 0);
    zs0 += src.z[0];
    zs1 += src.z[1];
  };
  if (nl > 0) {
    Blk ga, gb, gc;
    gload(ga, 0);
    gload(gb, 1);
    for (int bk = 0;;) {
      gload(gc, bk + 2);
      gadd(ga);
      if (++bk == nl) break;
      gload(ga, bk + 2);
      gadd(gb);
      if (++bk == nl) break;
      gload(gb, bk + 2);
      gadd(gc);
      if (++bk == nl) break;
    }
  }
  if (w == 0) {
    const f32x2 zt = sub ? *reinterpret_cast<const f32x2*>(ztot + static_cast<size_t>(bh) * kD + static_cast<unsigned>(2 * lane))
                         : f32x2{0.f, 0.f};
    zsh[2 * lane] = fmaf(sgn, zs0, zt[0]);
    zsh[2 * lane + 1] = fmaf(sgn, zs1, zt[1]);
  }
  group_arrive(cl, w);
  ++larr;
  group_wait(cl, larr, err);   // Z_i visible
  {
    // den = phi(q) . Z_i from the half row of phi in LDS (read by the sparse wavefronts after
    // the hand-over). Chunk c of group G holds d = 16 G + 8 (b / 4) + 4 c + b % 4 at element b.
    float dn = 0.f;
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(prow + 16 * G + 8 * c);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const uint32_t wd = static_cast<uint32_t>(v[b >> 1]);
          const float phv = __uint_as_float((b & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
          dn = fmaf(phv, zsh[64 * ph + 16 * G + 8 * (b >> 2) + 4 * c + (b & 3)], dn);
        }
      }
    dn += __shfl_xor(dn, 1);
    if (ph == 0) dsh[pq] = dn;
  }
  // ---- N_l^T = H_i^T phi(Q_i)^T: K step ks = 2 tl4 + u takes registers 8 u .. 8 u + 7 of
  // hacc[tl4] (d_phi = 32 tl4 + 16 u + 8 (b/4) + 4 g + b%4), split into bf16 hi + lo; accl[qt]
  // holds rows d_v = 32 w + 8 (i/4) + 4 g + i%4 of query 32 qt + l32
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) accl[qt] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int tl4 = ks >> 1, u = ks & 1;
    bf16x8 ahi, alo;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const float h = hacc[tl4][8 * u + b];
      ahi[b] = to_bf16(h);
      alo[b] = to_bf16(h - static_cast<float>(ahi[b]));
    }
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const bf16x8 bph = *reinterpret_cast<const bf16x8*>(phs + (32 * qt + l32) * kPadPhi + 16 * ks + 8 * g);
      accl[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bph, accl[qt], 0, 0, 0);
      accl[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bph, accl[qt], 0, 0, 0);
    }
  }
  }   // do_lin
  // ---- the next row's values for the sparse group (its count, alpha, s_q and the block
  // index, s_k, s_v of kept blocks 0 .. 127, entries past the count clamped and unused)
  {
    Row nx;
    if (w == 0 && row_at(kr + 1, nx)) {
      RowStage& st = stage[(kr + 1) & 1];
      int lj[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        lj[c] = min(max(nx.L[static_cast<unsigned>(min(64 * c + lane, list_stride - 1))], 0), nkb - 1);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        st.lj[64 * c + lane] = lj[c];
        st.lsk[64 * c + lane] = (sk + nx.tile0)[static_cast<unsigned>(lj[c])];
        st.lsv[64 * c + lane] = (sv + nx.tile0)[static_cast<unsigned>(lj[c])];
      }
      if (lane == 0) {
        st.n = cnt[nx.row];
        st.a = alpha[static_cast<size_t>(nx.bh % H) * nqb + nx.i];
        st.sq = sq[nx.row];
      }
    }
  }
  lds_barrier();   // rings idle
  if (do_lin) {
    const unsigned ln = lane_off(static_cast<unsigned>(lane));
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
        *reinterpret_cast<f32x4*>(nl_slot(w, qt, k4, ln)) =
            f32x4{accl[qt][4 * k4], accl[qt][4 * k4 + 1], accl[qt][4 * k4 + 2], accl[qt][4 * k4 + 3]};
  }
  lds_barrier();   // N_l handed over
  }   // rows
}

// compute units of the current device (cached per device): the persistent grid's size
static int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        ncu <= 0)
      ncu = 256;
    cache[dev] = ncu;
  }
  return cache[dev];
}

template <typename T, bool kTaps, bool kSparse>
static void launch_attn_v(const Geom& g, const void* Q, const AttnArgs& x, hipStream_t s) {
  dim3 grid(std::min(g.nqb * g.BH, cu_count()));
  hipLaunchKernelGGL((attn_kernel<T, kTaps, kSparse>), grid, dim3(kAttnThreads), 0, s,
                     static_cast<const T*>(Q), x.qc, x.kc, x.vc, x.sq, x.sk, x.sv, x.ht_bf16, x.z,
                     x.htot_t, x.ztot, x.mask, x.list, x.list_stride, x.cnt, x.alpha, x.O,
                     x.O_s_tap, x.O_l_tap, x.err, g.N, g.H, g.BH);
}

template <typename T>
static void launch_attn_t(const Geom& g, const void* Q, const AttnArgs& x, bool taps,
                          hipStream_t s) {
  if (x.sparse) {
    if (taps) launch_attn_v<T, true, true>(g, Q, x, s);
    else launch_attn_v<T, false, true>(g, Q, x, s);
  } else {
    if (taps) launch_attn_v<T, true, false>(g, Q, x, s);
    else launch_attn_v<T, false, false>(g, Q, x, s);
  }
}

hipError_t launch_attn(const Geom& g, int dtype, const void* Q, const AttnArgs& x,
                       hipStream_t s) {
  const bool taps = x.O_s_tap != nullptr || x.O_l_tap != nullptr;
  if (dtype == 0) launch_attn_t<float>(g, Q, x, taps, s);
  else launch_attn_t<uint16_t>(g, Q, x, taps, s);
  return hipGetLastError();
}

}  // namespace sla2
