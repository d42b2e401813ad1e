// Software-pipelined MFMA tile streams shared by the attention kernels: step
// plans, the compile-time issue-slot balancing of the non-MFMA work between MFMAs,
// the drivers that issue a tile's MFMAs with their LDS operands read ahead, and
// the staged store of a wave's 64-row output block.
#pragma once

#include "fa_common.hpp"

#include <type_traits>
#include <utility>

namespace fa {

// One pipeline step: up to four stages of MFMAs issued in order; stage k has Nk
// operands read from LDS, each feeding Gk consecutive MFMAs.  WODD: issue time of an
// MFMA of the odd stages in units of a 16x16x32 MFMA (2 for 32x32x16 products).
template <int N0, int G0, int N1, int G1, int N2, int G2, int N3, int G3, int WODD = 2>
struct StepPlan {
  static constexpr int B1 = N0 * G0, B2 = B1 + N1 * G1, B3 = B2 + N2 * G2, NM = B3 + N3 * G3;
  static constexpr int O1 = N0, O2 = O1 + N1, O3 = O2 + N2, NOP = O3 + N3;
  static constexpr int stage(int m) { return m < B1 ? 0 : m < B2 ? 1 : m < B3 ? 2 : 3; }
  static constexpr int start(int k) { return k == 0 ? 0 : k == 1 ? B1 : k == 2 ? B2 : B3; }
  static constexpr int gsz(int k) { return k == 0 ? G0 : k == 1 ? G1 : k == 2 ? G2 : G3; }
  static constexpr int obase(int k) { return k == 0 ? 0 : k == 1 ? O1 : k == 2 ? O2 : O3; }
  static constexpr int local(int m) { return m - start(stage(m)); }
  static constexpr int op_of(int m) { return obase(stage(m)) + local(m) / gsz(stage(m)); }
  static constexpr bool first(int m) { return local(m) % gsz(stage(m)) == 0; }
  static constexpr int op_stage(int o) { return o < O1 ? 0 : o < O2 ? 1 : o < O3 ? 2 : 3; }
  static constexpr int op_local(int o) { return o - obase(op_stage(o)); }
  // issue time of MFMA m in units of a 16x16x32 MFMA
  static constexpr int weight(int m) { return (stage(m) & 1) ? WODD : 1; }
};

// Issue-slot balancing.  Slot m of a step is the gap after its MFMA m.  Under one
// 16x16x32 MFMA a wave issues about two VALU instructions at no cost (measured);
// more work in one gap delays the next MFMA, while a gap with less leaves issue
// time unused.  So the non-MFMA work of a step (the LDS operand reads and the waits
// for them, the softmax and dS arithmetic, packing, copies) is placed at compile
// time: fixed work first, then each chain of dependent items in order, every item
// at the first slot of its window with room, else at the least loaded one.
// Weights are in units of one full-rate VALU instruction (measured costs: an LDS
// operand read about two, v_exp_f32 about two).
namespace issue {
constexpr int kRow = 2;   // one 16-byte LDS read of an operand
constexpr int kTr = 4;    // two transposed LDS reads of an operand
constexpr int kWait = 1;  // s_waitcnt before the first use of an operand
constexpr int kExp = 3;   // scale-and-subtract and exponential
constexpr int kMul = 1;
constexpr int kPack = 2;  // two conversions
constexpr int kCopy = 4;  // m0 set-up, its wait state and the copy
constexpr int kCap = 3;   // fill level of a gap before the next one is used
}  // namespace issue

template <int NM>
struct SlotLoad {
  int load[NM];
  int cap = issue::kCap;
  constexpr SlotLoad() : load() {}
  // Fill level for a chain of total weight w over slots [lo, hi]: the average
  // load the window will carry, rounded up, and at least kCap.
  constexpr void level(int w, int lo, int hi) {
    int t = w;
    for (int m = lo; m <= hi; ++m) t += load[m];
    const int n = hi - lo + 1, avg = (t + n - 1) / n;
    cap = avg > issue::kCap ? avg : issue::kCap;
  }
  // item of weight w at the first slot in [lo, hi] with room, else the least
  // loaded one (the earliest of equals)
  constexpr int put(int w, int lo, int hi) {
    for (int m = lo; m <= hi; ++m) {
      if (load[m] + w <= cap) {
        load[m] += w;
        return m;
      }
    }
    int best = lo;
    for (int m = lo; m <= hi; ++m)
      if (load[m] < load[best]) best = m;
    load[best] += w;
    return best;
  }
  // the LDS reads of a plan (after the first MFMA of each operand group, for the
  // operand LA groups ahead; odd stages are transposed) and the waits for them
  template <class Plan, int LA>
  constexpr void reads() {
    for (int m = 0; m < NM; ++m) {
      if (Plan::first(m)) {
        const int o2 = (Plan::op_of(m) + LA) % Plan::NOP;
        load[m] += (Plan::op_stage(o2) & 1) ? issue::kTr : issue::kRow;
      }
      if (m + 1 == NM || Plan::first(m + 1)) load[m] += issue::kWait;
    }
  }
};

// floor(a / b) for b > 0 and any sign of a.
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((b - 1 - a) / b); }

// The steps 0..NS-1 of one tile (StepPlan PlanOf<st> each) concatenated into one
// MFMA stream, so the operand lookahead runs across step boundaries.
template <template <int> class PlanOf, int... S>
struct TileStreamImpl {
  static constexpr int NS = sizeof...(S);
  static constexpr int nms[NS] = {PlanOf<S>::NM...};
  static constexpr int nops[NS] = {PlanOf<S>::NOP...};
  static constexpr int NM = (0 + ... + PlanOf<S>::NM);
  static constexpr int NOP = (0 + ... + PlanOf<S>::NOP);
  static constexpr int step_of_m(int m) {
    int st = 0;
    while (st < NS - 1 && m >= nms[st]) m -= nms[st++];
    return st;
  }
  static constexpr int m_base(int st) {
    int a = 0;
    for (int i = 0; i < st; ++i) a += nms[i];
    return a;
  }
  static constexpr int step_of_o(int o) {
    int st = 0;
    while (st < NS - 1 && o >= nops[st]) o -= nops[st++];
    return st;
  }
  static constexpr int o_base(int st) {
    int a = 0;
    for (int i = 0; i < st; ++i) a += nops[i];
    return a;
  }
};
template <template <int> class PlanOf, class Seq>
struct TileStreamOf;
template <template <int> class PlanOf, int... S>
struct TileStreamOf<PlanOf, std::integer_sequence<int, S...>> {
  using type = TileStreamImpl<PlanOf, S...>;
};

// Issue the MFMAs of one tile in order.  begin(st) runs before the first MFMA of
// step st; operand(st, o) reads operand o of step st from LDS, right after the
// first MFMA that uses operand o - LA; mfma(st, m, op) issues MFMA m of step st;
// valu(st, m, g) emits the work placed after it (g: index of the MFMA in the whole
// tile).  Scheduling fences after each MFMA and after each slot keep this order.
template <template <int> class PlanOf, int NS, int LA, class FBegin, class FOp, class FMma,
          class FValu>
__device__ __forceinline__ void run_tile(FBegin&& begin, FOp&& operand, FMma&& mfma, FValu&& valu) {
  using T = typename TileStreamOf<PlanOf, std::make_integer_sequence<int, NS>>::type;
  using ic0 = std::integral_constant<int, 0>;
  constexpr int PRE = LA < T::NOP ? LA : T::NOP;
  u32x4 ops[LA + 1];
  // A stand-alone stream (a flush) may follow VALU code that packed its first
  // operands: two wait states before its first MFMA.
  sched_fence();
  asm volatile("s_nop 1" ::: "memory");
  sched_fence();
  begin(ic0());
  static_for<PRE>([&](auto oc) {
    constexpr int o = decltype(oc)::value, st = T::step_of_o(o);
    ops[o] = operand(std::integral_constant<int, st>(), std::integral_constant<int, o - T::o_base(st)>());
  });
  static_for<T::NM>([&](auto mc) {
    constexpr int m = decltype(mc)::value, st = T::step_of_m(m), ml = m - T::m_base(st);
    using P = PlanOf<st>;
    using stc = std::integral_constant<int, st>;
    if constexpr (ml == 0 && st > 0) begin(stc());
    constexpr int o = T::o_base(st) + P::op_of(ml);
    mfma(stc(), std::integral_constant<int, ml>(), ops[o % (LA + 1)]);
    sched_fence();
    if constexpr (P::first(ml) && o + LA < T::NOP) {
      constexpr int o2 = o + LA, st2 = T::step_of_o(o2);
      ops[o2 % (LA + 1)] = operand(std::integral_constant<int, st2>(),
                                   std::integral_constant<int, o2 - T::o_base(st2)>());
    }
    valu(stc(), std::integral_constant<int, ml>(), mc);
    sched_fence();
  });
}

// run_tile for a stream of tiles: the first LA operands of this tile come from
// `carry`, and the first LA operands of the next tile are read into it
// (next(o) reads operand o of the next tile) as the lookahead passes the end of
// this one, so no tile starts by waiting for its operands.
template <template <int> class PlanOf, int NS, int LA, class FBegin, class FOp, class FNext, class FMma,
          class FValu>
__device__ __forceinline__ void run_tile_carry(u32x4 (&carry)[LA], FBegin&& begin, FOp&& operand,
                                               FNext&& next, FMma&& mfma, FValu&& valu) {
  using T = typename TileStreamOf<PlanOf, std::make_integer_sequence<int, NS>>::type;
  using ic0 = std::integral_constant<int, 0>;
  static_assert(T::NOP >= LA, "a tile must have at least LA operands");
  u32x4 ops[LA + 1];
  static_for<LA>([&](auto oc) { ops[decltype(oc)::value] = carry[decltype(oc)::value]; });
  begin(ic0());
  static_for<T::NM>([&](auto mc) {
    constexpr int m = decltype(mc)::value, st = T::step_of_m(m), ml = m - T::m_base(st);
    using P = PlanOf<st>;
    using stc = std::integral_constant<int, st>;
    if constexpr (ml == 0 && st > 0) begin(stc());
    constexpr int o = T::o_base(st) + P::op_of(ml);
    mfma(stc(), std::integral_constant<int, ml>(), ops[o % (LA + 1)]);
    sched_fence();
    if constexpr (P::first(ml)) {
      constexpr int o2 = o + LA;
      if constexpr (o2 < T::NOP) {
        constexpr int st2 = T::step_of_o(o2);
        ops[o2 % (LA + 1)] = operand(std::integral_constant<int, st2>(),
                                     std::integral_constant<int, o2 - T::o_base(st2)>());
      } else {
        carry[o2 - T::NOP] = next(std::integral_constant<int, o2 - T::NOP>());
      }
    }
    valu(stc(), std::integral_constant<int, ml>(), mc);
    sched_fence();
  });
}

// Copy a wave's staged ROWS x D block (rows of D + 8 elements in LDS) to rows
// row0.. of a row-major [*, D] tensor in 16-byte pieces of whole rows, skipping
// rows at or past n_rows: lane L of round k moves granule 64 k + L of the block
// (row (64 k + L) / (D / 8)).
template <int D, int ROWS>
__device__ __forceinline__ void store_staged(const uint16_t* __restrict__ stage, uint16_t* __restrict__ dst,
                                             int row0, int n_rows, int lane) {
  constexpr int SS = D + 8;
  constexpr int CPR = D / 8;
  static_assert((ROWS * CPR) % 64 == 0, "whole rounds of 64 granules");
  if constexpr (64 % CPR == 0) {
    // whole rows per round: 64 / CPR rows of CPR granules
    constexpr int RPI = 64 / CPR;
#pragma unroll
    for (int k = 0; k < ROWS / RPI; ++k) {
      const int r = k * RPI + lane / CPR, c = lane % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * SS + 8 * c);
      if (row0 + r < n_rows) st16(dst + (size_t)(row0 + r) * D + 8 * c, v);
    }
  } else {
#pragma unroll
    for (int k = 0; k < ROWS * CPR / 64; ++k) {
      const int g = 64 * k + lane;
      const int r = g / CPR, c = g % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * SS + 8 * c);
      if (row0 + r < n_rows) st16(dst + (size_t)(row0 + r) * D + 8 * c, v);
    }
  }
}

// Store a wave's (16 RT) x D block held in 16x16 accumulators (acc[t][n] element i
// of lane (l16, j4) is row 16t + 4 j4 + i, column 16n + l16), times `scale`, to
// rows row0.. of a row-major [*, D] tensor; rows at or past n_rows are skipped.
// The block goes through the wave's own LDS staging area (16 RT rows of D + 8
// elements): 2-byte writes in the accumulator layout, then 16-byte row reads, so
// the global stores are whole 16-byte pieces of consecutive rows instead of
// 2-byte pieces of many rows each.
template <int DT, int D, int RT>
__device__ __forceinline__ void store_block_c16(const f32x4 (&acc)[RT][D / 16], float scale,
                                                uint16_t* __restrict__ stage, uint16_t* __restrict__ dst,
                                                int row0, int n_rows, int lane) {
  constexpr int SS = D + 8;
  const int l16 = lane & 15, j4 = lane >> 4;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        stage[(16 * t + 4 * j4 + i) * SS + 16 * n + l16] = Dt<DT>::one(acc[t][n][i] * scale);
    }
  }
  store_staged<D, 16 * RT>(stage, dst, row0, n_rows, lane);
}

// store_block_c16 with a scale per row: row 16t + 4 j4 + i of the lane's
// accumulators is multiplied by scale[t][i]; acc holds D / 16 head-dim tiles per
// query tile (further tiles are ignored).
template <int DT, int D, int RT, int NT>
__device__ __forceinline__ void store_block_rows(const f32x4 (&acc)[RT][NT], const float (&scale)[RT][4],
                                                 uint16_t* __restrict__ stage, uint16_t* __restrict__ dst,
                                                 int row0, int n_rows, int lane) {
  static_assert(NT >= D / 16, "a head-dim tile per 16 columns");
  constexpr int SS = D + 8;
  const int l16 = lane & 15, j4 = lane >> 4;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        stage[(16 * t + 4 * j4 + i) * SS + 16 * n + l16] = Dt<DT>::one(acc[t][n][i] * scale[t][i]);
    }
  }
  store_staged<D, 16 * RT>(stage, dst, row0, n_rows, lane);
}

}  // namespace fa
