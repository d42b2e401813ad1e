// Backward kernels of exact softmax attention.
//
//   bwd_dq    query-block-parallel dQ pass (the decomposition of the rustytorch
//             kernel's grid), recomputing S, P, dP and dS; writes dQ once.  It runs
//             first and also does the row preprocess of its rows: D_i = sum_d
//             dO_id O_id (rustytorch "flash_attention_backward.cu" computes this
//             row dot product inside its tiled kernel; the Triton issue "Extra
//             transposes cause 8x speedup for sequence-parallel Flash Attention
//             backward" loads it precomputed) and LSE in the log2 domain, stored
//             for the dK/dV kernel.
//   bwd_dkdv  key/value-block-parallel dK and dV (the Triton issue's _bwd_kernel
//             structure: one program per key block, K and V resident, a loop over
//             query blocks).
//   bwd_pre   the row preprocess as a kernel of its own, for the atomic dQ path,
//             which also needs its float32 dQ buffer cleared.
//   dq_convert  float32 dQ buffer -> dtype (atomic path).
//
// Per (query tile i, key tile j) the math is, with s the softmax scale:
//   S = s Q_i K_j^T,  P = exp(S - LSE_i),  dV_j += P^T dO_i,  dP = dO_i V_j^T,
//   dS = P o (dP - D_i),  dK_j += s dS^T Q_i,  dQ_i += s dS K_j.
// Exponentials run in the log2 domain: P = exp2(S * s * log2 e - LSE_i * log2 e).
//
// Both main kernels give each wave 64 resident rows (keys for dK/dV, queries for
// dQ; 32 at d = 256 and in the bias / dropout instances) so that every operand
// read from LDS feeds several MFMAs: all products are 16x16x32 MFMAs; an LDS
// operand of a score product (S, dP or their transposes) serves the 4 tiles of 16
// resident rows, and one of a gradient product serves every head-dim tile of the
// accumulator.  The streamed tile is processed in sub-blocks of 16 rows,
// software-pipelined so that the softmax / dS arithmetic of one sub-block runs
// while the matrix pipe works on the products of the next.
#pragma once

#include "fa_bwd_common.hpp"
#include "fa_pipeline.hpp"

#include <type_traits>

namespace fa {

// Step plans.  dK/dV: S_st | half of a dK product | dP_st | half of a dV product;
// the gradient products of a pair of sub-blocks (16x16x32 over their 32 query
// rows) are issued in halves (head-dim tiles) in the steps after the pair (dV
// from its second step on, dK one step later), so every step of a tile has the
// same shape; a flush step issues what is left after the last tile.
// dQ: S^T_st | half of a dQ product | dP^T_st.  The dQ product of a pair of
// sub-blocks (16x16x32, contraction over their 32 keys) is issued in two halves
// (head-dim tiles), in the two steps after the pair: steps 0-1 finish the previous
// tile's second pair, steps 2-3 this tile's first; a flush step issues both halves
// of the last pair.
template <int NK, int KT>
struct DkdvSteps {
  template <int ST>
  using P = StepPlan<NK, KT, NK, KT, NK, KT, NK, KT, 1>;
  template <int ST>
  using Flush = StepPlan<0, KT, 2 * NK, KT, 0, KT, NK, KT, 1>;
};
template <int NK, int QT>
struct DqSteps {
  template <int ST>
  using P = StepPlan<NK, QT, NK, QT, NK, QT, 0, 1, 1>;
  template <int ST>
  using Flush = StepPlan<0, QT, 2 * NK, QT, 0, QT, 0, 1, 1>;
};

// Resident rows per wave and LDS buffers per head dim and feature set: 64 rows
// (four 16-row tiles) and triple-buffered streamed tiles up to d = 128; above
// d = 128 the resident operands and accumulators of 64 rows exceed the 512
// registers of a lane, so a wave keeps 32 rows, and the streamed tiles stay
// triple-buffered while three buffers fit the 160 KB of LDS (d = 160 and 192;
// at 192 not with the dQ pass's key-bias slots), else double-buffered.  The bias
// and dropout instances take the 32-row shape too: the bias tiles need the LDS
// (two buffers), the bias and dropout work the registers.
template <int D, int FT = 0, bool KV = false>
struct TileShape {
  // KV: the dK/dV kernel, whose 64-row shape leaves no registers for dropout at
  // d = 128
  static constexpr bool SMALL = D > 128 || tile_bias(FT) || (KV && FT == FT_DROP && D > 64);
  static constexpr int RT = SMALL ? 2 : 4;    // resident 16-row tiles per wave
  // LDS buffers of the streamed tiles
  static constexpr int NBUF =
      !SMALL || (!tile_bias(FT) && (D == 160 || (D == 192 && (KV || FT != FT_KEYBIAS)))) ? 3 : 2;
};

// Slots of the non-MFMA work of dK/dV step ST (NC copies in steps 2-3):
//   exp[kt][i] (the exponentials of P_st), pack_p[kt] (odd ST), mul[kt][i] (dS_st),
//   pack_ds[kt] (odd ST), copy[c] (-1 where a step has no such item).
// Fixed: the deferred packs (even ST: P_st after the dV half's last read of the
// previous pair, slots NM-4+kt; odd ST: dS_{st-1} after the dK half's, slots
// B2-4+kt), the next step's LSE and -D reads, the mid-tile wait.
template <int NK, int KT, int ST, int LA, int NC>
struct DkdvPlace {
  using Plan = typename DkdvSteps<NK, KT>::template P<ST>;
  static constexpr int NM = Plan::NM;
  int exp[KT][4], pack_p[KT], mul[KT][4], pack_ds[KT], copy[NC];
  constexpr DkdvPlace() : exp(), pack_p(), mul(), pack_ds(), copy() {
    SlotLoad<NM> L;
    L.template reads<Plan, LA>();
    L.load[NM - 1] += 2 * issue::kRow + (ST == 1 ? 2 : 0);
    for (int kt = 0; kt < KT; ++kt) {
      if (ST % 2 == 0) L.load[NM - KT + kt] += issue::kPack;
      else L.load[Plan::B2 - KT + kt] += issue::kPack;
    }
    const int c0 = ST == 2 ? 0 : (NC + 1) / 2, c1 = ST == 2 ? (NC + 1) / 2 : NC;
    for (int c = 0; c < NC; ++c) copy[c] = -1;
    if (ST >= 2) {
      int prev = 0;
      L.level((c1 - c0) * issue::kCopy, 0, Plan::B1 - 1);
      for (int c = c0; c < c1; ++c) prev = copy[c] = L.put(issue::kCopy, prev, Plan::B1 - 1);
    }
    int prev = Plan::B1;
    L.level(4 * KT * issue::kExp + (ST % 2) * KT * issue::kPack, Plan::B1, Plan::B3 - 2);
    for (int kt = 0; kt < KT; ++kt) {
      for (int i = 0; i < 4; ++i) prev = exp[kt][i] = L.put(issue::kExp, prev, Plan::B3 - 2);
      pack_p[kt] = ST % 2 == 1 ? (prev = L.put(issue::kPack, prev, Plan::B3 - 2)) : -1;
    }
    prev = Plan::B3;
    L.level(4 * KT * issue::kMul + (ST % 2) * KT * issue::kPack, Plan::B3, NM - 1);
    for (int kt = 0; kt < KT; ++kt) {
      for (int i = 0; i < 4; ++i) prev = mul[kt][i] = L.put(issue::kMul, prev, NM - 1);
      pack_ds[kt] = ST % 2 == 1 ? (prev = L.put(issue::kPack, prev, NM - 1)) : -1;
    }
  }
};

// Slots of the non-MFMA work of dQ step ST (NC copies in steps 2-3):
//   mul[t][i], pack[t] (dS of the previous sub-block; the packs at least two slots
//   before the dQ half, which may read them), exp[t][i] (P_st), copy[c].
// EARLY: the copies go under the S^T MFMAs of steps 2-3 (double buffering waits
// for them before the last operand reads of the tile, which read the next tile).
template <int NK, int QT, int ST, int LA, int NC, bool EARLY>
struct DqPlace {
  using Plan = typename DqSteps<NK, QT>::template P<ST>;
  static constexpr int NM = Plan::NM;
  int mul[QT][4], pack[QT], exp[QT][4], copy[NC];
  constexpr DqPlace() : mul(), pack(), exp(), copy() {
    SlotLoad<NM> L;
    L.template reads<Plan, LA>();
    if (ST == 1) L.load[NM - 1] += 2;
    int prev = 0;
    L.level(4 * QT * issue::kMul + QT * issue::kPack, 0, Plan::B1 - 2);
    for (int t = 0; t < QT; ++t) {
      for (int i = 0; i < 4; ++i) prev = mul[t][i] = L.put(issue::kMul, prev, Plan::B1 - 2);
      prev = pack[t] = L.put(issue::kPack, prev, Plan::B1 - 2);
    }
    prev = Plan::B1;
    L.level(4 * QT * issue::kExp, Plan::B1, NM - 1);
    for (int t = 0; t < QT; ++t)
      for (int i = 0; i < 4; ++i) prev = exp[t][i] = L.put(issue::kExp, prev, NM - 1);
    const int c0 = ST == 2 ? 0 : (NC + 1) / 2, c1 = ST == 2 ? (NC + 1) / 2 : NC;
    for (int c = 0; c < NC; ++c) copy[c] = -1;
    if (ST >= 2) {
      const int hi = EARLY ? Plan::B1 - 1 : NM - 1;
      prev = 0;
      L.level((c1 - c0) * issue::kCopy, 0, hi);
      for (int c = c0; c < c1; ++c) prev = copy[c] = L.put(issue::kCopy, prev, hi);
    }
  }
};

// ---------------------------------------------------------------------------
// Row preprocess of the atomic dQ path (on the separate path the dQ pass does it
// for its own rows): -D, LSE * log2(e), the work-queue counters cleared and the
// float32 dQ buffer zeroed.  A row is handled by LPR lanes (D/8 rounded up to a
// power of two); lane `part` < D/8 reads 16 bytes of O and dO, the others add
// nothing.
template <int D>
constexpr int pre_lanes_per_row() {
  int n = 1;
  while (n < D / 8) n *= 2;
  return n;
}
template <int DT, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int LPR = pre_lanes_per_row<D>();
  constexpr int RPB = 256 / LPR;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  if (blockIdx.x == 0 && threadIdx.x < 32 && p.sched) p.sched[threadIdx.x] = 0;
  float s = 0.f;
  if (row < p.rows && part < D / 8) {
    const u32x4 a = ld16(p.o + row * D + part * 8);
    const u32x4 c = ld16(p.dout + row * D + part * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s += Dt<DT>::lo(a[j]) * Dt<DT>::lo(c[j]) + Dt<DT>::hi(a[j]) * Dt<DT>::hi(c[j]);
    {
      float* z = p.dq_acc + row * D + part * 8;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(z) = zero;
      *reinterpret_cast<f32x4*>(z + 4) = zero;
    }
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (row < p.rows && part == 0) {
    p.ndelta[row] = -s;
    const float L = p.lse[row];
    p.lse2[row] = (L == -INFINITY) ? INFINITY : L * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel.  Workgroup = 4 waves = 256 key rows of one (batch, kv head); wave w
// owns keys kvw = kv0 + 64w .. +63 and keeps
//   K and V as the B operands of S = Q K^T and dP = dO V^T (16x16x32; key tile kt
//   of 16 keys, contraction step s of 32 head dims), and
//   dK and dV as float32 16x16 accumulators (key tile kt, head-dim tile n).
// The loop runs over the G query heads of the group and their 64-row query tiles
// from the first one that can see the key block (causal) to the end.  Query tiles
// (Q, dO, LSE, D) are triple-buffered in LDS and copied straight from global
// memory two iterations ahead.  A tile is processed in four 16-row sub-blocks; per
// sub-block a wave computes
//   S (4 key tiles), P = exp2(S s log2e - LSE log2e), dP, dS = P o (dP - D),
// and per pair of sub-blocks dV += P^T dO and dK += dS^T Q (16x16x32, contraction
// over the pair's 32 query rows).  P and dS come out of the 16x16 accumulators
// with the key in the lane and four query rows of the sub-block in the elements;
// the packed tiles of the two sub-blocks side by side are the A operand's eight
// contraction slots, with no lane exchange.  The B operand (dO or Q with the same
// query rows along the slots) is two transposed LDS reads.  All MFMAs are
// 16x16x32, which under the power limit sustain a higher clock than 32x32x16.
//
// Sub-blocks are software-pipelined: step st issues the MFMA stream
//   S_st | half of a dK product | dP_st | half of a dV product
// with P_st computed under the dK half and dP_st, and dS_st under the dV half.
// The dV product of pair J runs in steps 2J+1 and 2J+2, its dK product in steps
// 2J+2 and 2J+3 (steps 4 and 5 are steps 0 and 1 of the next tile); a final step
// issues what is left of the last pair.  Tiles that cross the causal boundary or a
// ragged end of this wave's block take a masked variant of the softmax.
template <int DT, int D, bool CAUSAL, int FT>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr bool BIAS = tile_bias(FT), DROP = FT == FT_DROPOUT || FT == FT_DROP, KB = FT == FT_KEYBIAS;
  constexpr int KT = TileShape<D, FT, true>::RT;  // key tiles of 16 per wave
  constexpr int KW = 16 * KT, BN = 4 * KW, BM = 64, NSB = BM / 16;
  constexpr int NK = D / 32;
  constexpr int NBUF = TileShape<D, FT, true>::NBUF;
  constexpr int RS = PadTile<D>::RS;
  // bias tile of a query tile: BM rows x the workgroup's BN keys (4 pad granules a
  // row: 320-byte rows for BN = 128)
  using BiasDma = StridedTileDma<BM, BN, 4>;
  constexpr int BRS = BiasDma::RS;
  constexpr int BPW = BIAS ? BiasDma::PER_WAVE : 0;
  // copy instructions per fetch per wave: Q or dO, LSE, -D, bias
  constexpr int OPS = 2 * BM * PadTile<D>::GR / 256 + 2 + BPW;
  constexpr int LA = 2;                                     // operand lookahead
  // Q and dO of a buffer are one padded tile pair (as are LSE and D), so both are
  // read through the same per-lane address registers with immediate offsets.
  __shared__ __attribute__((aligned(16))) uint16_t sQdO[NBUF][2 * BM * RS];
  static_assert(NBUF * 2 * BM * RS >= 4 * KW * (D + 8), "the output staging must fit the tile buffers");
  __shared__ __attribute__((aligned(16))) float sLD[NBUF][2][BM];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BIAS ? NBUF : 1][BIAS ? BM * BRS : 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int l16 = lane & 15, j4 = lane >> 4;  // 16x16 tiles: column, row group
  __shared__ int s_item;
  const WorkQueue wq(p.sched, p.B * p.Hkv, (p.Nkv + BN - 1) / BN);
  long long ticket = tid == 0 ? wq.first() : 0;
  for (;;) {
    if (tid == 0) s_item = wq.resolve(ticket);
    lds_barrier();  // also: the previous item's staging reads are done
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item < 0 || item >= wq.n_items) break;
    const int rank = item / wq.n_heads, head = item % wq.n_heads;
    const int b = head / p.Hkv, hk = head % p.Hkv;
    const int kv0 = rank * BN;  // rank 0 = first key block = most query rows under the mask
    const int kvw = kv0 + KW * w;
    const size_t kbase = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;

    u32x4 kb[KT][NK], vb[KT][NK];
    {
      const uint16_t* __restrict__ K = p.k + kbase * D;
      const uint16_t* __restrict__ V = p.v + kbase * D;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int key = kvw + 16 * kt + l16;
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          kb[kt][s] = key < p.Nkv ? ld16(K + (size_t)key * D + 32 * s + 8 * j4) : zero_u4();
          vb[kt][s] = key < p.Nkv ? ld16(V + (size_t)key * D + 32 * s + 8 * j4) : zero_u4();
        }
      }
    }
    // key-bias instances: bias * log2(e) of this lane's key per key tile (the key is
    // the lane's column of every score tile)
    float bl[KB ? KT : 1];
    if constexpr (KB) {
      const uint16_t* __restrict__ brow = p.bias + (long long)b * p.bias_sb;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int key = kvw + 16 * kt + l16;
        bl[kt] = key < p.Nkv ? Dt<DT>::lo(brow[key]) * kLog2e : 0.f;
      }
    }
    f32x4 dk[KT][2 * NK], dv[KT][2 * NK];  // per key tile and 16-column head-dim tile
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int n = 0; n < 2 * NK; ++n) {
        dk[kt][n] = zero4();
        dv[kt][n] = zero4();
      }
    }

    const int q_begin = CAUSAL ? max(0, kv0 - p.off) : 0;
    const int nqt = (p.Nq + BM - 1) / BM;
    const int qt_begin = q_begin < p.Nq ? q_begin / BM : nqt;
    const int per_head = nqt - qt_begin;
    const int n_it = p.G * per_head;

    // Iteration it covers query tile nqt - 1 - it / G of query head it % G of the
    // group: tiles outer, last tile first, heads inner.  Every key block of a group
    // starts at the last query tile, so the workgroups of a group resident together
    // read the same query tiles at about the same time and share them through L2.
    //
    // Iteration it copies tile it + NBUF - 1 into the buffer of iteration it - 1; past
    // the last tile it copies the last tile again, into a buffer no later iteration
    // reads, so every iteration issues the same OPS copies per wave (spread over its
    // MFMA stream) and one vmcnt bound covers them.  Waves 0-1 copy the Q tile,
    // waves 2-3 the dO tile, each through a buffer resource based at the tile's first
    // row; rows past N_q arrive as zeros, and so do their LSE and -D, so without a
    // bias they add nothing to dK and dV.  Every wave copies LSE and -D (identical
    // bytes to the same place).
    using Copy = PadPairDma<D, BM>;
    struct Src {
      i32x4 t, l, d, bs;  // this wave's Q or dO tile; LSE*log2e; -D; bias (bias instances)
    };
    // Fetch cursor: the tile of iteration c_fit (query head c_hh of the group, rows
    // from the start of this wave's Q or dO tile, LSE and -D), moved one iteration
    // per copy round and held at the last one.
    const size_t row0 = ((size_t)b * p.Hq + (size_t)hk * p.G) * (size_t)p.Nq + (size_t)(nqt - 1) * BM;
    const uint16_t* __restrict__ ct = (w < 2 ? p.q : p.dout) + row0 * D;
    const float* __restrict__ cl = p.lse2 + row0;
    const float* __restrict__ cd = p.ndelta + row0;
    int c_left = p.Nq - (nqt - 1) * BM, c_hh = 0, c_fit = 0;
    // bias element offset of the cursor's tile: its first row, this block's first key
    long long cb = BIAS ? (long long)b * p.bias_sb + (long long)hk * p.G * p.bias_sh +
                              (long long)(nqt - 1) * BM * p.bias_sq + kv0
                        : 0;
    auto src_now = [&]() {
      Src sr;
      sr.t = buf_rsrc(ct, c_left * D * 2);
      sr.l = buf_rsrc(cl, c_left * 4);
      sr.d = buf_rsrc(cd, c_left * 4);
      if constexpr (BIAS) {
        // rows past N_q and a null bias read zeros (the resource ends there); a row is
        // read in whole 16-byte pieces, up to N_kv rounded up to 8 elements
        const int rows = min(BM, c_left);
        const int bytes = p.bias ? 2 * ((rows - 1) * (int)p.bias_sq + (((p.Nkv + 7) & ~7) - kv0)) : 0;
        sr.bs = buf_rsrc(p.bias ? p.bias + cb : p.k, bytes);
      }
      return sr;
    };
    auto advance = [&]() {
      if (c_fit < n_it - 1) {
        ++c_fit;
        if (++c_hh == p.G) {  // next (earlier) query tile of head 0
          c_hh = 0;
          const ptrdiff_t back = (ptrdiff_t)(p.G - 1) * p.Nq + BM;
          ct -= back * D;
          cl -= back;
          cd -= back;
          c_left += BM;
          if constexpr (BIAS) cb -= (long long)(p.G - 1) * p.bias_sh + (long long)BM * p.bias_sq;
        } else {
          ct += (size_t)p.Nq * D;
          cl += p.Nq;
          cd += p.Nq;
          if constexpr (BIAS) cb += p.bias_sh;
        }
      }
    };
    int voff[Copy::PER_WAVE];
#pragma unroll
    for (int c = 0; c < Copy::PER_WAVE; ++c) voff[c] = Copy::src_offset(c, w, lane);
    const uint32_t wave_off = Copy::lds_wave_offset(w);
    int voffb[BIAS ? BPW : 1];
    if constexpr (BIAS) {
#pragma unroll
      for (int c = 0; c < BPW; ++c) voffb[c] = BiasDma::src_offset(c, w, lane, (int)p.bias_sq);
    }
    auto copy_part = [&](auto cc, const Src& sr, int buf) {
      constexpr int c = decltype(cc)::value;
      if constexpr (c < Copy::PER_WAVE)
        bdma16<Copy::template lds_offset<c>>(voff[c], sr.t, lds_u32(sQdO[buf]) + wave_off);
      else if constexpr (c == Copy::PER_WAVE)
        bdma4(4 * lane, sr.l, lds_u32(sLD[buf][0]));
      else if constexpr (c == Copy::PER_WAVE + 1)
        bdma4(4 * lane, sr.d, lds_u32(sLD[buf][1]));
      else {
        constexpr int cb_ = c - Copy::PER_WAVE - 2;
        bdma16<BiasDma::template lds_offset<cb_>>(voffb[cb_], sr.bs,
                                                  lds_u32(sB[buf]) + BiasDma::lds_wave_offset(w));
      }
    };
    auto copy_all = [&](const Src& sr, int buf) {
      static_for<OPS>([&](auto cc) { copy_part(cc, sr, buf); });
    };

    // Carried from tile to tile: the first LA operands of the next tile, and the
    // packed P^T and dS^T of the second sub-block pair, whose dV and dK products run
    // in steps 0-1 of the next tile with dO and Q read from the previous buffer
    // (zero before the first tile, which makes those products no-ops).
    //
    // pa[J][kt] / sa[J][kt]: A operand of the dV / dK product of sub-block pair J
    // for key tile kt: slots 0-3 the packed P^T (dS^T) of sub-block 2J (queries
    // 4 j4 .. + 3 for this lane's key), slots 4-7 those of sub-block 2J + 1.  The
    // first half of a pair is packed only once the previous pair's tuple has been
    // read for the last time, so the two pairs can share registers.
    u32x4 carry[LA];
    u32x4 pa[2][KT], sa[2][KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      pa[1][kt] = zero_u4();
      sa[1][kt] = zero_u4();
    }
    int prev = 0;  // buffer of the previous tile

    // Operand o of step st of a tile in buffer Q_ (Q, then dO) whose previous tile
    // is in buffer Qp_ (the operand order of DkdvSteps; see compute below).
    auto dkdv_operand = [&](auto stc, auto oc, const uint16_t* Q_, const uint16_t* Qp_) -> u32x4 {
      constexpr int st = decltype(stc)::value, o = decltype(oc)::value;
      using Plan = typename DkdvSteps<NK, KT>::template P<st>;
      constexpr int k = Plan::op_stage(o), n = Plan::op_local(o);
      const uint16_t* dO_ = Q_ + BM * RS;
      const uint16_t* dOp_ = Qp_ + BM * RS;
      if constexpr (k == 0) {
        return pad_row16<D>(Q_, 16 * st + l16, 4 * n + j4);
      } else if constexpr (k == 1) {
        constexpr int J = st < 2 ? 1 : 0, nn = (st % 2) * NK + n;
        const int k0 = 32 * J + 4 * j4;
        return pad_tr_operand<D>(st < 2 ? Qp_ : Q_, k0, k0 + 16, 16 * nn);
      } else if constexpr (k == 2) {
        return pad_row16<D>(dO_, 16 * st + l16, 4 * n + j4);
      } else {
        constexpr int J = (st == 0 || st == 3) ? 1 : 0, nn = ((st + 1) % 2) * NK + n;
        const int k0 = 32 * J + 4 * j4;
        return pad_tr_operand<D>(st == 0 ? dOp_ : dO_, k0, k0 + 16, 16 * nn);
      }
    };

    auto compute = [&](int cur, int nxt, auto mask_c, int q0, int hq, const Src& fsrc, int fbuf) {
      constexpr bool MASK = decltype(mask_c)::value;
      const uint16_t* Qt = sQdO[cur];
      const uint16_t* Qp = sQdO[prev];
      const uint16_t* Qn = sQdO[nxt];
      const float* Lt = sLD[cur][0];
      const float* Dtl = Lt + BM;
      f32x4 sc[KT];   // S, then P, of the current sub-block, per key tile
      f32x4 dp[KT];   // dP, then dS
      f32x4 lq, dn;   // LSE*log2e and -D of the current sub-block's rows
      u32x2 bv[KT];   // bias of the current sub-block per key tile (rows in elements)
      f32x4 zf[KT];   // dropout keep factors of the current sub-block per key tile
      u32x4 kw;       // keep bytes of this lane's key in the blocks drawn last
      static_assert(!DROP || KT == 4 || (KT == 2 && NSB % 2 == 0), "dropout block draw");
      (void)hq;
      const int keyl = kvw + l16;    // key of this lane's column in key tile 0
      const int qrow = q0 + 4 * j4;  // query row of element 0 in sub-block 0

      using Steps = DkdvSteps<NK, KT>;
      // packed sub-block st into half st % 2 of pair st / 2
      auto pack_p = [&](auto stc, auto ktc) {
        constexpr int st = decltype(stc)::value, kt = decltype(ktc)::value;
        // dV is weighted by the kept probabilities P o Z
        u32x2 v = pack_c4<DT>(DROP ? sc[kt] * zf[kt] : sc[kt]);
        pin<FT != FT_PLAIN>(v);
        pa[st / 2][kt][2 * (st % 2)] = v[0];
        pa[st / 2][kt][2 * (st % 2) + 1] = v[1];
      };
      auto pack_ds = [&](auto stc, auto ktc) {
        constexpr int st = decltype(stc)::value, kt = decltype(ktc)::value;
        u32x2 v = pack_c4<DT>(dp[kt]);
        pin<FT != FT_PLAIN>(v);
        sa[st / 2][kt][2 * (st % 2)] = v[0];
        sa[st / 2][kt][2 * (st % 2) + 1] = v[1];
      };
      // P_st item e of 4 KT (key tile e / 4, row e % 4)
      auto p_item = [&](auto ec, auto st_c) {
        constexpr int e = decltype(ec)::value, st = decltype(st_c)::value;
        constexpr int kt = e / 4, i = e % 4;
        if constexpr (DROP && i == 0) {
          // One Philox call per 4 x 4 block (keys k & ~3 .., rows 0..3 of a row group):
          // word r is row r, byte k % 4 the key.  The four lanes of a key quad share
          // their blocks, so lane j of the quad draws one of them (key tile j % KT of
          // sub-block st + j / KT; with two key tiles, the even step draws the odd
          // step's blocks too) and a byte and quad transpose give every lane its bytes:
          // word w, byte r = row r of block w of this lane's key.
          constexpr bool DRAW = kt == 0 && st % (4 / KT) == 0;
          if constexpr (DRAW) {
            const int q4 = l16 & 3, bkt = q4 % KT, bst = st + q4 / KT;
            const u32x4 ctr = {(uint32_t)(keyl + 16 * bkt) >> 2, (uint32_t)(qrow + 16 * bst) >> 2,
                               (uint32_t)hq, (uint32_t)b};
            kw = quad_transpose(byte_transpose(philox4x32_10(ctr, p.seed_lo, p.seed_hi)), q4);
          }
          const uint32_t word = kw[KT == 4 ? kt : 2 * (st % 2) + kt];
#pragma unroll
          for (int r = 0; r < 4; ++r) zf[kt][r] = keep_factor(word, r, p.keep_t, p.drop_scale);
        }
        float v;
        if constexpr (BIAS)
          v = fmaf(sc[kt][i], p.scale_log2, fmaf(elem4<DT>(bv[kt], i), kLog2e, -lq[i]));
        else if constexpr (KB)
          v = fmaf(sc[kt][i], p.scale_log2, bl[kt] - lq[i]);
        else
          v = sc[kt][i] * p.scale_log2 - lq[i];
        if constexpr (MASK && (BIAS || KB)) {
          // a bias could make the P of a row past N_q overflow the 16-bit type (and
          // inf * 0 is NaN): every bound
          const int key = keyl + 16 * kt, q = qrow + 16 * st + i;
          if (key >= p.Nkv || q >= p.Nq || (CAUSAL && key > q + p.off)) v = -INFINITY;
        } else if constexpr (MASK && CAUSAL) {
          // Only the causal bound.  A key past N_kv only feeds its own dK and dV rows,
          // which are not stored.  A row past N_q has zero Q, dO, LSE and -D, so its
          // P is 1 and its terms of dV (P^T dO) and dK (dS^T Q) vanish.
          const int key = keyl + 16 * kt, q = qrow + 16 * st + i;
          if (key > q + p.off) v = -INFINITY;
        }
        sc[kt][i] = fast_exp2(v);
      };

      auto begin = [&](auto stc) {
        constexpr int st = decltype(stc)::value;
        lq = *reinterpret_cast<const f32x4*>(&Lt[16 * st + 4 * j4]);
        dn = *reinterpret_cast<const f32x4*>(&Dtl[16 * st + 4 * j4]);
        if constexpr (BIAS) {
          // the bias of the 16x16 S tiles of this sub-block in their C layout: one
          // transposed read per key tile (lane l16 addresses row l16 / 4 of its row
          // group and receives column l16)
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
            bv[kt] = lds_tr16(sB[cur] + (16 * st + 4 * j4 + (l16 >> 2)) * BRS + KW * w + 16 * kt +
                              4 * (l16 & 3));
        }
        if constexpr (st == 2) {
          // Mid-tile: every wave is past steps 0-1 (its last reads of the previous
          // buffer) and, once its own copies have landed, the next tile is complete
          // (triple buffering), so the copies of steps 2-3 may refill the previous
          // buffer.
          wait_vmem();
          tile_barrier();
        }
      };
      // Stage 1 of step st: half st % 2 of the dK product of pair 1 of the previous
      // tile (steps 0-1) or pair 0 of this one (steps 2-3).  Stage 3: half
      // (st + 1) % 2 of the dV product of pair 0 (steps 1-2) or pair 1 (step 3, and
      // of the previous tile in step 0).
      auto operand = [&](auto stc, auto oc) -> u32x4 {
        return dkdv_operand(stc, oc, Qt, Qp);
      };
      // operand oc of the next tile, whose previous buffer is this one
      auto next = [&](auto oc) -> u32x4 {
        if constexpr (NBUF == 2 && decltype(oc)::value == 0) {
          // double buffering: the next tile was copied in this tile's second half
          wait_vmem();
          tile_barrier();
        }
        return dkdv_operand(std::integral_constant<int, 0>(), oc, Qn, Qt);
      };
      auto mfma = [&](auto stc, auto mc, const u32x4& op) {
        constexpr int st = decltype(stc)::value, m = decltype(mc)::value;
        using Plan = typename Steps::template P<st>;
        constexpr int k = Plan::stage(m), loc = Plan::local(m), o = loc / KT, kt = loc % KT;
        if constexpr (k == 0) {
          if constexpr (o == 0)
            sc[kt] = Mx<DT>::first16(op, kb[kt][o]);
          else
            Mx<DT>::acc16(sc[kt], op, kb[kt][o]);
        } else if constexpr (k == 1) {
          constexpr int J = st < 2 ? 1 : 0, nn = (st % 2) * NK + o;
          Mx<DT>::acc16a(dk[kt][nn], sa[J][kt], op);
        } else if constexpr (k == 2) {
          // dP - D (dropout: dP alone, as the keep factors apply to dP before D)
          if constexpr (o == 0 && DROP)
            dp[kt] = Mx<DT>::first16(op, vb[kt][o]);
          else if constexpr (o == 0)
            dp[kt] = Mx<DT>::first16c(op, vb[kt][o], dn);
          else
            Mx<DT>::acc16(dp[kt], op, vb[kt][o]);
        } else {
          constexpr int J = (st == 0 || st == 3) ? 1 : 0, nn = ((st + 1) % 2) * NK + o;
          Mx<DT>::acc16a(dv[kt][nn], pa[J][kt], op);
        }
      };
      auto valu = [&](auto stc, auto mc, auto gc) {
        constexpr int st = decltype(stc)::value, m = decltype(mc)::value;
        using Plan = typename Steps::template P<st>;
        using stp = std::integral_constant<int, st>;
        constexpr DkdvPlace<NK, KT, st, LA, OPS> PL{};
        static_assert(!DROP || none_before(PL.exp, PL.exp[0][0]), "key tile 0 draws the dropout blocks");
        (void)gc;
        // The copies of a later tile, in steps 2-3 (after the mid-tile barrier).
        static_for<OPS>([&](auto cc) {
          if constexpr (PL.copy[decltype(cc)::value] == m) copy_part(cc, fsrc, fbuf);
        });
        // P_st under the dK half and dP_st: four exponentials per key tile, then
        // (odd st) the packed tile, before the dV half reads it
        static_for<KT>([&](auto ktc) {
          constexpr int kt = decltype(ktc)::value;
          static_for<4>([&](auto ic) {
            if constexpr (PL.exp[kt][decltype(ic)::value] == m)
              p_item(std::integral_constant<int, 4 * kt + decltype(ic)::value>(), stp());
          });
          if constexpr (PL.pack_p[kt] == m) pack_p(stp(), ktc);
        });
        // dS_st under the dV half; odd st packs it at once
        static_for<KT>([&](auto ktc) {
          constexpr int kt = decltype(ktc)::value;
          static_for<4>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (PL.mul[kt][i] == m) {
              if constexpr (DROP)
                dp[kt][i] = sc[kt][i] * fmaf(zf[kt][i], dp[kt][i], dn[i]);  // P o (Z o dP - D)
              else
                dp[kt][i] = sc[kt][i] * dp[kt][i];  // the dP product starts from -D
            }
          });
          if constexpr (PL.pack_ds[kt] == m) pack_ds(stp(), ktc);
        });
        // even st: P_st is packed into a new pair once the dV half of this step has
        // read key tile kt of the previous pair for the last time, and dS_{st-1}
        // once the dK half has done the same
        if constexpr (st % 2 == 0 && m >= Plan::NM - KT)
          pack_p(stp(), std::integral_constant<int, m - (Plan::NM - KT)>());
        if constexpr (st % 2 == 1 && m >= Plan::B2 - KT && m < Plan::B2)
          pack_ds(std::integral_constant<int, st - 1>(), std::integral_constant<int, m - (Plan::B2 - KT)>());
      };
      run_tile_carry<Steps::template P, NSB, LA>(carry, begin, operand, next, mfma, valu);
    };
    // The dV and dK products of the last computed tile's second pair (no-ops when
    // no tile was computed; skipped when no tile was even copied, as the buffers
    // then hold no data).
    auto flush = [&]() {
      const uint16_t* Qp = sQdO[prev];
      const uint16_t* dOp = Qp + BM * RS;
      using Steps = DkdvSteps<NK, KT>;
      using Plan = typename Steps::template Flush<0>;
      run_tile<Steps::template Flush, 1, LA>(
          [&](auto) {},
          [&](auto, auto oc) -> u32x4 {
            constexpr int o = decltype(oc)::value, k = Plan::op_stage(o), n = Plan::op_local(o);
            const int k0 = 32 + 4 * j4;
            return k == 1 ? pad_tr_operand<D>(Qp, k0, k0 + 16, 16 * n)
                          : pad_tr_operand<D>(dOp, k0, k0 + 16, 16 * (NK + n));
          },
          [&](auto, auto mc, const u32x4& op) {
            constexpr int m = decltype(mc)::value, k = Plan::stage(m), loc = Plan::local(m);
            constexpr int o = loc / KT, kt = loc % KT;
            if constexpr (k == 1)
              Mx<DT>::acc16a(dk[kt][o], sa[1][kt], op);
            else
              Mx<DT>::acc16a(dv[kt][NK + o], pa[1][kt], op);
          },
          [&](auto, auto, auto) {});
    };

    // This wave's split of the query tiles (each phase runs one variant of the
    // math, so the loops carry the accumulators without branches around MFMAs);
    // in iteration order:
    //   [qe, nqt)       ragged query end                      masked
    //   [qb, qe)        every pair visible                    unmasked
    //   [qa, qb)        causal boundary or ragged key end     masked
    //   [qt_begin, qa)  no query sees the wave's keys         skipped
    int qa = qt_begin, qb = qt_begin, qe = nqt;
    if (kvw >= p.Nkv) {
      qa = qb = qe = nqt;
    } else {
      if (CAUSAL) {
        qa = max(qt_begin, floor_div(kvw - p.off - (BM - 1) + BM - 1, BM));  // q0 + BM - 1 >= kvw - off
        qb = max(qa, floor_div(kvw + KW - 1 - p.off + BM - 1, BM));        // q0 >= kvw + KW - 1 - off
      }
      if (kvw + KW > p.Nkv) qb = nqt;  // ragged key end: every visible tile is masked
      qa = min(qa, nqt);
      qb = min(qb, nqt);
      qe = max(qb, min(nqt, p.Nq / BM));
    }
    if (n_it > 0) {
      static_for<NBUF - 1>([&](auto bc) {
        copy_all(src_now(), decltype(bc)::value);
        advance();
      });
    }
    // The register preloads and the first tiles' copies are in flight together.  The
    // copies are not visible to the compiler's wait counting, so everything is waited
    // for here: the compiler then knows the preloads have landed and puts no wait of
    // its own (which would count the copies wrongly) into the loop.
    wait_vmem();
    lds_barrier();
    // the first tile's leading operands (its "previous" buffer is the same one; the
    // previous-pair products it feeds are multiplied by zeros)
    static_for<LA>([&](auto oc) {
      carry[decltype(oc)::value] = dkdv_operand(std::integral_constant<int, 0>(), oc, sQdO[0], sQdO[0]);
    });
    // Iteration it works on buffer it % NBUF; from its middle on it copies tile
    // it + NBUF - 1 into the buffer of iteration it - 1.
    int it = 0, cur = 0;
    auto phase = [&](int qt_low, auto variant) {  // down to query tile qt_low
      constexpr int VAR = decltype(variant)::value;  // 0 skip, 1 masked, 2 unmasked
      for (const int end = (nqt - qt_low) * p.G; it < end; ++it) {
        const Src fsrc = src_now();  // tile it + NBUF - 1
        advance();
        const int fbuf = cur == 0 ? NBUF - 1 : cur - 1;
        const int nxt = cur == NBUF - 1 ? 0 : cur + 1;
        const int q0 = (nqt - 1 - it / p.G) * BM;
        const int hq = hk * p.G + it % p.G;  // query head of this iteration
        if constexpr (VAR == 0) {
          wait_vmem();
          tile_barrier();
          copy_all(fsrc, fbuf);
          if constexpr (NBUF == 2) {  // the second barrier a computed tile has
            wait_vmem();
            tile_barrier();
          }
        }
        if constexpr (VAR == 1) compute(cur, nxt, std::true_type(), q0, hq, fsrc, fbuf);
        if constexpr (VAR == 2) compute(cur, nxt, std::false_type(), q0, hq, fsrc, fbuf);
        prev = cur;
        cur = nxt;
      }
    };
    phase(qe, std::integral_constant<int, 1>());
    phase(qb, std::integral_constant<int, 2>());
    phase(qa, std::integral_constant<int, 1>());
    if (n_it > 0) flush();
    phase(qt_begin, std::integral_constant<int, 0>());
    wait_vmem();    // no copy may land in LDS after the tile buffers are reused below
    lds_barrier();  // every wave is done with the tile buffers
    // The next item is claimed only now, after the last wait for memory: the stores
    // below hide the atomic's latency (claimed at the start, it would be waited for
    // with the item's first loads, and the assignment fixed a whole item ahead).
    if (tid == 0) ticket = wq.next_ticket(ticket);
    settle(dk);
    settle(dv);
    uint16_t* stage = &sQdO[0][0] + w * KW * (D + 8);
    store_block_c16<DT, D, KT>(dk, p.scale, stage, p.dk + kbase * D, kvw, p.Nkv, lane);
    store_block_c16<DT, D, KT>(dv, 1.f, stage, p.dv + kbase * D, kvw, p.Nkv, lane);
  }
}

// ---------------------------------------------------------------------------
// Separate dQ pass.  Workgroup = 4 waves = 256 query rows of one (batch, query
// head); wave w owns queries qw = q0 + 64w .. +63 and keeps
//   Q and dO as the B operands of S^T = K Q^T and dP^T = V dO^T (16x16x32; query
//   tile t of 16 queries, contraction step s of 32 head dims), their LSE and D,
//   and dQ as float32 16x16 accumulators (query tile t, head-dim tile n).
// Key/value tiles of 64 rows are triple-buffered in LDS and copied straight from
// global memory.  A tile is processed in four 16-key sub-blocks; per sub-block a
// wave computes S^T and dP^T (4 query tiles), P^T and dS^T.  Per pair of
// sub-blocks it adds dQ += dS K (16x16x32 over the pair's 32 keys): a lane holds
// keys 4 j4 .. 4 j4 + 3 of each sub-block for its query, which, put side by side,
// are its 8 contraction slots, so the A operand is the two packed dS tiles as they
// are; the B operand (K with the same keys along the slots) is two transposed LDS
// reads.  All MFMAs are 16x16x32, which under the power limit sustain a higher
// clock than 32x32x16 ones.
//
// Step st issues the MFMA stream  S^T_st | dQ half | dP^T_st  with dS_{st-1}
// computed under S^T_st and P_st under the dQ half and dP^T_st.
// DBW (bias instances): dBias chunks of 4 keys stored as one 8-byte piece, which
// needs N_kv % 4 == 0 (8-byte aligned rows, and no chunk straddles a row end);
// otherwise each key is stored on its own.
template <int DT, int D, bool CAUSAL, int FT, bool DBW = false>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdParams p) {
  constexpr bool BIAS = tile_bias(FT), DROP = FT == FT_DROPOUT || FT == FT_DROP, KB = FT == FT_KEYBIAS;
  constexpr int QT = TileShape<D, FT>::RT;  // query tiles of 16 per wave
  constexpr int QW = 16 * QT, BM = 4 * QW, BN = 64, NSB = BN / 16;
  constexpr int NK = D / 32;
  constexpr int NBUF = TileShape<D, FT>::NBUF;  // key/value tiles fetched NBUF - 1 ahead
  constexpr int RS = PadTile<D>::RS;
  // bias tile of a key tile: the workgroup's BM queries x BN keys (2 pad granules a
  // row: 160-byte rows)
  using BiasDma = StridedTileDma<BM, BN, 2>;
  constexpr int BRS = BiasDma::RS;
  constexpr int BPW = BIAS ? BiasDma::PER_WAVE : 0;
  constexpr int KVPW = 2 * BN * PadTile<D>::GR / 256;
  // copy instructions per fetch per wave: K or V, bias tile, key-bias row
  constexpr int OPS = KVPW + BPW + (KB ? 1 : 0);
  constexpr int LA = 2;
  __shared__ __attribute__((aligned(16))) uint16_t sKV[NBUF][2 * BN * RS];  // K, V: a padded pair
  __shared__ __attribute__((aligned(16))) uint16_t sB[BIAS ? NBUF : 1][BIAS ? BM * BRS : 8];
  // key-bias instances: each wave's copy of the tile's keys' bias (keys k0 .. k0 + 63
  // in its first 128 bytes; a 16-byte-per-lane copy fills 1 KB)
  __shared__ __attribute__((aligned(16))) uint16_t sKB[KB ? NBUF : 1][KB ? 4 * 512 : 8];
  static_assert(NBUF * 2 * BN * RS >= 4 * QW * (D + 8), "the output staging must fit the tile buffers");

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int l16 = lane & 15, j4 = lane >> 4;
  const int nqt = (p.Nq + BM - 1) / BM;
  __shared__ int s_item;
  const WorkQueue wq(p.sched ? p.sched + 16 : nullptr, p.B * p.Hq, nqt);
  long long ticket = tid == 0 ? wq.first() : 0;
  for (;;) {
    if (tid == 0) s_item = wq.resolve(ticket);
    lds_barrier();  // also: the previous item's staging reads are done
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item < 0 || item >= wq.n_items) break;
    const int rank = item / wq.n_heads, head = item % wq.n_heads;
    const int qt = CAUSAL ? nqt - 1 - rank : rank;
    const int b = head / p.Hq, h = head % p.Hq;
    const int hk = h / p.G;
    const int q0 = qt * BM;
    const int qw = q0 + QW * w;  // first query row of this wave
    const size_t qbase = ((size_t)b * p.Hq + h) * (size_t)p.Nq;
    const size_t kbase = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;
    const uint16_t* __restrict__ K = p.k + kbase * D;
    const uint16_t* __restrict__ V = p.v + kbase * D;

    // The row preprocess of this item's query rows: D = rowsum(dO o O) and
    // LSE * log2(e) (+inf for a row that sees no key), kept for the softmax here
    // and stored at the end of the item for the dK/dV kernel, which runs after
    // this pass.  A query row's head dims are spread over the four lanes
    // j4 = 0..3 of its column, as its Q and dO operands are.  O is loaded with the
    // other preloads and D formed after the one wait for them below.
    u32x4 qb[QT][NK], db[QT][NK], ob[QT][NK];
    float lq[QT];
    f32x4 nd[QT];  // -D of the lane's query, in every element: where dP^T starts
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int q = qw + 16 * t + l16;
      const bool ok = q < p.Nq;
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        qb[t][s] = ok ? ld16(p.q + (qbase + q) * D + 32 * s + 8 * j4) : zero_u4();
        db[t][s] = ok ? ld16(p.dout + (qbase + q) * D + 32 * s + 8 * j4) : zero_u4();
        ob[t][s] = ok ? ld16(p.o + (qbase + q) * D + 32 * s + 8 * j4) : zero_u4();
      }
      const float L = ok ? p.lse[qbase + q] : -INFINITY;
      lq[t] = L == -INFINITY ? INFINITY : L * kLog2e;
    }
    f32x4 acc[QT][2 * NK];  // dQ, per query tile and 16-column head-dim tile
#pragma unroll
    for (int t = 0; t < QT; ++t) {
#pragma unroll
      for (int n = 0; n < 2 * NK; ++n) acc[t][n] = zero4();
    }


    int kv_end = p.Nkv;
    if (CAUSAL) {
      const int q_last = min(q0 + BM, p.Nq) - 1;
      kv_end = min(p.Nkv, q_last + p.off + 1);
    }
    const int nkt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;

    // Iteration kt copies key/value tile kt + NBUF - 1 into the buffer of iteration
    // kt - 1 (past the last tile, the last tile again, into a buffer no later
    // iteration reads), OPS copies per wave spread over its MFMA stream.  Waves 0-1
    // copy the K tile, waves 2-3 the V tile, through a buffer resource based at the
    // tile's first row; rows past N_kv arrive as zeros (and are masked in the math).
    using Copy = PadPairDma<D, BN>;
    static_assert(Copy::PER_WAVE == KVPW, "key/value copies per wave");
    const uint16_t* __restrict__ tsrc = w < 2 ? K : V;
    struct Src {
      i32x4 t, bs;  // this wave's K or V tile; bias tile or key-bias row (bias instances)
    };
    // bias element offset of this item's first query row (key 0)
    const long long bq0 = BIAS ? (long long)b * p.bias_sb + (long long)h * p.bias_sh +
                                     (long long)q0 * p.bias_sq
                               : KB ? (long long)b * p.bias_sb : 0;
    auto src_of = [&](int kt) {
      const int k0 = min(kt, nkt - 1) * BN;
      Src sr;
      sr.t = buf_rsrc(tsrc + (size_t)k0 * D, (p.Nkv - k0) * D * 2);
      if constexpr (BIAS) {
        // rows past N_q and a null bias read zeros (the resource ends there); a row is
        // read in whole 16-byte pieces, up to N_kv rounded up to 8 elements
        const int rows = min(BM, p.Nq - q0);
        const int bytes = p.bias ? 2 * ((rows - 1) * (int)p.bias_sq + (((p.Nkv + 7) & ~7) - k0)) : 0;
        sr.bs = buf_rsrc(p.bias ? p.bias + bq0 + k0 : p.k, bytes);
      }
      if constexpr (KB) {
        // the row of batch b from key k0, readable up to N_kv rounded up to 8
        sr.bs = buf_rsrc(p.bias + bq0 + k0, 2 * (((p.Nkv + 7) & ~7) - k0));
      }
      return sr;
    };
    int voff[Copy::PER_WAVE];
#pragma unroll
    for (int c = 0; c < Copy::PER_WAVE; ++c) voff[c] = Copy::src_offset(c, w, lane);
    const uint32_t wave_off = Copy::lds_wave_offset(w);
    int voffb[BIAS ? BPW : 1];
    if constexpr (BIAS) {
#pragma unroll
      for (int c = 0; c < BPW; ++c) voffb[c] = BiasDma::src_offset(c, w, lane, (int)p.bias_sq);
    }
    auto copy_part = [&](auto cc, const Src& sr, int buf) {
      constexpr int c = decltype(cc)::value;
      if constexpr (c < KVPW) {
        bdma16<Copy::template lds_offset<c>>(voff[c], sr.t, lds_u32(sKV[buf]) + wave_off);
      } else if constexpr (KB) {
        bdma16<0>(16 * lane, sr.bs, lds_u32(sKB[buf]) + 1024 * w);
      } else {
        constexpr int cb_ = c - KVPW;
        bdma16<BiasDma::template lds_offset<cb_>>(voffb[cb_], sr.bs,
                                                  lds_u32(sB[buf]) + BiasDma::lds_wave_offset(w));
      }
    };
    auto copy_all = [&](int kt, int buf) {
      const Src sr = src_of(kt);
      static_for<OPS>([&](auto cc) { copy_part(cc, sr, buf); });
    };
    // dS^T of a finished sub-block (packed: keys key0 .. key0 + 3 of query q) into
    // dBias = dS, row q of this head, through a resource over this item's rows:
    // rows past N_q fall past its end, and elements with a key past N_kv, or of the
    // sub-block "before" the first tile (key0 < 0, all zeros), get an offset past
    // it, so no branch splits the MFMA stream (which would make the register
    // allocator move the AGPR accumulators).
    const i32x4 dbr = BIAS && p.dbias
                          ? buf_rsrc(p.dbias + (qbase + q0) * (size_t)p.Nkv,
                                     2 * min(BM, p.Nq - q0) * p.Nkv)
                          : buf_rsrc(p.k, 0);
    auto store_dbias = [&](const u32x2& v, int q, int key0) {
      const int base = 2 * ((q - q0) * p.Nkv + key0);
      if constexpr (DBW) {
        // key0 and N_kv are multiples of 4: the chunk is wholly in or out of the row
        bstore64(v, key0 >= 0 && key0 < p.Nkv ? base : 0x7ffffff0, dbr);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = key0 + r >= 0 && key0 + r < p.Nkv;
          const int off = ok ? base + 2 * r : 0x7ffffff0;
          if (r & 1)
            bstore16_hi(v[r >> 1], off, dbr);
          else
            bstore16_lo(v[r >> 1], off, dbr);
        }
      }
    };

    // key-bias instances: bias / scale of keys 4 j4 .. + 3 of sub-block sb of the
    // tile in buffer buf, the accumulator the S^T product starts from (so that
    // c (S + b / scale) = c S + b log2 e); cbk[sb % 2] for sub-block sb, filled one
    // step ahead
    auto key_bias = [&](int buf, int sb) -> f32x4 {
      const u32x2 v = *reinterpret_cast<const u32x2*>(sKB[buf] + 512 * w + 16 * sb + 4 * j4);
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = elem4<DT>(v, i) * p.inv_scale;
      return r;
    };
    f32x4 cbk[2];

    // Carried from tile to tile: the first LA operands of the next tile, P^T and
    // dP^T of the last sub-block (sc[1], dp), whose dS^T is computed in step 0 of
    // the next tile, and the packed dS of the second pair (da[1]), whose dQ product
    // runs in steps 0-1 of the next tile with K read from the previous buffer (zero
    // before the first tile, which makes that product a no-op).
    u32x4 carry[LA];
    f32x4 sc[2][QT];  // S^T, then P^T, of sub-block st in sc[st % 2], per query tile
    f32x4 dp[QT];     // dP^T, then dS^T, of the sub-block being finished
    u32x4 da[2][QT];  // dS A operands of sub-block pair J, per query tile
    f32x4 zf[2][QT];  // dropout keep factors of sub-block st in zf[st % 2]
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      sc[1][t] = zero4();
      dp[t] = zero4();
      da[1][t] = zero_u4();
      zf[1][t] = zero4();
    }
    int prev = 0;     // buffer of the previous tile
    int kv_last = 0;  // first key of the last computed tile

    // Operand o of step st of a tile in buffer K_ (K, then V) whose previous tile is
    // in buffer Kp_ (the operand order of DqSteps).  Stage 1: half st % 2 of the dQ
    // product of pair 1 of the previous tile (steps 0-1) or pair 0 of this one
    // (steps 2-3): keys 4 j4 .. + 3 of both sub-blocks of the pair, head-dim tile
    // (st % 2) NK + n.
    auto dq_operand = [&](auto stc, auto oc, const uint16_t* K_, const uint16_t* Kp_) -> u32x4 {
      constexpr int st = decltype(stc)::value, o = decltype(oc)::value;
      using Plan = typename DqSteps<NK, QT>::template P<st>;
      constexpr int k = Plan::op_stage(o), n = Plan::op_local(o);
      if constexpr (k == 0) {
        return pad_row16<D>(K_, 16 * st + l16, 4 * n + j4);
      } else if constexpr (k == 1) {
        constexpr int J = st < 2 ? 1 : 0, nn = (st % 2) * NK + n;
        const int k0 = 32 * J + 4 * j4;
        return pad_tr_operand<D>(st < 2 ? Kp_ : K_, k0, k0 + 16, 16 * nn);
      } else {
        return pad_row16<D>(K_ + BN * RS, 16 * st + l16, 4 * n + j4);
      }
    };

    auto compute = [&](int cur, int nxt, auto mask_c, int kv0, const Src& fsrc, int fbuf) {
      constexpr bool MASK = decltype(mask_c)::value;
      const uint16_t* Kt = sKV[cur];
      const uint16_t* Kp = sKV[prev];
      const uint16_t* Kn = sKV[nxt];
      const int krow = kv0 + 4 * j4;  // key of element 0 in sub-block 0
      const int qcol = qw + l16;      // query of this lane's column in query tile 0
      u32x2 bv[QT];  // bias of the current sub-block per query tile (keys in elements)
      u32x4 qwd;     // keep words of this lane's query in the blocks drawn last
      static_assert(!DROP || QT == 4 || (QT == 2 && NSB % 2 == 0), "dropout block draw");

      // dS of sub-block sb (kept in sc[cp], dp), item e of 5 QT: per query tile four
      // products, then the packed tile into its half of the pair's A operand
      auto ds_item = [&](auto ec, auto cp_c, auto sb_c) {
        constexpr int e = decltype(ec)::value, cp = decltype(cp_c)::value, sb = decltype(sb_c)::value;
        constexpr int t = e / 5, i = e % 5;
        if constexpr (i == 4) {
          u32x2 v = pack_c4<DT>(dp[t]);
          pin<FT != FT_PLAIN>(v);
          da[sb / 2][t][2 * (sb % 2)] = v[0];
          da[sb / 2][t][2 * (sb % 2) + 1] = v[1];
          if constexpr (BIAS) {
            // the finished sub-block is sub-block sb of this tile, or the last one of
            // the previous tile (step 0); without dBias the resource is empty
            store_dbias(v, qcol + 16 * t, (sb == NSB - 1 ? kv0 - BN : kv0) + 16 * sb + 4 * j4);
          }
        } else if constexpr (DROP) {
          dp[t][i] = sc[cp][t][i] * fmaf(zf[cp][t][i], dp[t][i], nd[t][i]);  // P o (Z o dP - D)
        } else {
          dp[t][i] = sc[cp][t][i] * dp[t][i];  // dP - D: the dP^T product starts from -D
        }
      };
      auto p_item = [&](auto ec, auto st_c) {
        constexpr int e = decltype(ec)::value, st = decltype(st_c)::value, cs = st & 1;
        constexpr int t = e / 4, i = e % 4;
        if constexpr (DROP && i == 0) {
          // One Philox call per 4 x 4 block (queries q & ~3 .., keys of a 4-key group):
          // word q % 4 is query q, byte r key r.  The four lanes of a query quad share
          // their blocks, so lane j of the quad draws one of them (query tile j % QT of
          // sub-block st + j / QT; with two query tiles, the even step draws the odd
          // step's blocks too) and a quad transpose hands every lane its word of each:
          // word w of block w.
          constexpr bool DRAW = t == 0 && st % (4 / QT) == 0;
          if constexpr (DRAW) {
            const int q4 = l16 & 3, bt = q4 % QT, bst = st + q4 / QT;
            const u32x4 ctr = {(uint32_t)(krow + 16 * bst) >> 2, (uint32_t)(qcol + 16 * bt) >> 2,
                               (uint32_t)h, (uint32_t)b};
            qwd = quad_transpose(philox4x32_10(ctr, p.seed_lo, p.seed_hi), q4);
          }
          const uint32_t word = qwd[QT == 4 ? t : 2 * (st % 2) + t];
#pragma unroll
          for (int r = 0; r < 4; ++r) zf[cs][t][r] = keep_factor(word, r, p.keep_t, p.drop_scale);
        }
        float v;
        if constexpr (BIAS)
          v = fmaf(sc[cs][t][i], p.scale_log2, fmaf(elem4<DT>(bv[t], i), kLog2e, -lq[t]));
        else
          v = sc[cs][t][i] * p.scale_log2 - lq[t];
        if constexpr (MASK) {
          const int key = krow + 16 * st + i, q = qcol + 16 * t;
          if (key >= p.Nkv || (CAUSAL && key > q + p.off)) v = -INFINITY;
        }
        sc[cs][t][i] = fast_exp2(v);
      };

      using Steps = DqSteps<NK, QT>;
      auto begin = [&](auto stc) {
        constexpr int st = decltype(stc)::value;
        if constexpr (BIAS) {
          // bias of this sub-block: 4 keys of this lane's query per query tile
#pragma unroll
          for (int t = 0; t < QT; ++t)
            bv[t] = *reinterpret_cast<const u32x2*>(sB[cur] + (QW * w + 16 * t + l16) * BRS + 16 * st + 4 * j4);
        }
        if constexpr (st == 2) {
          // Mid-tile: every wave is past step 0 (its last reads of the previous
          // buffer) and, once its own copies have landed, the next tile is complete
          // (triple buffering), so the copies of steps 2-3 may refill the previous
          // buffer.
          wait_vmem();
          tile_barrier();
        }
        if constexpr (KB) {
          // the next sub-block's: of this tile, or (step 3, after the mid-tile
          // barrier, which completes the next tile when it is triple-buffered) the
          // next tile's first; past the last tile a buffer no product reads.  A
          // double-buffered next tile is complete only after the barrier in next().
          if constexpr (st < NSB - 1)
            cbk[(st + 1) % 2] = key_bias(cur, st + 1);
          else if constexpr (NBUF > 2)
            cbk[0] = key_bias(nxt, 0);
        }
      };
      auto operand = [&](auto stc, auto oc) -> u32x4 { return dq_operand(stc, oc, Kt, Kp); };
      // operand oc of the next tile, whose previous buffer is this one
      auto next = [&](auto oc) -> u32x4 {
        if constexpr (NBUF == 2 && decltype(oc)::value == 0) {
          // double buffering: the next tile was copied in this tile's second half
          wait_vmem();
          tile_barrier();
          if constexpr (KB) cbk[0] = key_bias(nxt, 0);  // now complete
        }
        return dq_operand(std::integral_constant<int, 0>(), oc, Kn, Kt);
      };
      auto mfma = [&](auto stc, auto mc, const u32x4& op) {
        constexpr int st = decltype(stc)::value, m = decltype(mc)::value, cs = st & 1;
        using Plan = typename Steps::template P<st>;
        constexpr int k = Plan::stage(m), loc = Plan::local(m);
        if constexpr (k == 0) {
          constexpr int s = loc / QT, t = loc % QT;
          if constexpr (s == 0 && KB)
            sc[cs][t] = Mx<DT>::first16c(op, qb[t][s], cbk[st % 2]);
          else if constexpr (s == 0)
            sc[cs][t] = Mx<DT>::first16(op, qb[t][s]);
          else
            Mx<DT>::acc16(sc[cs][t], op, qb[t][s]);
        } else if constexpr (k == 1) {
          constexpr int J = st < 2 ? 1 : 0, t = loc % QT, nn = (st % 2) * NK + loc / QT;
          Mx<DT>::acc16a(acc[t][nn], da[J][t], op);
        } else {
          // dP^T - D (dropout: dP^T alone, as the keep factors apply to dP before D)
          constexpr int s = loc / QT, t = loc % QT;
          if constexpr (s == 0 && DROP)
            dp[t] = Mx<DT>::first16(op, db[t][s]);
          else if constexpr (s == 0)
            dp[t] = Mx<DT>::first16c(op, db[t][s], nd[t]);
          else
            Mx<DT>::acc16(dp[t], op, db[t][s]);
        }
      };
      auto valu = [&](auto stc, auto mc, auto gc) {
        constexpr int st = decltype(stc)::value, m = decltype(mc)::value, cp = (st + 1) & 1;
        constexpr DqPlace<NK, QT, st, LA, OPS, NBUF == 2> PL{};
        static_assert(!DROP || none_before(PL.exp, PL.exp[0][0]), "query tile 0 draws the dropout blocks");
        (void)gc;
        // the copies of a later tile, in steps 2-3 (after the mid-tile barrier)
        static_for<OPS>([&](auto cc) {
          if constexpr (PL.copy[decltype(cc)::value] == m) copy_part(cc, fsrc, fbuf);
        });
        // dS of the previous sub-block (of the previous tile in step 0) under S^T_st
        static_for<5 * QT>([&](auto ec) {
          constexpr int e = decltype(ec)::value, t = e / 5, i = e % 5;
          if constexpr ((i < 4 ? PL.mul[t][i % 4] : PL.pack[t]) == m)
            ds_item(ec, std::integral_constant<int, cp>(), std::integral_constant<int, (st + NSB - 1) % NSB>());
        });
        static_for<4 * QT>([&](auto ec) {
          constexpr int e = decltype(ec)::value;
          if constexpr (PL.exp[e / 4][e % 4] == m) p_item(ec, stc);
        });
      };
      run_tile_carry<Steps::template P, NSB, LA>(carry, begin, operand, next, mfma, valu);
    };
    // dS of the last computed tile's last sub-block and the dQ product of its
    // second pair (a no-op when no tile was computed; skipped when no tile was
    // even copied, as the buffers then hold no data).
    auto flush = [&]() {
      const uint16_t* Kp = sKV[prev];
      static_for<5 * QT>([&](auto ec) {
        constexpr int e = decltype(ec)::value, t = e / 5, i = e % 5;
        if constexpr (i == 4) {
          const u32x2 v = pack_c4<DT>(dp[t]);
          da[1][t][2] = v[0];
          da[1][t][3] = v[1];
          if constexpr (BIAS) store_dbias(v, qw + l16 + 16 * t, kv_last + 16 * (NSB - 1) + 4 * j4);
        } else if constexpr (DROP) {
          dp[t][i] = sc[1][t][i] * fmaf(zf[1][t][i], dp[t][i], nd[t][i]);
        } else {
          dp[t][i] = sc[1][t][i] * dp[t][i];
        }
      });
      using Steps = DqSteps<NK, QT>;
      run_tile<Steps::template Flush, 1, LA>(
          [&](auto) {},
          [&](auto, auto oc) -> u32x4 {
            constexpr int n = decltype(oc)::value;
            const int k0 = 32 + 4 * j4;
            return pad_tr_operand<D>(Kp, k0, k0 + 16, 16 * n);
          },
          [&](auto, auto mc, const u32x4& op) {
            constexpr int loc = decltype(mc)::value, t = loc % QT, n = loc / QT;
            Mx<DT>::acc16a(acc[t][n], da[1][t], op);
          },
          [&](auto, auto, auto) {});
    };

    // This wave's split of the key tiles (one variant of the math per loop):
    //   [0, n_un)      every pair visible          unmasked
    //   [n_un, n_vis)  causal boundary / ragged    masked
    //   [n_vis, nkt)   no key visible to the wave  skipped
    int n_vis = nkt;
    if (qw >= p.Nq) n_vis = 0;
    else if (CAUSAL) n_vis = min(nkt, max(0, floor_div(qw + QW - 1 + p.off, BN) + 1));
    int n_un = min(n_vis, p.Nkv / BN);
    if (CAUSAL) n_un = min(n_un, max(0, floor_div(qw + p.off - (BN - 1), BN) + 1));

    if (nkt > 0) {
      static_for<NBUF - 1>([&](auto bc) { copy_all(decltype(bc)::value, decltype(bc)::value); });
    }
    // The register preloads and the first tiles' copies are in flight together.  The
    // copies are not visible to the compiler's wait counting, so everything is waited
    // for here: the compiler then knows the preloads have landed and puts no wait of
    // its own (which would count the copies wrongly) into the loop.
    wait_vmem();
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      float dsum = 0.f;
#pragma unroll
      for (int s = 0; s < NK; ++s) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dsum = Dt<DT>::dot2(ob[t][s][j], db[t][s][j], dsum);
      }
      dsum += __shfl_xor(dsum, 16);
      dsum += __shfl_xor(dsum, 32);
      nd[t][0] = -dsum;
      nd[t][1] = -dsum;
      nd[t][2] = -dsum;
      nd[t][3] = -dsum;
    }
    lds_barrier();
    // the first tile's leading operands (its "previous" buffer is the same one; the
    // previous-pair product it feeds is multiplied by zeros)
    static_for<LA>([&](auto oc) {
      carry[decltype(oc)::value] = dq_operand(std::integral_constant<int, 0>(), oc, sKV[0], sKV[0]);
    });
    if constexpr (KB) cbk[0] = key_bias(0, 0);
    // Iteration kt works on buffer kt % NBUF; from its middle on it copies tile
    // kt + NBUF - 1 into the buffer of iteration kt - 1.
    int kt = 0, cur = 0;
    auto phase = [&](int end, auto variant) {
      constexpr int VAR = decltype(variant)::value;  // 0 skip, 1 masked, 2 unmasked
      for (; kt < end; ++kt) {
        const int fbuf = cur == 0 ? NBUF - 1 : cur - 1;
        const int nxt = cur == NBUF - 1 ? 0 : cur + 1;
        const Src fsrc = src_of(kt + NBUF - 1);
        if constexpr (VAR == 0) {
          wait_vmem();
          tile_barrier();
          copy_all(kt + NBUF - 1, fbuf);
          if constexpr (NBUF == 2) {  // the second barrier a computed tile has
            wait_vmem();
            tile_barrier();
          }
        }
        if constexpr (VAR == 1) compute(cur, nxt, std::true_type(), kt * BN, fsrc, fbuf);
        if constexpr (VAR == 2) compute(cur, nxt, std::false_type(), kt * BN, fsrc, fbuf);
        if constexpr (VAR != 0) kv_last = kt * BN;
        prev = cur;
        cur = nxt;
      }
    };
    phase(n_un, std::integral_constant<int, 2>());
    phase(n_vis, std::integral_constant<int, 1>());
    if (nkt > 0) flush();
    phase(nkt, std::integral_constant<int, 0>());
    wait_vmem();    // no copy may land in LDS after the tile buffers are reused below
    lds_barrier();  // every wave is done with the tile buffers
    // the next item, claimed after the last wait for memory (see the dK/dV kernel)
    if (tid == 0) ticket = wq.next_ticket(ticket);
    settle(acc);
    uint16_t* stage = &sKV[0][0] + w * QW * (D + 8);
    store_block_c16<DT, D, QT>(acc, p.scale, stage, p.dq + qbase * D, qw, p.Nq, lane);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int q = qw + 16 * t + l16;
      if (q < p.Nq && j4 == 0) {
        p.ndelta[qbase + q] = nd[t][0];
        p.lse2[qbase + q] = lq[t];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers of one template instance (explicitly instantiated per instance in
// fa_bwd_inst.hip, so the instances compile in parallel).
template <int DT, int D, bool CAUSAL>
hipError_t run_pre(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  constexpr int RPB = 256 / pre_lanes_per_row<D>();
  const dim3 grid((unsigned)((p.rows + RPB - 1) / RPB));
  hipLaunchKernelGGL((bwd_pre_kernel<DT, D>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int DT, int D, bool CAUSAL, int FT>
hipError_t run_dkdv(const BwdArgs& a, hipStream_t s) {
  BwdParams p = make_params(a);
  constexpr int BN = 4 * 16 * TileShape<D, FT, true>::RT;  // keys per work item
  const int items = ((a.pb.Nkv + BN - 1) / BN) * a.pb.Hkv * a.pb.B;
  const int ncu = device_cu_count();
  const dim3 grid((unsigned)(p.sched && ncu > 0 && ncu < items ? ncu : items));
  hipLaunchKernelGGL((bwd_dkdv_kernel<DT, D, CAUSAL, FT>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int DT, int D, bool CAUSAL, int FT>
hipError_t run_dq(const BwdArgs& a, hipStream_t s) {
  BwdParams p = make_params(a);
  constexpr int BM = 4 * 16 * TileShape<D, FT>::RT;  // queries per work item
  const int items = ((a.pb.Nq + BM - 1) / BM) * a.pb.Hq * a.pb.B;
  const int ncu = device_cu_count();
  const dim3 grid((unsigned)(p.sched && ncu > 0 && ncu < items ? ncu : items));
  if constexpr (tile_bias(FT)) {
    if (p.dbias && p.Nkv % 4 == 0) {
      hipLaunchKernelGGL((bwd_dq_kernel<DT, D, CAUSAL, FT, true>), grid, dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_dq_kernel<DT, D, CAUSAL, FT>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
