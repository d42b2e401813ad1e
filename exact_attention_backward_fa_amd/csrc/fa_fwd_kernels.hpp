// Forward kernel: O and LSE of exact softmax attention.
//
// The backward needs the per-row log-sum-exp of the scaled scores (rustytorch
// "flash_attention_backward.cu" and the Triton issue "Extra transposes cause 8x
// speedup for sequence-parallel Flash Attention backward" both rebuild P as
// exp(S - LSE) from it); no page prints a forward kernel, so this one is the
// usual streaming (online) softmax over key tiles, built from the same pieces as
// the backward's dQ pass.
//
// One workgroup = 4 waves = 256 query rows of one (batch, query head); wave w owns
// queries qw = q0 + 64w .. +63 and keeps Q as the B operand of S^T = K Q^T
// (16x16x32; query tile t of 16 queries) and O as float32 16x16 accumulators
// (query tile t, head-dim tile n).  Key/value tiles of 64 rows are triple-buffered
// in LDS and copied straight from global memory.  A tile is processed as two pairs
// of 16-key sub-blocks; step J of a tile issues
//   S^T of pair J | O += P V of the previous pair
// P of a pair is the two sub-blocks' packed 16x16 tiles side by side (a lane holds
// keys 4 j4 .. + 3 of each for its query), the A operand of a 16x16x32 product
// whose B operand (V with the same keys along the slots) is two transposed reads.
//
// Online softmax without rescaling: each query column keeps a reference m (log2
// domain, scale * log2 e folded in), set from the first pair in which the column
// sees a key, and P = exp2(s c - m).  P is rounded to the input type for the P V
// product, so the headroom H above m that a score may reach is set by that type's
// range: 64 for bf16 (float32's exponent range, P < 2^64) and 15 for fp16, whose
// largest finite value is 65504 < 2^16 (P < 2^15; with dropout, whose kept P is
// scaled by Z before rounding, the largest H with 2^H Z < 65520).  Relative
// precision does not depend on the size of P, so O and the row sums never need
// rescaling while no score exceeds m + H.  A score above m + H after the first
// pair (logits rising by more than 44 nats along the row for bf16, 10.4 nats for
// fp16) raises m and marks the item; the workgroup then runs the item a second
// time from zero with the raised references, which no score can exceed by more
// than H.
// The instances without bias (plain, and dropout alone) run in two launches.  The
// first (MODE 1) sets each column's reference from the first pair before its loop,
// takes no per-pair maxima, and checks at the end that no column's row sum exceeds
// 2^H: then no P did either and the result is the one the per-pair test would have
// given.  Otherwise it marks the item (LSE = NaN on its rows) and writes no O, and
// the second launch (MODE 2) runs the marked items with the per-pair test; its
// other workgroups exit at once.  The bias instances run every item with the
// per-pair test (MODE 0): a bias may hide a row's first keys, leaving its
// reference unset before the loop.
// The row sums l of P are float32 (each lane sums its keys; the four lanes of a
// column are added at the end; summing the bf16-rounded P through the matrix
// pipe was measured to miss the LSE bound on short rows).  At the end O is divided
// by l and LSE = ln 2 (m + log2 l).
#pragma once

#include "fa_internal.hpp"
#include "fa_pipeline.hpp"

#include <type_traits>

namespace fa {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nkv, G, off;  // off = Nkv - Nq (bottom-right causal offset)
  float scale_log2, inv_scale;
  // score bias (null: zero) with element strides; dropout of the P that weights V
  // (keep iff the element's random byte < keep_t, kept P scaled by drop_scale)
  const uint16_t* bias;
  long long bias_sb, bias_sh, bias_sq;
  unsigned keep_t, seed_lo, seed_hi;
  float drop_scale;
  float headroom;  // H of the dropout instances (fwd_headroom_dropout)
};

// log2 headroom above the reference of a query column: P = exp2(score - m) stays
// below 2^H, inside the range of the 16-bit type P is rounded to (fp16: 65504)
template <int DT>
constexpr float fwd_headroom() { return DT == 0 ? 15.f : 64.f; }

// With dropout, P o Z is rounded (Z = drop_scale, up to 256): for fp16 the headroom
// drops by whole units until 2^H Z is below 65520, the least value that rounds to
// inf.  bf16 keeps its 64.
template <int DT>
inline float fwd_headroom_dropout(float z) {
  float h = fwd_headroom<DT>(), top = 32768.f;
  if (DT == 0) {
    while (h > 0.f && top * z >= 65520.f) {
      h -= 1.f;
      top *= 0.5f;
    }
  }
  return h;
}

// Step J: S^T of pair J (2 NK operands x QT query tiles) | P V of the previous pair
// (2 NK head-dim tiles x QT).
template <int NK, int QT>
struct FwdSteps {
  template <int ST>
  using P = StepPlan<2 * NK, QT, 2 * NK, QT, 0, 1, 0, 1, 1>;
  template <int ST>
  using Flush = StepPlan<0, QT, 2 * NK, QT, 0, 1, 0, 1, 1>;
};

// Resident query rows per wave and LDS buffers per head dim: 64 queries (four
// 16-row tiles) and triple-buffered key/value tiles up to d = 128; above d = 128 a
// wave keeps 32 queries (Q and the O accumulators of 64 would not fit its
// registers), with three tile buffers at d = 160 and 192 and two above, where
// three would not fit the LDS.  The bias-tile instances (with or without dropout)
// take the small shape too (the bias tiles need the LDS, the bias and dropout work
// the registers); the key-bias and dropout-only instances keep the plain shape.
template <int D, int FT = 0>
struct FwdShape {
  static constexpr bool SMALL = D > 128 || tile_bias(FT);
  static constexpr int QT = SMALL ? 2 : 4;
  // three K/V buffers while they fit the LDS (at d = 192 not beside the key-bias
  // slots), else two
  static constexpr int NBUF =
      !SMALL || (!tile_bias(FT) && (D == 160 || (D == 192 && FT != FT_KEYBIAS))) ? 3 : 2;
};

// Slots of the non-MFMA work of forward step ST (NC copies in step 1): mx[t] (the
// pair's maxima), check (the test for a raised reference), exp[sb][t][i],
// pack[sb][t] and sum[sb][t] (the tile's P into the row sums).
// EARLY: the copies go under the S^T MFMAs of step 1 (double buffering waits for
// them before the last operand reads of the tile, which read the next tile).
template <int NK, int QT, int ST, int LA, int NC, bool EARLY>
struct FwdPlace {
  using Plan = typename FwdSteps<NK, QT>::template P<ST>;
  static constexpr int NM = Plan::NM;
  int mx[QT], check, exp[2][QT][4], pack[2][QT], sum[2][QT], copy[NC];
  constexpr FwdPlace() : mx(), check(), exp(), pack(), sum(), copy() {
    SlotLoad<NM> L;
    L.template reads<Plan, LA>();
    if (ST == 0) L.load[NM - 1] += 2;  // the mid-tile wait and barrier
    // the maxima within twelve slots after the S^T MFMAs (fewer in the short
    // steps of small head dims, leaving room for the exponentials)
    constexpr int HI = Plan::B1 + 11 < NM - 4 ? Plan::B1 + 11 : NM - 4;
    int prev = Plan::B1;
    L.level(QT * 4 + 3, Plan::B1, HI);
    for (int t = 0; t < QT; ++t) prev = mx[t] = L.put(4, prev, HI);
    prev = check = L.put(3, prev + 1, HI + 1);
    L.level(8 * QT * issue::kExp + 2 * QT * (issue::kPack + 4 * issue::kMul), prev + 1, NM - 2);
    prev = prev + 1;
    for (int g = 0; g <= 2 * QT; ++g) {  // g: (sub-block, query tile) g / QT, g % QT
      if (g < 2 * QT)
        for (int i = 0; i < 4; ++i) prev = exp[g / QT][g % QT][i] = L.put(issue::kExp, prev, NM - 2);
      if (g > 0) {
        prev = pack[(g - 1) / QT][(g - 1) % QT] = L.put(issue::kPack, prev, NM - 2);
        prev = sum[(g - 1) / QT][(g - 1) % QT] = L.put(4 * issue::kMul, prev, NM - 2);
      }
    }
    for (int c = 0; c < NC; ++c) copy[c] = -1;
    if (ST == 1) {
      const int hi = EARLY ? Plan::B1 - 1 : NM - 1;
      prev = 0;
      L.level(NC * issue::kCopy, 0, hi);
      for (int c = 0; c < NC; ++c) prev = copy[c] = L.put(issue::kCopy, prev, hi);
    }
  }
};

// Sub-block 1's dropout draw (at exp[1][0][0]) comes after every item of sub-block
// 0 that reads the first draw (exp[0][t][0]; the same slot runs sub-block 0 first).
template <int QT>
constexpr bool fwd_draw_after_uses(const int (&exp)[2][QT][4]) {
  for (int t = 0; t < QT; ++t)
    if (exp[0][t][0] > exp[1][0][0]) return false;
  return true;
}

template <int DT, int D, bool CAUSAL, int FT, int MODE = 0>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdParams p) {
  constexpr bool BIAS = tile_bias(FT), DROP = FT == FT_DROPOUT || FT == FT_DROP, KB = FT == FT_KEYBIAS;
  // per-pair maxima and the test for a raised reference (all but the fast pass)
  constexpr bool FULL = MODE != 1;
  constexpr int QT = FwdShape<D, FT>::QT;  // query tiles of 16 per wave
  constexpr int QW = 16 * QT, BM = 4 * QW, BN = 64, NST = 2;
  constexpr int NK = D / 32;
  constexpr int NBUF = FwdShape<D, FT>::NBUF;
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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;
  const int nqt = (p.Nq + BM - 1) / BM;
  const int n_heads = p.B * p.Hq;
  const int rank = blockIdx.x / n_heads, head = blockIdx.x % n_heads;
  // causal: the last query block sees the most keys, so it goes out first
  const int qt = CAUSAL ? nqt - 1 - rank : rank;
  const int b = head / p.Hq, h = head % p.Hq;
  const int hk = h / p.G;
  const int q0 = qt * BM;
  const int qw = q0 + QW * w;
  const size_t qbase = ((size_t)b * p.Hq + h) * (size_t)p.Nq;
  const size_t kbase = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;
  const uint16_t* __restrict__ K = p.k + kbase * D;
  const uint16_t* __restrict__ V = p.v + kbase * D;
  const float c = p.scale_log2;
  if constexpr (MODE == 2) {
    // only an item the fast pass marked (LSE of its first row NaN)
    const float mark = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(p.lse[qbase + q0])));
    if (!__builtin_isnan(mark)) return;
  }

  u32x4 qb[QT][NK];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int q = qw + 16 * t + l16;
#pragma unroll
    for (int s = 0; s < NK; ++s)
      qb[t][s] = q < p.Nq ? ld16(p.q + (qbase + q) * D + 32 * s + 8 * j4) : zero_u4();
  }
  f32x4 acc[QT][2 * NK];  // O per query tile and head-dim tile
#pragma unroll
  for (int t = 0; t < QT; ++t) {
#pragma unroll
    for (int n = 0; n < 2 * NK; ++n) acc[t][n] = zero4();
  }
  float lsum[QT] = {};  // this lane's part of its column's row sum
  // reference of this lane's query column per query tile, and the threshold above
  // which it is raised: (m + H) / c on raw scores, or m + H on the biased log2
  // logits of the bias instances; finite, so that a column with no visible key yet
  // gives exp2(-inf - m) = 0
  constexpr float kUnset = -1e30f;
  const float H = DROP ? p.headroom : fwd_headroom<DT>();
  float m[QT], thr[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m[t] = kUnset;
    thr[t] = BIAS ? m[t] + H : (m[t] + H) / c;
  }
  bool dirty = false;  // a reference was raised after it had been used
  __shared__ int s_dirty;

  int kv_end = p.Nkv;
  if (CAUSAL) {
    const int q_last = min(q0 + BM, p.Nq) - 1;
    kv_end = min(p.Nkv, q_last + p.off + 1);
  }
  const int nkt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;

  using Copy = PadPairDma<D, BN>;
  static_assert(Copy::PER_WAVE == KVPW, "key/value copies per wave");
  const uint16_t* __restrict__ tsrc = w < 2 ? K : V;
  struct Src {
    i32x4 t, bs;  // this wave's K or V tile; bias tile or key-bias row (bias instances)
  };
  // bias element offset of this workgroup's first query row (key 0)
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
  for (int cc = 0; cc < Copy::PER_WAVE; ++cc) voff[cc] = Copy::src_offset(cc, w, lane);
  const uint32_t wave_off = Copy::lds_wave_offset(w);
  int voffb[BIAS ? BPW : 1];
  if constexpr (BIAS) {
#pragma unroll
    for (int cc = 0; cc < BPW; ++cc) voffb[cc] = BiasDma::src_offset(cc, w, lane, (int)p.bias_sq);
  }
  auto copy_part = [&](auto cc, const Src& sr, int buf) {
    constexpr int ci = decltype(cc)::value;
    if constexpr (ci < KVPW) {
      bdma16<Copy::template lds_offset<ci>>(voff[ci], sr.t, lds_u32(sKV[buf]) + wave_off);
    } else if constexpr (KB) {
      bdma16<0>(16 * lane, sr.bs, lds_u32(sKB[buf]) + 1024 * w);
    } else {
      constexpr int cb_ = ci - KVPW;
      bdma16<BiasDma::template lds_offset<cb_>>(voffb[cb_], sr.bs,
                                                lds_u32(sB[buf]) + BiasDma::lds_wave_offset(w));
    }
  };
  // key-bias instances: bias / scale of keys 4 j4 .. + 3 of sub-block sb of pair J
  // of the tile in buffer buf: the accumulator the S^T product starts from, so the
  // scores come out biased (c (S + b / scale) = c S + b log2 e)
  auto key_bias = [&](int buf, int J, int sb) -> f32x4 {
    const u32x2 v = *reinterpret_cast<const u32x2*>(sKB[buf] + 512 * w + 16 * (2 * J + sb) + 4 * j4);
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = elem4<DT>(v, i) * p.inv_scale;
    return r;
  };
  f32x4 cbk[2][2];  // key bias accumulator starts of pair J, sub-block sb
  auto copy_all = [&](int kt, int buf) {
    const Src sr = src_of(kt);
    static_for<OPS>([&](auto cc) { copy_part(cc, sr, buf); });
  };

  // Carried from tile to tile: the first LA operands of the next tile and the packed
  // P of the second pair (pa[1]), whose product runs in step 0 of the next tile
  // with V read from the previous buffer (zero before the first tile).
  u32x4 carry[LA];
  u32x4 pa[2][QT];  // P A operands of pair J, per query tile
  f32x4 sc[2][QT];  // S^T of the current pair's sub-blocks, then P
#pragma unroll
  for (int t = 0; t < QT; ++t) pa[1][t] = zero_u4();
  int prev = 0;

  auto compute = [&](int cur, int nxt, auto mask_c, int kv0, const Src& fsrc, int fbuf) {
    constexpr bool MASK = decltype(mask_c)::value;
    const uint16_t* Kt = sKV[cur];
    const uint16_t* Vt = Kt + BN * RS;
    const uint16_t* Vp = sKV[prev] + BN * RS;
    const uint16_t* Kn = sKV[nxt];
    float mx[QT];
    u32x2 bv[2][QT];  // bias of the pair's sub-blocks per query tile (keys in elements)
    f32x4 zf[2][QT];  // dropout keep factors of the pair's sub-blocks
    u32x4 qwd;        // keep words of this lane's query in the blocks drawn last
    static_assert(QT == 4 || QT == 2, "dropout block draw");

    using Steps = FwdSteps<NK, QT>;
    auto begin = [&](auto stc) {
      constexpr int st = decltype(stc)::value;
      if constexpr (KB && st == 0) {
        // pair 1 of this tile (pair 0's products read cbk[0])
        cbk[1][0] = key_bias(cur, 1, 0);
        cbk[1][1] = key_bias(cur, 1, 1);
      }
      if constexpr (BIAS) {
        // bias of sub-blocks 2 st and 2 st + 1: 4 keys of this lane's query each
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
          for (int t = 0; t < QT; ++t)
            bv[sb][t] = *reinterpret_cast<const u32x2*>(sB[cur] + (QW * w + 16 * t + l16) * BRS +
                                                        16 * (2 * st + sb) + 4 * j4);
        }
      }
      if constexpr (st == 1) {
        // Mid-tile: every wave is past step 0 (its last read of the previous buffer)
        // and, once its own copies have landed, the next tile is complete, so the
        // copies of step 1 may refill the previous buffer.
        wait_vmem();
        tile_barrier();
        if constexpr (KB && NBUF > 2) {
          // pair 0 of the next tile, complete after the barrier when triple-buffered
          // (pair 1 of this one reads cbk[1]); past the last tile a buffer no product
          // reads.  A double-buffered next tile is complete only after the barrier
          // in next().
          cbk[0][0] = key_bias(nxt, 0, 0);
          cbk[0][1] = key_bias(nxt, 0, 1);
        }
      }
    };
    auto operand = [&](auto stc, auto oc) -> u32x4 {
      constexpr int st = decltype(stc)::value, o = decltype(oc)::value;
      using Plan = typename Steps::template P<st>;
      constexpr int k = Plan::op_stage(o), n = Plan::op_local(o);
      if constexpr (k == 0) {
        return pad_row16<D>(Kt, 16 * (2 * st + n / NK) + l16, 4 * (n % NK) + j4);
      } else {
        // pair 1 of the previous tile (step 0) or pair 0 of this one (step 1)
        constexpr int J = st == 0 ? 1 : 0;
        const int k0 = 32 * J + 4 * j4;
        return pad_tr_operand<D>(st == 0 ? Vp : Vt, k0, k0 + 16, 16 * n);
      }
    };
    auto next = [&](auto oc) -> u32x4 {  // operand oc of the next tile: S^T of pair 0
      constexpr int o = decltype(oc)::value;
      if constexpr (NBUF == 2 && o == 0) {
        // double buffering: the next tile was copied in this tile's second half
        wait_vmem();
        tile_barrier();
        if constexpr (KB) {  // pair 0 of the next tile, now complete
          cbk[0][0] = key_bias(nxt, 0, 0);
          cbk[0][1] = key_bias(nxt, 0, 1);
        }
      }
      return pad_row16<D>(Kn, 16 * (o / NK) + l16, 4 * (o % NK) + j4);
    };
    auto mfma = [&](auto stc, auto mc, const u32x4& op) {
      constexpr int st = decltype(stc)::value, mi = decltype(mc)::value;
      using Plan = typename Steps::template P<st>;
      constexpr int k = Plan::stage(mi), loc = Plan::local(mi), o = loc / QT, t = loc % QT;
      constexpr int J = st == 0 ? 1 : 0;
      if constexpr (k == 0) {
        constexpr int sb = o / NK, s = o % NK;
        if constexpr (s == 0 && KB)
          sc[sb][t] = Mx<DT>::first16c(op, qb[t][s], cbk[st][sb]);
        else if constexpr (s == 0)
          sc[sb][t] = Mx<DT>::first16(op, qb[t][s]);
        else
          Mx<DT>::acc16(sc[sb][t], op, qb[t][s]);
      } else {
        Mx<DT>::acc16a(acc[t][o], pa[J][t], op);
      }
    };
    auto valu = [&](auto stc, auto mc, auto gc) {
      constexpr int st = decltype(stc)::value, mi = decltype(mc)::value;
      using Plan = typename Steps::template P<st>;
      constexpr FwdPlace<NK, QT, st, LA, OPS, NBUF == 2> PL{};
      // dropout: the draws come first, and a second draw (four query tiles) after
      // every use of the first
      static_assert(!DROP || (none_before(PL.exp[0], PL.exp[0][0][0]) &&
                              none_before(PL.exp[1], QT == 4 ? PL.exp[1][0][0] : PL.exp[0][0][0])),
                    "the dropout draws precede their uses");
      static_assert(!DROP || QT == 2 || fwd_draw_after_uses(PL.exp), "second dropout draw after the first's uses");
      (void)gc;
      static_for<OPS>([&](auto cc) {
        if constexpr (PL.copy[decltype(cc)::value] == mi) copy_part(cc, fsrc, fbuf);
      });
      // the pair's maximum per query column (masked scores first)
      static_for<QT>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr (PL.mx[t] == mi) {
          if constexpr (BIAS) {
            // biased logits in log2 units: s c + bias log2 e
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                sc[sb][t][i] = fmaf(sc[sb][t][i], c, elem4<DT>(bv[sb][t], i) * kLog2e);
            }
          }
          if constexpr (MASK) {
            const int q = qw + 16 * t + l16;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int key = kv0 + 16 * (2 * st + sb) + 4 * j4 + i;
                if (key >= p.Nkv || (CAUSAL && key > q + p.off)) sc[sb][t][i] = -INFINITY;
              }
            }
          }
          const float m0 = FULL ? vmax3(sc[0][t][0], sc[0][t][1], sc[0][t][2]) : 0.f;
          const float m1 = FULL ? vmax3(sc[0][t][3], sc[1][t][0], sc[1][t][1]) : 0.f;
          if constexpr (FULL) mx[t] = vmax3(m0, m1, vmax3(sc[1][t][2], sc[1][t][3], sc[1][t][3]));
        }
      });
      if constexpr (FULL && PL.check == mi) {
        bool any = false;
#pragma unroll
        for (int t = 0; t < QT; ++t) any = any || mx[t] > thr[t];
        if (__builtin_amdgcn_ballot_w64(any) != 0) {  // rare: set or raise references
#pragma unroll
          for (int t = 0; t < QT; ++t) {
            float v = BIAS ? mx[t] : mx[t] * c;
            v = fmaxf(v, __shfl_xor(v, 16));
            v = fmaxf(v, __shfl_xor(v, 32));
            if (v > m[t] + H) {
              dirty = dirty || m[t] != kUnset;
              m[t] = v;
              thr[t] = BIAS ? v + H : (v + H) / c;
            }
          }
        }
      }
      static_for<2>([&](auto sbc) {
        constexpr int sb = decltype(sbc)::value;
        static_for<QT>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          static_for<4>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (PL.exp[sb][t][i] == mi) {
              if constexpr (DROP && i == 0) {
                // One Philox call per 4 x 4 block (queries q & ~3 .., keys of a 4-key
                // group): word q % 4 is query q, byte r key r.  The four lanes of a
                // query quad share their blocks, so lane j of the quad draws one of
                // them (query tile j % QT of sub-block sb + j / QT; with two query
                // tiles, sub-block 0 draws sub-block 1's blocks too) and a quad
                // transpose hands every lane its word of each: word w of block w.
                constexpr bool DRAW = t == 0 && sb % (4 / QT) == 0;
                if constexpr (DRAW) {
                  const int q4 = l16 & 3, bt = q4 % QT, bsb = sb + q4 / QT;
                  const u32x4 ctr = {(uint32_t)(kv0 + 16 * (2 * st + bsb) + 4 * j4) >> 2,
                                     (uint32_t)(qw + 16 * bt + l16) >> 2, (uint32_t)h, (uint32_t)b};
                  qwd = quad_transpose(philox4x32_10(ctr, p.seed_lo, p.seed_hi), q4);
                }
                const uint32_t word = qwd[QT == 4 ? t : 2 * sb + t];
#pragma unroll
                for (int r = 0; r < 4; ++r) zf[sb][t][r] = keep_factor(word, r, p.keep_t, p.drop_scale);
              }
              sc[sb][t][i] = BIAS ? fast_exp2(sc[sb][t][i] - m[t]) : fast_exp2(sc[sb][t][i] * c - m[t]);
            }
          });
          if constexpr (PL.pack[sb][t] == mi) {
            // V is weighted by the kept probabilities P o Z; the row sums take P
            u32x2 v = pack_c4<DT>(DROP ? sc[sb][t] * zf[sb][t] : sc[sb][t]);
            pin<FT != FT_PLAIN>(v);
            pa[st][t][2 * sb] = v[0];
            pa[st][t][2 * sb + 1] = v[1];
          }
          if constexpr (PL.sum[sb][t] == mi)
            lsum[t] += (sc[sb][t][0] + sc[sb][t][1]) + (sc[sb][t][2] + sc[sb][t][3]);
        });
      });
    };
    run_tile_carry<Steps::template P, NST, LA>(carry, begin, operand, next, mfma, valu);
  };
  // P V and row sums of the last computed tile's second pair (a no-op when no tile
  // was computed).
  auto flush = [&]() {
    const uint16_t* Vp = sKV[prev] + BN * RS;
    using Steps = FwdSteps<NK, QT>;
    using Plan = typename Steps::template Flush<0>;
    run_tile<Steps::template Flush, 1, LA>(
        [&](auto) {},
        [&](auto, auto oc) -> u32x4 {
          constexpr int n = Plan::op_local(decltype(oc)::value);
          const int k0 = 32 + 4 * j4;
          return pad_tr_operand<D>(Vp, k0, k0 + 16, 16 * n);
        },
        [&](auto, auto mc, const u32x4& op) {
          constexpr int loc = Plan::local(decltype(mc)::value), o = loc / QT, t = loc % QT;
          Mx<DT>::acc16a(acc[t][o], pa[1][t], op);
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

  if (tid == 0) s_dirty = 0;
  // One pass, or two when a reference had to be raised after use (see the top).
  for (int pass = 0;; ++pass) {
    if (nkt > 0) {
      static_for<NBUF - 1>([&](auto bc) { copy_all(decltype(bc)::value, decltype(bc)::value); });
    }
    // The register preloads and the first tiles' copies are in flight together; the
    // copies are invisible to the compiler's wait counting, so all are waited for.
    wait_vmem();
    lds_barrier();
    static_for<LA>([&](auto oc) {
      constexpr int o = decltype(oc)::value;
      carry[o] = pad_row16<D>(sKV[0], 16 * (o / NK) + l16, 4 * (o % NK) + j4);
    });
    if constexpr (KB) {
      cbk[0][0] = key_bias(0, 0, 0);
      cbk[0][1] = key_bias(0, 0, 1);
    }
    if constexpr (MODE == 1) {
      // each column's reference from its first pair (keys 0 .. 31), as the per-pair
      // test would set it; unset for a column that sees none of them (an empty row)
      if (nkt > 0) {
#pragma unroll
        for (int t = 0; t < QT; ++t) {
          f32x4 s2[2];
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int s = 0; s < NK; ++s) {
              const u32x4 op = pad_row16<D>(sKV[0], 16 * sb + l16, 4 * s + j4);
              if (s == 0)
                s2[sb] = Mx<DT>::first16(op, qb[t][s]);
              else
                Mx<DT>::acc16(s2[sb], op, qb[t][s]);
            }
          }
          wait_mfma();
          asm volatile("" : "+v"(s2[0]), "+v"(s2[1]));
          const int q = qw + 16 * t + l16;
          float v = -INFINITY;
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = 16 * sb + 4 * j4 + i;
              const bool vis = key < p.Nkv && (!CAUSAL || key <= q + p.off);
              v = fmaxf(v, vis ? s2[sb][i] : -INFINITY);
            }
          }
          v = fmaxf(v, __shfl_xor(v, 16));
          v = fmaxf(v, __shfl_xor(v, 32));
          if (v > -INFINITY) m[t] = v * c;
        }
      }
    }
    int kt = 0, cur = 0;
    prev = 0;
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
        prev = cur;
        cur = nxt;
      }
    };
    phase(n_un, std::integral_constant<int, 2>());
    phase(n_vis, std::integral_constant<int, 1>());
    if (nkt > 0) flush();
    phase(nkt, std::integral_constant<int, 0>());
    if constexpr (MODE == 1) {
      // no P above 2^H if no column's row sum is (also true for inf and NaN sums)
      const float limit = exp2f(H);
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        float l = lsum[t];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (!(l <= limit)) dirty = true;
      }
    }
    wait_vmem();    // no copy may land in LDS after the tile buffers are reused below
    if (dirty) s_dirty = 1;
    lds_barrier();  // every wave is done with the tile buffers; s_dirty is final
    if (MODE == 1 || pass > 0 || __builtin_amdgcn_readfirstlane(s_dirty) == 0) break;
    // run again from zero with the raised references
    settle(acc);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      pa[1][t] = zero_u4();
      lsum[t] = 0.f;
#pragma unroll
      for (int n = 0; n < 2 * NK; ++n) acc[t][n] = zero4();
    }
    dirty = false;
    lds_barrier();  // the s_dirty reads are done before the next pass's copies
  }
  settle(acc);
  if constexpr (MODE == 1) {
    if (__builtin_amdgcn_readfirstlane(s_dirty) != 0) {
      // marked for the second launch: LSE NaN on this wave's rows, no O
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const int q = qw + 16 * t + l16;
        if (j4 == 0 && q < p.Nq) p.lse[qbase + q] = __builtin_nanf("");
      }
      return;
    }
  }

  // O = acc / l per row; LSE = ln 2 (m + log2 l), -inf for a row that sees no key
  float inv[QT][4];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    float l = lsum[t];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int q = qw + 16 * t + l16;
    if (j4 == 0 && q < p.Nq) p.lse[qbase + q] = l > 0.f ? (m[t] + log2f(l)) * kLn2 : -INFINITY;
    const float il = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[t][i] = __shfl(il, 4 * j4 + i);  // row 16t + 4 j4 + i
  }
  uint16_t* stage = &sKV[0][0] + w * QW * (D + 8);
  store_block_rows<DT, D, QT>(acc, inv, stage, p.o + qbase * D, qw, p.Nq, lane);
}

// Launcher of one instance (explicitly instantiated per instance in fa_fwd_inst.hip).
template <int DT, int D, bool CAUSAL, int FT>
hipError_t run_fwd(const FwdArgs& a, hipStream_t s) {
  const Problem& pb = a.pb;
  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.B = pb.B;
  p.Hq = pb.Hq;
  p.Hkv = pb.Hkv;
  p.Nq = pb.Nq;
  p.Nkv = pb.Nkv;
  p.G = pb.Hq / pb.Hkv;
  p.off = pb.Nkv - pb.Nq;
  p.scale_log2 = pb.scale * kLog2e;
  p.inv_scale = 1.0f / pb.scale;
  p.bias = static_cast<const uint16_t*>(a.x.bias);
  p.bias_sb = a.x.bias_sb;
  p.bias_sh = a.x.bias_sh;
  p.bias_sq = a.x.bias_sq;
  p.keep_t = a.x.keep_t;
  p.seed_lo = (unsigned)(a.x.seed & 0xffffffffu);
  p.seed_hi = (unsigned)(a.x.seed >> 32);
  p.drop_scale = a.x.keep_t > 0 ? 256.f / (float)a.x.keep_t : 0.f;
  p.headroom = fwd_headroom_dropout<DT>(p.drop_scale);
  constexpr int BM = 4 * 16 * FwdShape<D, FT>::QT;  // queries per workgroup
  const dim3 grid((unsigned)(((pb.Nq + BM - 1) / BM) * pb.Hq * pb.B));
  if constexpr (FT == FT_PLAIN || FT == FT_DROP) {
    // the fast pass, then the items it marked
    hipLaunchKernelGGL((fwd_kernel<DT, D, CAUSAL, FT, 1>), grid, dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fwd_kernel<DT, D, CAUSAL, FT, 2>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((fwd_kernel<DT, D, CAUSAL, FT>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace fa
