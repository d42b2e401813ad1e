// Backward kernels of exact softmax attention.
//
//   bwd_pre   D_i = sum_d dO_id O_id per query row (rustytorch
//             "flash_attention_backward.cu" computes this row dot product inside
//             its tiled kernel; the Triton issue "Extra transposes cause 8x speedup
//             for sequence-parallel Flash Attention backward" loads it precomputed),
//             LSE rescaled to the log2 domain, and, for the atomic dQ path, the
//             float32 dQ buffer cleared.
//   bwd_dkdv  key/value-block-parallel dK and dV (the Triton issue's _bwd_kernel
//             structure: one program per key block, K and V resident, a loop over
//             query blocks).  Optionally also dQ += dS K with float atomics.
//   bwd_dq    query-block-parallel dQ pass (the decomposition of the rustytorch
//             kernel's grid), recomputing S, P, dP and dS; writes dQ once.
//   dq_convert  float32 dQ buffer -> dtype.
//
// Per (query tile i, key tile j) the math is, with s the softmax scale:
//   S = s Q_i K_j^T,  P = exp(S - LSE_i),  dV_j += P^T dO_i,  dP = dO_i V_j^T,
//   dS = P o (dP - D_i),  dK_j += s dS^T Q_i,  dQ_i += s dS K_j.
// Exponentials run in the log2 domain: P = exp2(S * s * log2 e - LSE_i * log2 e).
#include "fa_common.hpp"
#include "fa_internal.hpp"

#include <type_traits>

namespace fa {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;
  float* lse2;
  float* dq_acc;
  int B, Hq, Hkv, Nq, Nkv, G, off;  // off = Nkv - Nq (bottom-right causal offset)
  float scale, scale_log2;
  size_t rows;  // B * Hq * Nq
};

static BwdParams make_params(const BwdArgs& a) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<const uint16_t*>(a.o);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.delta = a.delta;
  p.lse2 = a.lse2;
  p.dq_acc = a.dq_acc;
  p.B = a.pb.B;
  p.Hq = a.pb.Hq;
  p.Hkv = a.pb.Hkv;
  p.Nq = a.pb.Nq;
  p.Nkv = a.pb.Nkv;
  p.G = a.pb.Hq / a.pb.Hkv;
  p.off = a.pb.Nkv - a.pb.Nq;
  p.scale = a.pb.scale;
  p.scale_log2 = a.pb.scale * kLog2e;
  p.rows = (size_t)a.pb.B * a.pb.Hq * a.pb.Nq;
  return p;
}

// ---------------------------------------------------------------------------
// Row preprocess.  D/8 lanes share a row; each lane reads 16 bytes of O and dO.
template <int DT, int D, bool ZERO_DQ>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float s = 0.f;
  if (row < p.rows) {
    const u32x4 a = ld16(p.o + row * D + part * 8);
    const u32x4 c = ld16(p.dout + row * D + part * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s += Dt<DT>::lo(a[j]) * Dt<DT>::lo(c[j]) + Dt<DT>::hi(a[j]) * Dt<DT>::hi(c[j]);
    if (ZERO_DQ) {
      float* z = p.dq_acc + row * D + part * 8;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(z) = zero;
      *reinterpret_cast<f32x4*>(z + 4) = zero;
    }
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (row < p.rows && part == 0) {
    p.delta[row] = s;
    const float L = p.lse[row];
    p.lse2[row] = (L == -INFINITY) ? INFINITY : L * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel.  Workgroup = 4 waves = 128 key rows of one (batch, kv head); wave w
// owns key rows 32w..32w+31 of the tile and keeps their K and V as MFMA operands in
// registers and their dK and dV as float32 accumulators.  The loop runs over the
// G query heads of the group and, per head, over 64-row query tiles from the first
// one that can see the key tile (causal) to the end.  Query tiles (Q, dO, LSE, D)
// are double-buffered in LDS: the next one is copied straight from global memory
// into the other buffer while the current one is used, so each iteration needs one
// barrier.  Tiles that touch the causal boundary or a ragged end take a masked
// variant of the math; interior tiles skip the per-element mask.
//
// S = Q K^T is computed with the key index in the lane (C column), so P^T and dS^T
// feed dV += P^T dO and dK += dS^T Q straight from the accumulators; dO and Q are
// then needed with the query index along the operand slots, which transposed LDS
// reads of the row-major tiles provide.
//
// With ATOMIC_DQ the workgroup also adds dQ_i += scale * dS K_j into a float32
// buffer: dS^T is staged in LDS (double-buffered) and the product for iteration i
// runs at the start of iteration i+1, after the barrier that publishes it.
template <int DT, int D, bool CAUSAL, bool ATOMIC_DQ>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int BN = 128, BM = 64, NG = D / 8;
  constexpr int TILE = BM * D;
  // Query tiles in flight: fetched NBUF-1 iterations ahead (the atomic variant's
  // LDS holds the K and dS^T tiles as well, so it keeps two buffers).
  constexpr int NBUF = ATOMIC_DQ ? 2 : 3;
  constexpr int OPS = 2 * (BM * NG / 256) + 2;  // copy instructions per fetch per wave
  __shared__ __attribute__((aligned(16))) uint16_t sQ[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) float sL[NBUF][BM];
  __shared__ __attribute__((aligned(16))) float sD[NBUF][BM];
  __shared__ __attribute__((aligned(16))) uint16_t sK[ATOMIC_DQ ? BN * D : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sdST[ATOMIC_DQ ? 2 : 1][ATOMIC_DQ ? BN * BM : 8];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5, hi16 = (lane >> 4) & 1;
  int rank, head;
  map_block(blockIdx.x, p.B * p.Hkv, rank, head);
  const int b = head / p.Hkv, hk = head % p.Hkv;
  const int kv0 = rank * BN;  // rank 0 = first key tile = most query rows under the mask
  const int kvw = kv0 + 32 * w;
  const int kv_lane = kvw + l32;  // key row this lane carries as S column
  const size_t kbase = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;
  const uint16_t* __restrict__ K = p.k + kbase * D;
  const uint16_t* __restrict__ V = p.v + kbase * D;

  u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kf[s] = kv_lane < p.Nkv ? ld16(K + (size_t)kv_lane * D + 16 * s + 8 * g) : zero_u4();
    vf[s] = kv_lane < p.Nkv ? ld16(V + (size_t)kv_lane * D + 16 * s + 8 * g) : zero_u4();
  }
  if (ATOMIC_DQ) {
    for (int c = tid; c < BN * NG; c += 256) {
      const int r = c / NG, j = c % NG;
      const int kr = kv0 + r;
      *reinterpret_cast<u32x4*>(&sK[soff<NG>(r, 8 * j)]) =
          kr < p.Nkv ? ld16(K + (size_t)kr * D + 8 * j) : zero_u4();
    }
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    dk[n] = zero16();
    dv[n] = zero16();
  }

  const int q_begin = CAUSAL ? max(0, kv0 - p.off) : 0;
  const int nqt = (p.Nq + BM - 1) / BM;
  const int qt_begin = q_begin < p.Nq ? q_begin / BM : nqt;
  const int per_head = nqt - qt_begin;
  const int n_it = p.G * per_head;

  // iteration -> (query row base of the head, first query row of the tile)
  auto tile_of = [&](int it, size_t& qbase, int& q0) {
    const int hh = it / per_head;
    q0 = (qt_begin + it % per_head) * BM;
    qbase = ((size_t)b * p.Hq + (size_t)hk * p.G + hh) * (size_t)p.Nq;
  };

  // Query tile `it` straight into LDS buffer `buf`; rows past N_q repeat row
  // N_q-1 and are masked in the math.
  auto fetch = [&](int it, int buf) {
    size_t qbase;
    int q0;
    tile_of(it, qbase, q0);
    dma_tile<NG, BM>(p.q + qbase * D, q0, p.Nq, sQ[buf], w, lane);
    dma_tile<NG, BM>(p.dout + qbase * D, q0, p.Nq, sdO[buf], w, lane);
    // every wave copies LSE and D (identical bytes to the same place), so all
    // waves issue OPS copies per fetch and can share one vmcnt immediate
    const size_t r = qbase + min(q0 + lane, p.Nq - 1);
    dma4(p.lse2 + r, sL[buf]);
    dma4(p.delta + r, sD[buf]);
  };

  // dQ_i += scale * dS_i K_j for the query tile staged in sdST[buf]; wave w takes
  // output tiles w, w+4, ... of the BM x D block.
  auto dq_product = [&](int buf, int it) {
    size_t qbase;
    int q0;
    tile_of(it, qbase, q0);
    float* __restrict__ dQacc = p.dq_acc + qbase * D;
    constexpr int NT = (BM / 32) * (D / 32);
#pragma unroll 1
    for (int tt = w; tt < NT; tt += 4) {
      const int tq = tt / (D / 32), tn = tt % (D / 32);
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) {
        const int k0 = 16 * ks + 8 * g;
        const u32x4 a = lds_tr_operand<BM / 8>(sdST[buf], k0, k0 + 4, 32 * tq + 16 * hi16);
        const u32x4 bk = lds_tr_operand<NG>(sK, k0, k0 + 4, 32 * tn + 16 * hi16);
        acc = Dt<DT>::mma(a, bk, acc);
      }
      float* rowp = dQacc + (size_t)(q0 + 32 * tq + 4 * g) * D + 32 * tn + l32;
      if (q0 + BM <= p.Nq) {
#pragma unroll
        for (int i = 0; i < 16; ++i) atomicAdd(rowp + (8 * (i >> 2) + (i & 3)) * D, acc[i] * p.scale);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (q0 + 32 * tq + crow_of(i, g) < p.Nq)
            atomicAdd(rowp + (8 * (i >> 2) + (i & 3)) * D, acc[i] * p.scale);
      }
    }
  };

  // The math of one query tile on LDS buffer CUR.  MASK: some (query, key) pair of
  // this wave's block is outside the causal mask or past N_q / N_kv.
  //
  // The iteration is one stream of 4*NM MFMAs (NM = D/8), in four quarters:
  //   S_0, dP_0 | S_1, dP_1 | dV, dK from half 0 | dV, dK from half 1
  // (half t = query rows 32t..32t+31 of the tile).  Step j issues the LDS reads of
  // the operand of MFMA j+LA, then MFMA j, then a fixed share of the VALU work:
  // the softmax of half 0 rides on quarter 1, that of half 1 on quarter 2, and
  // each half's P / dS operands are packed just before they are consumed.  A fence
  // after every step keeps this order, so LDS latency hides behind LA MFMAs and the
  // VALU behind the matrix pipe.
  auto compute = [&](auto cur_c, auto mask_c, int q0, f32x16* dp) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr int NM = D / 8;  // MFMAs per quarter
    constexpr int NS = 4 * NM;
    constexpr int LA = 4;      // operand lookahead, in MFMAs
    f32x16 sp[2];
    u32x4 pa[2][2], sa[2][2];  // packed P^T / dS^T operands [half][k-step]
    f32x4 L4[4], D4[4];

    // operand of MFMA J
    auto operand = [&](auto jc) -> u32x4 {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < 2 * NM) {
        constexpr int t = j / NM, s = (j % NM) / 2;
        if constexpr (j & 1)
          return lds_row16<NG>(sdO[cur], 32 * t + l32, 2 * s + g);
        else
          return lds_row16<NG>(sQ[cur], 32 * t + l32, 2 * s + g);
      } else {
        constexpr int jj = j - 2 * NM, t = jj / NM, k = jj % NM;
        constexpr int c = k / (NM / 2), n = (k % (NM / 2)) / 2;
        const int k0 = 32 * t + 16 * c + 4 * g;
        if constexpr (k & 1)
          return lds_tr_operand<NG>(sQ[cur], k0, k0 + 8, 32 * n + 16 * hi16);
        else
          return lds_tr_operand<NG>(sdO[cur], k0, k0 + 8, 32 * n + 16 * hi16);
      }
    };
    auto mfma = [&](auto jc, const u32x4& op) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < 2 * NM) {
        constexpr int t = j / NM, s = (j % NM) / 2;
        if constexpr (j & 1)
          dp[t] = Dt<DT>::mma(op, vf[s], dp[t]);
        else
          sp[t] = Dt<DT>::mma(op, kf[s], sp[t]);
      } else {
        constexpr int jj = j - 2 * NM, t = jj / NM, k = jj % NM;
        constexpr int c = k / (NM / 2), n = (k % (NM / 2)) / 2;
        if constexpr (k & 1)
          dk[n] = Dt<DT>::mma(sa[t][c], op, dk[n]);
        else
          dv[n] = Dt<DT>::mma(pa[t][c], op, dv[n]);
      }
    };
    // P and dS for element I of half T, in place (sp <- P, dp <- dS)
    auto softmax_elem = [&](auto tc, auto ic) {
      constexpr int t = decltype(tc)::value, i = decltype(ic)::value;
      constexpr int j4 = i >> 2, e = i & 3;
      float x = sp[t][i] * p.scale_log2 - L4[j4][e];
      if constexpr (MASK) {
        const int q = q0 + 32 * t + 8 * j4 + 4 * g + e;
        const bool masked = kv_lane >= p.Nkv || q >= p.Nq || (CAUSAL && kv_lane > q + p.off);
        x = masked ? -INFINITY : x;
      }
      const float pv = fast_exp2(x);
      sp[t][i] = pv;
      dp[t][i] = pv * (dp[t][i] - D4[j4][e]);
    };
    auto load_lse = [&](int t) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        L4[j4] = *reinterpret_cast<const f32x4*>(&sL[cur][32 * t + 8 * j4 + 4 * g]);
        D4[j4] = *reinterpret_cast<const f32x4*>(&sD[cur][32 * t + 8 * j4 + 4 * g]);
      }
    };
    // VALU share of step J: half 0's softmax rides on quarter 1 (steps NM..2NM-1,
    // spread over its first NM-4 steps, then its packing), half 1's on quarter 2.
    auto valu = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      static_for<2>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int base = (t + 1) * NM;
        constexpr int r = j - base;
        if constexpr (j == base - 2) load_lse(t);
        if constexpr (r >= 0 && r < NM - 4) {
          constexpr int e0 = (16 * r) / (NM - 4), e1 = (16 * (r + 1)) / (NM - 4);
          static_for<e1 - e0>([&](auto ic) {
            softmax_elem(tc, std::integral_constant<int, e0 + decltype(ic)::value>());
          });
        }
        if constexpr (r == NM - 4) pa[t][0] = pack_c_slice<DT>(sp[t], 0);
        if constexpr (r == NM - 3) pa[t][1] = pack_c_slice<DT>(sp[t], 1);
        if constexpr (r == NM - 2) sa[t][0] = pack_c_slice<DT>(dp[t], 0);
        if constexpr (r == NM - 1) sa[t][1] = pack_c_slice<DT>(dp[t], 1);
      });
    };

#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sp[t] = zero16();
      dp[t] = zero16();
    }
    u32x4 ops[LA];
    static_for<LA>([&](auto jc) { ops[decltype(jc)::value] = operand(jc); });
    static_for<NS>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const u32x4 op = ops[j % LA];
      if constexpr (j + LA < NS) ops[j % LA] = operand(std::integral_constant<int, j + LA>());
      mfma(jc, op);
      valu(jc);
      sched_fence();
    });
  };

  // One iteration on LDS buffer CUR (a compile-time constant, so LDS addresses are
  // fixed offsets from per-lane bases).
  auto body = [&](int it, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int last = (cur + NBUF - 1) % NBUF;  // buffer of iteration it-1 and it+NBUF-1
    if (ATOMIC_DQ && it > 0) dq_product(last, it - 1);
    const bool ahead = it + NBUF - 1 < n_it;
    if (ahead) fetch(it + NBUF - 1, last);
    size_t qbase_unused;
    int q0;
    tile_of(it, qbase_unused, q0);
    f32x16 dp[BM / 32];
    const bool all_masked = kvw >= p.Nkv || (CAUSAL && kvw > q0 + BM - 1 + p.off);
    const bool need_mask = kvw + 31 >= p.Nkv || q0 + BM > p.Nq || (CAUSAL && kvw + 31 > q0 + p.off);
    if (all_masked) {
#pragma unroll
      for (int t = 0; t < BM / 32; ++t) dp[t] = zero16();
    } else if (need_mask) {
      compute(cur_c, std::true_type(), q0, dp);
    } else {
      compute(cur_c, std::false_type(), q0, dp);
    }
    if (ATOMIC_DQ) {
      // dS^T[key][query]: 4 consecutive query rows per 8-byte store
#pragma unroll
      for (int t = 0; t < BM / 32; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 v2;
          v2[0] = Dt<DT>::pack2(dp[t][4 * j + 0], dp[t][4 * j + 1]);
          v2[1] = Dt<DT>::pack2(dp[t][4 * j + 2], dp[t][4 * j + 3]);
          *reinterpret_cast<u32x2*>(&sdST[cur][soff<BM / 8>(32 * w + l32, 32 * t + 8 * j + 4 * g)]) = v2;
        }
      }
    }
    // tile it+1 must have landed; the fetch of tile it+NBUF-1 may stay in flight
    if (ahead)
      wait_vmem_n<OPS * (NBUF - 2)>();
    else
      wait_vmem();
    lds_barrier();
  };

  static_for<NBUF - 1>([&](auto bc) {
    constexpr int k = decltype(bc)::value;
    if (k < n_it) fetch(k, k);
  });
  if (n_it >= NBUF - 1)
    wait_vmem_n<OPS * (NBUF - 2)>();
  else
    wait_vmem();
  lds_barrier();

  for (int it = 0; it < n_it; it += NBUF) {
    static_for<NBUF>([&](auto bc) {
      if (it + decltype(bc)::value < n_it) body(it + decltype(bc)::value, bc);
    });
  }
  if (ATOMIC_DQ && n_it > 0) {
    static_for<NBUF>([&](auto bc) {
      if ((n_it - 1) % NBUF == decltype(bc)::value) dq_product(decltype(bc)::value, n_it - 1);
    });
  }

  uint16_t* __restrict__ dK = p.dk + kbase * D;
  uint16_t* __restrict__ dV = p.dv + kbase * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = kvw + crow_of(i, g);
      if (kr < p.Nkv) {
        dK[(size_t)kr * D + 32 * n + l32] = Dt<DT>::one(dk[n][i] * p.scale);
        dV[(size_t)kr * D + 32 * n + l32] = Dt<DT>::one(dv[n][i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel for the separate-dQ path: two waves per SIMD with split roles.
//
// Workgroup = 8 waves = 128 key rows of one (batch, kv head).  Wave w works on key
// rows 32*(w%4) .. +31 (its "key group", kg) with role w/4:
//   role 0: S = Q K^T, P = exp(S - LSE) (masked), hands P to its partner through
//           LDS, then dV += P^T dO;            keeps K and dV in registers;
//   role 1: dP = dO V^T, then (with the partner's P) dS = P o (dP - D),
//           dK += dS^T Q;                      keeps V and dK in registers.
// The two waves of a key group run on the same SIMD, so while one runs VALU
// (softmax, dS) the other's MFMAs keep the matrix pipe busy.  Each wave needs about
// half the registers of a single wave doing all five steps.  The loop over query
// tiles (all G heads of the group) has two barriers per tile: after P is published
// and at the end of the tile.  Query tiles are triple-buffered in LDS and filled by
// direct copies, two tiles ahead.
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_rs_kernel(BwdParams p) {
  constexpr int NT = 512;
  constexpr int BN = 128, BM = 64, NG = D / 8;
  constexpr int TILE = BM * D;
  constexpr int NBUF = 3;
  constexpr int OPS = 2 * (BM * NG / NT) + 2;  // copy instructions per fetch per wave
  constexpr int NM = D / 8;                    // MFMAs per product per tile and wave
  __shared__ __attribute__((aligned(16))) uint16_t sQ[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) float sL[NBUF][BM];
  __shared__ __attribute__((aligned(16))) float sD[NBUF][BM];
  __shared__ __attribute__((aligned(16))) u32x4 sP[4][2][2][64];  // [kg][half][k-step][lane]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = w & 3, role = w >> 2;
  const int l32 = lane & 31, g = lane >> 5, hi16 = (lane >> 4) & 1;
  int rank, head;
  map_block(blockIdx.x, p.B * p.Hkv, rank, head);
  const int b = head / p.Hkv, hk = head % p.Hkv;
  const int kv0 = rank * BN;
  const int kvw = kv0 + 32 * kg;
  const int kv_lane = kvw + l32;
  const size_t kbase = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;

  // role 0 holds K (B operand of S = Q K^T), role 1 holds V (of dP = dO V^T)
  const uint16_t* __restrict__ KV = (role == 0 ? p.k : p.v) + kbase * D;
  u32x4 bf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    bf[s] = kv_lane < p.Nkv ? ld16(KV + (size_t)kv_lane * D + 16 * s + 8 * g) : zero_u4();

  f32x16 acc[D / 32];  // role 0: dV, role 1: dK
#pragma unroll
  for (int n = 0; n < D / 32; ++n) acc[n] = zero16();

  const int q_begin = CAUSAL ? max(0, kv0 - p.off) : 0;
  const int nqt = (p.Nq + BM - 1) / BM;
  const int qt_begin = q_begin < p.Nq ? q_begin / BM : nqt;
  const int per_head = nqt - qt_begin;
  const int n_it = p.G * per_head;

  auto tile_of = [&](int it, size_t& qbase, int& q0) {
    const int hh = it / per_head;
    q0 = (qt_begin + it % per_head) * BM;
    qbase = ((size_t)b * p.Hq + (size_t)hk * p.G + hh) * (size_t)p.Nq;
  };
  auto fetch = [&](int it, int buf) {
    size_t qbase;
    int q0;
    tile_of(it, qbase, q0);
    dma_tile<NG, BM, NT>(p.q + qbase * D, q0, p.Nq, sQ[buf], w, lane);
    dma_tile<NG, BM, NT>(p.dout + qbase * D, q0, p.Nq, sdO[buf], w, lane);
    const size_t r = qbase + min(q0 + lane, p.Nq - 1);
    dma4(p.lse2 + r, sL[buf]);
    dma4(p.delta + r, sD[buf]);
  };

  // First product of the tile: role 0 S = Q K^T, role 1 dP = dO V^T (NM MFMAs,
  // operands 4 ahead).  Role 0 starts its softmax of half 0 once that half's scores
  // are done.
  auto scores = [&](auto cur_c, const uint16_t* X, f32x16* sc, auto valu) {
    constexpr int cur = decltype(cur_c)::value;
    (void)cur;
    constexpr int LA = 4;
    auto operand = [&](auto jc) -> u32x4 {
      constexpr int j = decltype(jc)::value, t = j / (NM / 2), s = j % (NM / 2);
      return lds_row16<NG>(X, 32 * t + l32, 2 * s + g);
    };
    sc[0] = zero16();
    sc[1] = zero16();
    u32x4 ops[LA];
    static_for<LA>([&](auto jc) { ops[decltype(jc)::value] = operand(jc); });
    static_for<NM>([&](auto jc) {
      constexpr int j = decltype(jc)::value, t = j / (NM / 2), s = j % (NM / 2);
      const u32x4 op = ops[j % LA];
      if constexpr (j + LA < NM) ops[j % LA] = operand(std::integral_constant<int, j + LA>());
      sc[t] = Dt<DT>::mma(op, bf[s], sc[t]);
      valu(jc);
      sched_fence();
    });
  };
  // Second product: acc[n] += A[t][c]^T-operand x (transposed read of X); NM MFMAs.
  auto grads = [&](const uint16_t* X, const u32x4 (*A)[2], auto valu) {
    constexpr int LA = 4;
    auto operand = [&](auto jc) -> u32x4 {
      constexpr int j = decltype(jc)::value, t = j / (NM / 2), k = j % (NM / 2);
      constexpr int c = k / (NM / 4), n = k % (NM / 4);
      const int k0 = 32 * t + 16 * c + 4 * g;
      return lds_tr_operand<NG>(X, k0, k0 + 8, 32 * n + 16 * hi16);
    };
    u32x4 ops[LA];
    static_for<LA>([&](auto jc) { ops[decltype(jc)::value] = operand(jc); });
    static_for<NM>([&](auto jc) {
      constexpr int j = decltype(jc)::value, t = j / (NM / 2), k = j % (NM / 2);
      constexpr int c = k / (NM / 4), n = k % (NM / 4);
      const u32x4 op = ops[j % LA];
      if constexpr (j + LA < NM) ops[j % LA] = operand(std::integral_constant<int, j + LA>());
      acc[n] = Dt<DT>::mma(A[t][c], op, acc[n]);
      valu(jc);
      sched_fence();
    });
  };

  // Role 0: S, P (masked), publish P.
  auto role0_first = [&](auto cur_c, auto mask_c, int q0, u32x4 (*pa)[2]) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    f32x16 sp[2];
    f32x4 L4[2][4];
    auto softmax_elem = [&](auto tc, auto ic) {
      constexpr int t = decltype(tc)::value, i = decltype(ic)::value, j4 = i >> 2, e = i & 3;
      float x = sp[t][i] * p.scale_log2 - L4[t][j4][e];
      if constexpr (MASK) {
        const int q = q0 + 32 * t + 8 * j4 + 4 * g + e;
        const bool masked = kv_lane >= p.Nkv || q >= p.Nq || (CAUSAL && kv_lane > q + p.off);
        x = masked ? -INFINITY : x;
      }
      sp[t][i] = fast_exp2(x);
    };
    auto load_l = [&](int t) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        L4[t][j4] = *reinterpret_cast<const f32x4*>(&sL[cur][32 * t + 8 * j4 + 4 * g]);
    };
    // half 0's softmax rides on the MFMAs of half 1
    constexpr int H = NM / 2;
    scores(cur_c, sQ[cur], sp, [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j == H - 2) load_l(0);
      if constexpr (j >= H + 1) {
        constexpr int r = j - (H + 1), steps = H - 1;
        constexpr int e0 = (16 * r) / steps, e1 = (16 * (r + 1)) / steps;
        static_for<e1 - e0>([&](auto ic) {
          softmax_elem(std::integral_constant<int, 0>(), std::integral_constant<int, e0 + decltype(ic)::value>());
        });
      }
    });
    load_l(1);
    static_for<16>([&](auto ic) { softmax_elem(std::integral_constant<int, 1>(), ic); });
    static_for<2>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      static_for<2>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        pa[t][c] = pack_c_slice<DT>(sp[t], c);
        sP[kg][t][c][lane] = pa[t][c];
      });
    });
  };

  // Role 1 after the barrier: dS = P o (dP - D) from the published P, then dK.
  auto role1_second = [&](auto cur_c, f32x16* dp) {
    constexpr int cur = decltype(cur_c)::value;
    u32x4 pk[2][2], sa[2][2];
    f32x4 D4[2][4];
    static_for<2>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      static_for<2>([&](auto cc) { pk[t][decltype(cc)::value] = sP[kg][t][decltype(cc)::value][lane]; });
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        D4[t][j4] = *reinterpret_cast<const f32x4*>(&sD[cur][32 * t + 8 * j4 + 4 * g]);
    });
    auto ds_elem = [&](auto tc, auto ic) {
      constexpr int t = decltype(tc)::value, i = decltype(ic)::value;
      constexpr int c = i >> 3, e = i & 7, j4 = i >> 2;
      const uint32_t wd = pk[t][c][e >> 1];
      const float pv = (e & 1) ? Dt<DT>::hi(wd) : Dt<DT>::lo(wd);
      dp[t][i] = pv * (dp[t][i] - D4[t][j4][i & 3]);
    };
    static_for<16>([&](auto ic) { ds_elem(std::integral_constant<int, 0>(), ic); });
    sa[0][0] = pack_c_slice<DT>(dp[0], 0);
    sa[0][1] = pack_c_slice<DT>(dp[0], 1);
    // half 1's dS rides on the MFMAs of half 0
    constexpr int H = NM / 2;
    grads(sQ[cur], sa, [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < H - 2) {
        constexpr int steps = H - 2;
        constexpr int e0 = (16 * j) / steps, e1 = (16 * (j + 1)) / steps;
        static_for<e1 - e0>([&](auto ic) {
          ds_elem(std::integral_constant<int, 1>(), std::integral_constant<int, e0 + decltype(ic)::value>());
        });
      }
      if constexpr (j == H - 2) sa[1][0] = pack_c_slice<DT>(dp[1], 0);
      if constexpr (j == H - 1) sa[1][1] = pack_c_slice<DT>(dp[1], 1);
    });
  };

  auto body = [&](int it, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int last = (cur + NBUF - 1) % NBUF;
    const bool ahead = it + NBUF - 1 < n_it;
    if (ahead) fetch(it + NBUF - 1, last);
    size_t qbase_unused;
    int q0;
    tile_of(it, qbase_unused, q0);
    const bool all_masked = kvw >= p.Nkv || (CAUSAL && kvw > q0 + BM - 1 + p.off);
    const bool need_mask = kvw + 31 >= p.Nkv || q0 + BM > p.Nq || (CAUSAL && kvw + 31 > q0 + p.off);
    u32x4 pa[2][2];
    f32x16 dp[2];
    if (!all_masked) {
      if (role == 0) {
        if (need_mask)
          role0_first(cur_c, std::true_type(), q0, pa);
        else
          role0_first(cur_c, std::false_type(), q0, pa);
      } else {
        scores(cur_c, sdO[cur], dp, [&](auto) {});
      }
    }
    lds_barrier();  // P published
    if (!all_masked) {
      if (role == 0)
        grads(sdO[cur], pa, [&](auto) {});
      else
        role1_second(cur_c, dp);
    }
    if (ahead)
      wait_vmem_n<OPS * (NBUF - 2)>();
    else
      wait_vmem();
    lds_barrier();
  };

  static_for<NBUF - 1>([&](auto bc) {
    constexpr int k = decltype(bc)::value;
    if (k < n_it) fetch(k, k);
  });
  if (n_it >= NBUF - 1)
    wait_vmem_n<OPS * (NBUF - 2)>();
  else
    wait_vmem();
  lds_barrier();
  for (int it = 0; it < n_it; it += NBUF) {
    static_for<NBUF>([&](auto bc) {
      if (it + decltype(bc)::value < n_it) body(it + decltype(bc)::value, bc);
    });
  }

  uint16_t* __restrict__ out = (role == 0 ? p.dv : p.dk) + kbase * D;
  const float oscale = role == 0 ? 1.f : p.scale;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = kvw + crow_of(i, g);
      if (kr < p.Nkv) out[(size_t)kr * D + 32 * n + l32] = Dt<DT>::one(acc[n][i] * oscale);
    }
  }
}

// ---------------------------------------------------------------------------
// Separate dQ pass.  Workgroup = 4 waves = 128 query rows of one (batch, query
// head); wave w owns 32 of them and keeps their Q and dO as MFMA operands in
// registers.  S^T = K Q^T puts the query index in the lane, so dS feeds
// dQ += dS K straight from the accumulators; K is read transposed from the
// row-major LDS tile.  Key/value tiles are double-buffered and copied straight from
// global memory, like the forward's.
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdParams p) {
  constexpr int BM = 128, BN = 64, NG = D / 8;
  constexpr int TILE = BN * D;
  constexpr int NBUF = 3;                   // key/value tiles fetched two ahead
  constexpr int OPS = 2 * (BN * NG / 256);  // copy instructions per fetch per wave
  __shared__ __attribute__((aligned(16))) uint16_t sK[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NBUF][TILE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5, hi16 = (lane >> 4) & 1;
  const int nqt = (p.Nq + BM - 1) / BM;
  int rank, head;
  map_block(blockIdx.x, p.B * p.Hq, rank, head);
  const int qt = CAUSAL ? nqt - 1 - rank : rank;
  const int b = head / p.Hq, h = head % p.Hq;
  const int hk = h / p.G;
  const int q0 = qt * BM;
  const int qw = q0 + 32 * w;  // first query row of this wave
  const int qrow = qw + l32;
  const size_t qbase = ((size_t)b * p.Hq + h) * (size_t)p.Nq;
  const size_t kbase = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;
  const uint16_t* __restrict__ K = p.k + kbase * D;
  const uint16_t* __restrict__ V = p.v + kbase * D;

  u32x4 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = qrow < p.Nq ? ld16(p.q + (qbase + qrow) * D + 16 * s + 8 * g) : zero_u4();
    df[s] = qrow < p.Nq ? ld16(p.dout + (qbase + qrow) * D + 16 * s + 8 * g) : zero_u4();
  }
  const float lse_q = qrow < p.Nq ? p.lse2[qbase + qrow] : INFINITY;
  const float dlt_q = qrow < p.Nq ? p.delta[qbase + qrow] : 0.f;

  f32x16 acc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) acc[n] = zero16();

  int kv_end = p.Nkv;
  if (CAUSAL) {
    const int q_last = min(q0 + BM, p.Nq) - 1;
    kv_end = min(p.Nkv, q_last + p.off + 1);
  }
  const int nkt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;

  auto fetch = [&](int kt, int buf) {
    dma_tile<NG, BN>(K, kt * BN, p.Nkv, sK[buf], w, lane);
    dma_tile<NG, BN>(V, kt * BN, p.Nkv, sV[buf], w, lane);
  };

  // One key tile on LDS buffer CUR; MASK: the tile crosses the causal boundary of
  // this wave's rows or the end of the keys.  The tile is one compile-time stream
  // of MFMAs in four parts:
  //   S^T_0, dP^T_0 | S^T_1, dP^T_1 | dQ from keys 0..31 | dQ from keys 32..63
  // (NS1 = D/8 MFMAs per score part, NQ = D/16 per dQ part).  Step j issues the
  // LDS reads of the operand LA MFMAs ahead, MFMA j, and a share of the VALU: half
  // 0's dS rides on part 1, half 1's on part 2; a fence after every step keeps the
  // order.
  auto compute = [&](auto cur_c, auto mask_c, int kv0) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr int NS1 = D / 8, NQ = D / 16;
    constexpr int NS = 2 * NS1 + 2 * NQ;
    constexpr int LA = 4;
    f32x16 st[2], dpt[2];
    u32x4 da[2][2];  // packed dS operands [half][k-step]

    auto operand = [&](auto jc) -> u32x4 {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < 2 * NS1) {
        constexpr int t = j / NS1, s = (j % NS1) / 2;
        if constexpr (j & 1)
          return lds_row16<NG>(sV[cur], 32 * t + l32, 2 * s + g);
        else
          return lds_row16<NG>(sK[cur], 32 * t + l32, 2 * s + g);
      } else {
        constexpr int jj = j - 2 * NS1, t = jj / NQ, k = jj % NQ;
        constexpr int c = k / (NQ / 2), n = k % (NQ / 2);
        const int k0 = 32 * t + 16 * c + 4 * g;
        return lds_tr_operand<NG>(sK[cur], k0, k0 + 8, 32 * n + 16 * hi16);
      }
    };
    auto mfma = [&](auto jc, const u32x4& op) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < 2 * NS1) {
        constexpr int t = j / NS1, s = (j % NS1) / 2;
        if constexpr (j & 1)
          dpt[t] = Dt<DT>::mma(op, df[s], dpt[t]);
        else
          st[t] = Dt<DT>::mma(op, qf[s], st[t]);
      } else {
        constexpr int jj = j - 2 * NS1, t = jj / NQ, k = jj % NQ;
        constexpr int c = k / (NQ / 2), n = k % (NQ / 2);
        acc[n] = Dt<DT>::mma(da[t][c], op, acc[n]);
      }
    };
    // dS for element I of half T, in place in dpt
    auto ds_elem = [&](auto tc, auto ic) {
      constexpr int t = decltype(tc)::value, i = decltype(ic)::value;
      float x = st[t][i] * p.scale_log2 - lse_q;
      if constexpr (MASK) {
        const int kv = kv0 + 32 * t + crow_of(i, g);
        if (kv >= p.Nkv || (CAUSAL && kv > qrow + p.off)) x = -INFINITY;
      }
      const float pv = fast_exp2(x);
      dpt[t][i] = pv * (dpt[t][i] - dlt_q);
    };
    // VALU share of step J: half t's dS is spread over the first steps of the part
    // after its scores, then packed in the last two steps of that part.
    auto valu = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      static_for<2>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int base = t == 0 ? NS1 : 2 * NS1;
        constexpr int len = t == 0 ? NS1 : NQ;
        constexpr int r = j - base;
        if constexpr (r >= 0 && r < len - 2) {
          constexpr int e0 = (16 * r) / (len - 2), e1 = (16 * (r + 1)) / (len - 2);
          static_for<e1 - e0>([&](auto ic) {
            ds_elem(tc, std::integral_constant<int, e0 + decltype(ic)::value>());
          });
        }
        if constexpr (r == len - 2) da[t][0] = pack_c_slice<DT>(dpt[t], 0);
        if constexpr (r == len - 1) da[t][1] = pack_c_slice<DT>(dpt[t], 1);
      });
    };

#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = zero16();
      dpt[t] = zero16();
    }
    u32x4 ops[LA];
    static_for<LA>([&](auto jc) { ops[decltype(jc)::value] = operand(jc); });
    static_for<NS>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const u32x4 op = ops[j % LA];
      if constexpr (j + LA < NS) ops[j % LA] = operand(std::integral_constant<int, j + LA>());
      mfma(jc, op);
      valu(jc);
      sched_fence();
    });
  };

  auto body = [&](int kt, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int last = (cur + NBUF - 1) % NBUF;
    const bool ahead = kt + NBUF - 1 < nkt;
    if (ahead) fetch(kt + NBUF - 1, last);
    const int kv0 = kt * BN;
    const bool need_mask = kv0 + BN > p.Nkv || (CAUSAL && kv0 + BN - 1 > qw + p.off);
    const bool all_masked = CAUSAL && kv0 > qw + 31 + p.off;
    if (!all_masked) {
      if (need_mask)
        compute(cur_c, std::true_type(), kv0);
      else
        compute(cur_c, std::false_type(), kv0);
    }
    if (ahead)
      wait_vmem_n<OPS * (NBUF - 2)>();
    else
      wait_vmem();
    lds_barrier();
  };

  static_for<NBUF - 1>([&](auto bc) {
    constexpr int k = decltype(bc)::value;
    if (k < nkt) fetch(k, k);
  });
  if (nkt >= NBUF - 1)
    wait_vmem_n<OPS * (NBUF - 2)>();
  else
    wait_vmem();
  lds_barrier();
  for (int kt = 0; kt < nkt; kt += NBUF) {
    static_for<NBUF>([&](auto bc) {
      if (kt + decltype(bc)::value < nkt) body(kt + decltype(bc)::value, bc);
    });
  }

  uint16_t* __restrict__ dQ = p.dq + qbase * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qr = qw + crow_of(i, g);
      if (qr < p.Nq) dQ[(size_t)qr * D + 32 * n + l32] = Dt<DT>::one(acc[n][i] * p.scale);
    }
  }
}

// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ src,
                                                         uint16_t* __restrict__ dst, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(src + 8 * i);
  const f32x4 c = *reinterpret_cast<const f32x4*>(src + 8 * i + 4);
  u32x4 r;
  r[0] = Dt<DT>::pack2(a[0], a[1]);
  r[1] = Dt<DT>::pack2(a[2], a[3]);
  r[2] = Dt<DT>::pack2(c[0], c[1]);
  r[3] = Dt<DT>::pack2(c[2], c[3]);
  st16(dst + 8 * i, r);
}

// ---------------------------------------------------------------------------
// Launchers.
static inline int dispatch_key(const Problem& pb) {
  return pb.dtype * 4 + (pb.d == 128 ? 2 : 0) + (pb.causal ? 1 : 0);
}

#define FA_DISPATCH(KEY, FN, ...)                        \
  switch (KEY) {                                         \
    case 0: return FN<0, 64, false>(__VA_ARGS__);        \
    case 1: return FN<0, 64, true>(__VA_ARGS__);         \
    case 2: return FN<0, 128, false>(__VA_ARGS__);       \
    case 3: return FN<0, 128, true>(__VA_ARGS__);        \
    case 4: return FN<1, 64, false>(__VA_ARGS__);        \
    case 5: return FN<1, 64, true>(__VA_ARGS__);         \
    case 6: return FN<1, 128, false>(__VA_ARGS__);       \
    default: return FN<1, 128, true>(__VA_ARGS__);       \
  }

template <int DT, int D, bool CAUSAL>
static hipError_t pre_t(const BwdArgs& a, bool zero, hipStream_t s) {
  const BwdParams p = make_params(a);
  constexpr int RPB = 256 / (D / 8);
  const dim3 grid((unsigned)((p.rows + RPB - 1) / RPB));
  if (zero)
    hipLaunchKernelGGL((bwd_pre_kernel<DT, D, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<DT, D, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdArgs& a, bool zero_dq_acc, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Hq * a.pb.Nq == 0) return hipSuccess;
  FA_DISPATCH(dispatch_key(a.pb), pre_t, a, zero_dq_acc, s)
}

template <int DT, int D, bool CAUSAL>
static hipError_t dkdv_t(const BwdArgs& a, bool atomic, hipStream_t s) {
  const BwdParams p = make_params(a);
  const dim3 grid((unsigned)(((a.pb.Nkv + 127) / 128) * a.pb.Hkv * a.pb.B));
  if (atomic)
    hipLaunchKernelGGL((bwd_dkdv_kernel<DT, D, CAUSAL, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_rs_kernel<DT, D, CAUSAL>), grid, dim3(512), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, bool atomic_dq, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Nkv == 0) return hipSuccess;
  FA_DISPATCH(dispatch_key(a.pb), dkdv_t, a, atomic_dq, s)
}

template <int DT, int D, bool CAUSAL>
static hipError_t dq_t(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  const dim3 grid((unsigned)(((a.pb.Nq + 127) / 128) * a.pb.Hq * a.pb.B));
  hipLaunchKernelGGL((bwd_dq_kernel<DT, D, CAUSAL>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Nq == 0) return hipSuccess;
  FA_DISPATCH(dispatch_key(a.pb), dq_t, a, s)
}

hipError_t launch_bwd_dq_convert(const BwdArgs& a, hipStream_t s) {
  const size_t n = (size_t)a.pb.B * a.pb.Hq * a.pb.Nq * a.pb.d;
  if (n == 0) return hipSuccess;
  const size_t n8 = n / 8;  // d is a multiple of 8
  const dim3 grid((unsigned)((n8 + 255) / 256));
  if (a.pb.dtype == 0)
    hipLaunchKernelGGL((dq_convert_kernel<0>), grid, dim3(256), 0, s, a.dq_acc,
                       static_cast<uint16_t*>(a.dq), n8);
  else
    hipLaunchKernelGGL((dq_convert_kernel<1>), grid, dim3(256), 0, s, a.dq_acc,
                       static_cast<uint16_t*>(a.dq), n8);
  return hipGetLastError();
}

}  // namespace fa
