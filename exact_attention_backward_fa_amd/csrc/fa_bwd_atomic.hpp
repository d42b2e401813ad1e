// Fused dK/dV + atomic dQ kernel: the float-atomic alternative to the separate
// query-parallel dQ pass.  The Triton issue "Extra transposes cause 8x speedup for
// sequence-parallel Flash Attention backward" accumulates dq with tl.atomic_add into
// a float32 buffer from its key-block-parallel kernel; this is that decomposition on
// MFMA.  It is kept as a selectable path (FA_DQ_ATOMIC) and measured against the
// separate pass, which is faster on MI355X and deterministic.
#pragma once

#include "fa_bwd_common.hpp"

#include <type_traits>

namespace fa {

// ---------------------------------------------------------------------------
// Workgroup = 4 waves = 128 key rows of one (batch, kv head); wave w owns key rows
// 32w..32w+31 of the tile and keeps their K and V as MFMA operands in registers and
// their dK and dV as float32 accumulators.  The loop runs over the G query heads of
// the group and, per head, over 64-row query tiles from the first one that can see
// the key tile (causal) to the end.  Query tiles (Q, dO, LSE, D) are double-buffered
// in LDS and copied straight from global memory.  Tiles that touch the causal
// boundary or a ragged end take a masked variant of the math.
//
// S = Q K^T is computed with the key index in the lane (C column), so P^T and dS^T
// feed dV += P^T dO and dK += dS^T Q straight from the accumulators; dO and Q are
// then needed with the query index along the operand slots, which transposed LDS
// reads of the row-major tiles provide.
//
// dQ_i += scale * dS K_j goes into the float32 buffer with atomics: dS^T is staged
// in LDS (double-buffered) and the product for iteration i runs at the start of
// iteration i+1, after the barrier that publishes it.
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_atomic_kernel(BwdParams p) {
  constexpr int BN = 128, BM = 64, NG = D / 8;
  constexpr int TILE = BM * D;
  // Query tiles double-buffered (LDS also holds the K and dS^T tiles).
  constexpr int NBUF = 2;
  constexpr int OPS = 2 * (BM * NG / 256) + 2;  // copy instructions per fetch per wave
  __shared__ __attribute__((aligned(16))) uint16_t sQ[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) float sL[NBUF][BM];
  __shared__ __attribute__((aligned(16))) float sD[NBUF][BM];
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sdST[2][BN * BM];

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
  {
    for (int c = tid; c < BN * NG; c += 256) {
      const int r = c / NG, j = c % NG;
      const int kr = kv0 + r;
      *reinterpret_cast<u32x4*>(&sK[soff<NG, SW_LOWREG>(r, 8 * j)]) =
          kr < p.Nkv ? ld16(K + (size_t)kr * D + 8 * j) : zero_u4();
    }
  }

  // The tile copies below are not visible to the compiler's wait counting, so the
  // register and K-tile preloads are waited for here, before the first copy.
  wait_vmem();
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
    dma_tile<NG, BM, 256, SW_LOWREG>(p.q + qbase * D, q0, p.Nq, sQ[buf], w, lane);
    dma_tile<NG, BM, 256, SW_LOWREG>(p.dout + qbase * D, q0, p.Nq, sdO[buf], w, lane);
    // every wave copies LSE and D (identical bytes to the same place), so all
    // waves issue OPS copies per fetch and can share one vmcnt immediate
    const size_t r = qbase + min(q0 + lane, p.Nq - 1);
    dma4(p.lse2 + r, sL[buf]);
    dma4(p.ndelta + r, sD[buf]);
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
        const u32x4 a = lds_tr_operand<BM / 8, SW_LOWREG>(sdST[buf], k0, k0 + 4, 32 * tq + 16 * hi16);
        const u32x4 bk = lds_tr_operand<NG, SW_LOWREG>(sK, k0, k0 + 4, 32 * tn + 16 * hi16);
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
          return lds_row16<NG, SW_LOWREG>(sdO[cur], 32 * t + l32, 2 * s + g);
        else
          return lds_row16<NG, SW_LOWREG>(sQ[cur], 32 * t + l32, 2 * s + g);
      } else {
        constexpr int jj = j - 2 * NM, t = jj / NM, k = jj % NM;
        constexpr int c = k / (NM / 2), n = (k % (NM / 2)) / 2;
        const int k0 = 32 * t + 16 * c + 4 * g;
        if constexpr (k & 1)
          return lds_tr_operand<NG, SW_LOWREG>(sQ[cur], k0, k0 + 8, 32 * n + 16 * hi16);
        else
          return lds_tr_operand<NG, SW_LOWREG>(sdO[cur], k0, k0 + 8, 32 * n + 16 * hi16);
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
      dp[t][i] = pv * (dp[t][i] + D4[j4][e]);  // sD holds -D
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
    if (it > 0) dq_product(last, it - 1);
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
    {
      // dS^T[key][query]: 4 consecutive query rows per 8-byte store
#pragma unroll
      for (int t = 0; t < BM / 32; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 v2;
          v2[0] = Dt<DT>::pack2(dp[t][4 * j + 0], dp[t][4 * j + 1]);
          v2[1] = Dt<DT>::pack2(dp[t][4 * j + 2], dp[t][4 * j + 3]);
          *reinterpret_cast<u32x2*>(&sdST[cur][soff<BM / 8, SW_LOWREG>(32 * w + l32, 32 * t + 8 * j + 4 * g)]) = v2;
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
  if (n_it > 0) {
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

template <int DT, int D, bool CAUSAL>
hipError_t run_dkdv_atomic(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  const dim3 grid((unsigned)(((a.pb.Nkv + 127) / 128) * a.pb.Hkv * a.pb.B));
  hipLaunchKernelGGL((bwd_dkdv_atomic_kernel<DT, D, CAUSAL>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
