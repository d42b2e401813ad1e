// Forward kernel: O and LSE of exact softmax attention.
//
// The backward needs the per-row log-sum-exp of the scaled scores (rustytorch
// "flash_attention_backward.cu" and the Triton issue "Extra transposes cause 8x
// speedup for sequence-parallel Flash Attention backward" both rebuild P as
// exp(S - LSE) from it); no page prints a forward kernel, so this one is the
// usual streaming (online) softmax over key tiles.
//
// One workgroup = 4 waves = 128 query rows of one (batch, query head); each wave
// owns 32 rows.  Key and value tiles of 64 rows are double-buffered in LDS: the
// next tile is copied straight from global memory into the other buffer while the
// current one is used.  Per tile:
//   S^T = K Q^T       (MFMA; Q stays in registers as the B operand for the whole
//                      loop, K is read from LDS)
//   online max / sum  (each lane owns one query column of S^T, so the row
//                      reductions are in-lane plus one swap between lane halves)
//   O^T += V^T P^T    (MFMA; P^T comes straight from the S^T accumulators, V^T is
//                      read from the row-major V tile with transposed LDS reads)
// Scores are kept in the log2 domain (scale * log2 e folded in) so the exponent is
// one v_exp_f32.
#include "fa_common.hpp"
#include "fa_internal.hpp"

#include <type_traits>

namespace fa {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nkv, G, off;  // off = Nkv - Nq (bottom-right causal offset)
  float scale_log2;
};

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdParams p) {
  constexpr int BM = 128, BN = 64, NG = D / 8;
  constexpr int TILE = BN * D;              // elements of one K or V tile
  constexpr int NBUF = 3;                   // key/value tiles fetched two ahead
  constexpr int OPS = 2 * (BN * NG / 256);  // copy instructions per fetch per wave
  __shared__ __attribute__((aligned(16))) uint16_t sK[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NBUF][TILE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int nqt = (p.Nq + BM - 1) / BM;
  int rank, head;
  map_block(blockIdx.x, p.B * p.Hq, rank, head);
  // causal: the last query tile sees the most keys, so it goes out first
  const int qt = CAUSAL ? nqt - 1 - rank : rank;
  const int b = head / p.Hq, h = head % p.Hq;
  const int hk = h / p.G;
  const int q0 = qt * BM;
  const size_t qbase = ((size_t)b * p.Hq + h) * (size_t)p.Nq;
  const size_t kbase = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;
  const uint16_t* __restrict__ Q = p.q + qbase * D;
  const uint16_t* __restrict__ K = p.k + kbase * D;
  const uint16_t* __restrict__ V = p.v + kbase * D;
  const int qrow = q0 + 32 * w + l32;  // this lane's query row

  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = qrow < p.Nq ? ld16(Q + (size_t)qrow * D + 16 * s + 8 * g) : zero_u4();

  // The tile copies below are not visible to the compiler's wait counting, so the
  // register preload is waited for here, before the first copy is issued.
  wait_vmem();
  f32x16 acc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) acc[n] = zero16();
  float m = -INFINITY, l = 0.f;

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
  // this wave's rows or the end of the keys.
  auto compute = [&](auto cur_c, auto mask_c, int kv0) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    // S^T = K Q^T for this wave's 32 query columns
    f32x16 st[BN / 32];
#pragma unroll
    for (int t = 0; t < BN / 32; ++t) {
      st[t] = zero16();
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        st[t] = Dt<DT>::mma(lds_row16<NG>(sK[cur], 32 * t + l32, 2 * s + g), qf[s], st[t]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < BN / 32; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = st[t][i] * p.scale_log2;
        if (MASK) {
          const int kv = kv0 + 32 * t + crow_of(i, g);
          if (kv >= p.Nkv || (CAUSAL && kv > qrow + p.off)) x = -INFINITY;
        }
        st[t][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < BN / 32; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(st[t][i] - m_use);
        st[t][i] = e;
        rs += e;
      }
    }
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[n][i] *= alpha;

    // O^T += V^T P^T; V^T comes from the row-major V tile by transposed reads
#pragma unroll
    for (int t = 0; t < BN / 32; ++t) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4 pb = pack_c_slice<DT>(st[t], c);
        const int k0 = 32 * t + 16 * c + 4 * g;
#pragma unroll
        for (int n = 0; n < D / 32; ++n) {
          const u32x4 a = lds_tr_operand<NG>(sV[cur], k0, k0 + 8, 32 * n + 16 * ((lane >> 4) & 1));
          acc[n] = Dt<DT>::mma(a, pb, acc[n]);
        }
      }
    }
  };

  const int qw = q0 + 32 * w;  // first query row of this wave
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

  if (qrow < p.Nq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* O = p.o + (qbase + qrow) * D;
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w2;
        w2[0] = Dt<DT>::pack2(acc[n][4 * j + 0] * inv, acc[n][4 * j + 1] * inv);
        w2[1] = Dt<DT>::pack2(acc[n][4 * j + 2] * inv, acc[n][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(O + 32 * n + 8 * j + 4 * g) = w2;
      }
    }
    if (g == 0) p.lse[qbase + qrow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int DT, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
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
  const dim3 grid((unsigned)(((pb.Nq + 127) / 128) * pb.Hq * pb.B));
  hipLaunchKernelGGL((fwd_kernel<DT, D, CAUSAL>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Nq == 0) return hipSuccess;
  const int key = a.pb.dtype * 4 + (a.pb.d == 128 ? 2 : 0) + (a.pb.causal ? 1 : 0);
  switch (key) {
    case 0: return launch_fwd_t<0, 64, false>(a, s);
    case 1: return launch_fwd_t<0, 64, true>(a, s);
    case 2: return launch_fwd_t<0, 128, false>(a, s);
    case 3: return launch_fwd_t<0, 128, true>(a, s);
    case 4: return launch_fwd_t<1, 64, false>(a, s);
    case 5: return launch_fwd_t<1, 64, true>(a, s);
    case 6: return launch_fwd_t<1, 128, false>(a, s);
    default: return launch_fwd_t<1, 128, true>(a, s);
  }
}

}  // namespace fa
