// Kernel parameters and dispatch shared by the backward kernels.
#pragma once

#include "fa_common.hpp"
#include "fa_internal.hpp"

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
  float* ndelta;  // minus D per query row
  float* lse2;
  float* dq_acc;
  int* sched;  // work-queue counters (8 x 64 bits each for dK/dV and dQ) or null
  int B, Hq, Hkv, Nq, Nkv, G, off;  // off = Nkv - Nq (bottom-right causal offset)
  float scale, scale_log2, inv_scale;
  size_t rows;  // B * Hq * Nq
  // score bias (null: zero) with element strides, its gradient (null: not wanted),
  // and dropout (keep iff the element's random byte < keep_t; kept P scaled by
  // drop_scale = 256 / keep_t; Philox key = seed words)
  const uint16_t* bias;
  long long bias_sb, bias_sh, bias_sq;
  uint16_t* dbias;
  unsigned keep_t, seed_lo, seed_hi;
  float drop_scale;
};

inline BwdParams make_params(const BwdArgs& a) {
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
  p.ndelta = a.ndelta;
  p.lse2 = a.lse2;
  p.dq_acc = a.dq_acc;
  p.sched = a.sched;
  p.B = a.pb.B;
  p.Hq = a.pb.Hq;
  p.Hkv = a.pb.Hkv;
  p.Nq = a.pb.Nq;
  p.Nkv = a.pb.Nkv;
  p.G = a.pb.Hq / a.pb.Hkv;
  p.off = a.pb.Nkv - a.pb.Nq;
  p.scale = a.pb.scale;
  p.scale_log2 = a.pb.scale * kLog2e;
  p.inv_scale = 1.0f / a.pb.scale;
  p.rows = (size_t)a.pb.B * a.pb.Hq * a.pb.Nq;
  p.bias = static_cast<const uint16_t*>(a.x.bias);
  p.bias_sb = a.x.bias_sb;
  p.bias_sh = a.x.bias_sh;
  p.bias_sq = a.x.bias_sq;
  p.dbias = static_cast<uint16_t*>(a.x.dbias);
  p.keep_t = a.x.keep_t;
  p.seed_lo = (unsigned)(a.x.seed & 0xffffffffu);
  p.seed_hi = (unsigned)(a.x.seed >> 32);
  p.drop_scale = a.x.keep_t > 0 ? 256.f / (float)a.x.keep_t : 0.f;
  return p;
}

// Work distribution of the persistent dK/dV and dQ kernels over items (rank,
// head), item id rank * n_heads + head, ranks numbered heaviest first.  With
// counters, each XCD of the device (eight, each with its own L2) owns an equal
// share of the heads when they split evenly (XCD x: heads x*hpx .. +hpx-1), so the
// workgroups that read one head's data share an L2.  A share is a deque: the
// XCD's own workgroups take its items from the front, heaviest first; a workgroup
// whose share is used up takes items of another share from the back, lightest
// first, which evens out XCDs that run at different clocks without handing a
// helper a long item.  One 64-bit counter per share holds both ends (front count
// in the low half, back count in the high half), so one atomic add both claims an
// end and tells whether the item still exists.  Without counters (the problems
// that need no workspace) item t goes to workgroup t % gridDim.x.  A ticket is
// drawn (next_ticket) before the current item's output stores and turned into an
// item (resolve) after them, so the atomic's latency hides behind the stores.
struct WorkQueue {
  unsigned long long* ctr;  // 8 zeroed counters, or null
  int n_heads, n_items, nq, hpx, per_q, x;
  __device__ WorkQueue(int* c, int heads, int ranks) {
    ctr = reinterpret_cast<unsigned long long*>(c);
    n_heads = heads;
    n_items = heads * ranks;
    nq = (c != nullptr && (heads & 7) == 0) ? 8 : 1;
    hpx = heads / nq;
    per_q = hpx * ranks;
    x = nq == 8 ? (int)(__builtin_amdgcn_s_getreg(63508) & 7) : 0;  // HW_REG_XCC_ID
  }
  __device__ unsigned long long add(int q, unsigned long long v) const {
    return __hip_atomic_fetch_add(ctr + q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ int lo(unsigned long long v) { return (int)(unsigned)v; }
  static __device__ int hi(unsigned long long v) { return (int)(unsigned)(v >> 32); }
  __device__ int item_of(int q, int i) const { return (i / hpx) * n_heads + q * hpx + i % hpx; }
  __device__ long long first() const { return ctr ? (long long)add(x, 1) : (long long)blockIdx.x; }
  __device__ long long next_ticket(long long t) const {
    return ctr ? (long long)add(x, 1) : t + (long long)gridDim.x;
  }
  // item id of a ticket, or -1 when no work is left
  __device__ int resolve(long long t) const {
    if (!ctr) return t < n_items ? (int)t : -1;
    const unsigned long long u = (unsigned long long)t;
    if (lo(u) + hi(u) < per_q) return item_of(x, lo(u));
    if (nq == 1) return -1;  // one shared deque: nothing else to take from
    unsigned long long seen[8];
#pragma unroll
    for (int d = 1; d < 8; ++d)
      seen[d] = __hip_atomic_load(ctr + ((x + d) & 7), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int d = 1; d < 8; ++d) {
      if (lo(seen[d]) + hi(seen[d]) >= per_q) continue;
      const int q = (x + d) & 7;
      const unsigned long long v = add(q, 1ull << 32);
      if (lo(v) + hi(v) < per_q) return item_of(q, per_q - 1 - hi(v));
    }
    return -1;
  }
};

// Launchers of one template instance; each is explicitly instantiated in its own
// compilation of fa_bwd_inst.hip.
template <int DT, int D, bool CAUSAL> hipError_t run_pre(const BwdArgs& a, hipStream_t s);
template <int DT, int D, bool CAUSAL, int FT> hipError_t run_dkdv(const BwdArgs& a, hipStream_t s);
template <int DT, int D, bool CAUSAL, int FT> hipError_t run_dq(const BwdArgs& a, hipStream_t s);
template <int DT, int D, bool CAUSAL> hipError_t run_dkdv_atomic(const BwdArgs& a, hipStream_t s);

}  // namespace fa
