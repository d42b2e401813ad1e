// Backward entry points: dispatch of a problem to its template instance (the
// kernels are in fa_bwd_kernels.hpp and fa_bwd_atomic.hpp, instantiated in
// fa_bwd_inst.hip) and the float32 -> dtype conversion of the atomic dQ buffer.
#include "fa_bwd_common.hpp"


namespace fa {

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


// Clears the dK/dV and dQ work-queue counters (the row preprocess does it on the
// atomic path).
__global__ __launch_bounds__(64) void sched_clear_kernel(int* __restrict__ sched) {
  if (threadIdx.x < 32) sched[threadIdx.x] = 0;
}

hipError_t launch_sched_clear(const BwdArgs& a, hipStream_t s) {
  if (a.sched == nullptr) return hipSuccess;
  hipLaunchKernelGGL(sched_clear_kernel, dim3(1), dim3(64), 0, s, a.sched);
  return hipGetLastError();
}

// dBias entries the dQ pass never visits: under the causal mask, (row i, key j)
// with j > i + N_kv - N_q is masked, P and dS are zero there, and whole key tiles
// of them are skipped.  Block (x, y) writes zeros to the masked keys among
// 8192 y .. 8192 y + 8191 of row x, in groups of 8 keys that are 16-byte aligned
// in memory: a whole group with one 16-byte store, a group cut by the range or
// the row's ends key by key.
constexpr int kFillKeys = 8192;
__global__ __launch_bounds__(256) void dbias_fill_masked_kernel(uint16_t* __restrict__ dbias, int Nq,
                                                                int Nkv, int off, size_t row0) {
  const size_t row = row0 + blockIdx.x;  // over B * Hq * N_q
  const int i = (int)(row % (size_t)Nq);
  const int lo = max(max(0, i + off + 1), (int)blockIdx.y * kFillKeys);  // first masked key
  const int hi = min(Nkv, (int)(blockIdx.y + 1) * kFillKeys);
  if (lo >= hi) return;
  uint16_t* dst = dbias + row * (size_t)Nkv;
  // e0: the first key whose address is 16-byte aligned (rows are 2-byte aligned)
  const int e0 = (int)(((16u - ((uint32_t)(uintptr_t)dst & 15u)) & 15u) >> 1);
  const int g0 = (lo - e0 >= 0) ? (lo - e0) / 8 : -((e0 - lo + 7) / 8);  // floor
  const int g1 = (hi - e0 + 7 >= 0) ? (hi - e0 + 7) / 8 : 0;              // ceil, exclusive
  for (int g = g0 + (int)threadIdx.x; g < g1; g += 256) {
    const int a = e0 + 8 * g;
    if (a >= lo && a + 8 <= hi) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(dst + a) = z;
    } else {
      for (int k = 0; k < 8; ++k)
        if (a + k >= lo && a + k < hi) dst[a + k] = 0;
    }
  }
}

hipError_t launch_dbias_fill(const BwdArgs& a, hipStream_t s) {
  const size_t rows = (size_t)a.pb.B * a.pb.Hq * a.pb.Nq;
  if (!a.pb.causal || a.x.dbias == nullptr || rows == 0 || a.pb.Nkv == 0) return hipSuccess;
  constexpr size_t kMaxRows = (size_t)1 << 30;  // per launch (grid x limit)
  for (size_t r0 = 0; r0 < rows; r0 += kMaxRows) {
    const size_t n = rows - r0 < kMaxRows ? rows - r0 : kMaxRows;
    const dim3 grid((unsigned)n, (unsigned)((a.pb.Nkv + kFillKeys - 1) / kFillKeys));
    hipLaunchKernelGGL(dbias_fill_masked_kernel, grid, dim3(256), 0, s,
                       static_cast<uint16_t*>(a.x.dbias), a.pb.Nq, a.pb.Nkv, a.pb.Nkv - a.pb.Nq, r0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = n;
  return n;
}

// ---------------------------------------------------------------------------
// Dispatch.
#define FA_TPARAMS decltype(dt)::value, decltype(d)::value, decltype(c)::value

hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Hq * a.pb.Nq == 0) return hipSuccess;
  // the atomic path's kernel: built for its head dims only
  return dispatch(a.pb, FT_PLAIN, [&](auto dt, auto d, auto c, auto) -> hipError_t {
    if constexpr (atomic_head_dim(decltype(d)::value)) return run_pre<FA_TPARAMS>(a, s);
    return hipErrorInvalidValue;
  });
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, bool atomic_dq, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Nkv == 0) return hipSuccess;
  if (atomic_dq) {
    // the fused atomic kernel exists for d = 64 and 128 without extras (the API
    // rejects the atomic path otherwise)
    return dispatch(a.pb, FT_PLAIN, [&](auto dt, auto d, auto c, auto) -> hipError_t {
      if constexpr (atomic_head_dim(decltype(d)::value)) return run_dkdv_atomic<FA_TPARAMS>(a, s);
      return hipErrorInvalidValue;
    });
  }
  return dispatch(a.pb, a.x.ft(), [&](auto dt, auto d, auto c, auto ft) {
    return run_dkdv<FA_TPARAMS, decltype(ft)::value>(a, s);
  });
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Nq == 0) return hipSuccess;
  return dispatch(a.pb, a.x.ft(), [&](auto dt, auto d, auto c, auto ft) {
    return run_dq<FA_TPARAMS, decltype(ft)::value>(a, s);
  });
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
