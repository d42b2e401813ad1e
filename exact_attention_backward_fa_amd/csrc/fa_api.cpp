// C entry points of libfa_mi355x.so: argument checks, workspace carve-up and
// kernel sequencing.  Every check runs on the host before the first launch, so a
// rejected call enqueues nothing and writes nothing.
#include "fa_mi355x.h"

#include <math.h>
#include <stdint.h>

#include "fa_internal.hpp"

namespace fa {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WorkspaceLayout workspace_layout(const Problem& pb, bool atomic_dq) {
  const size_t rows = (size_t)pb.B * pb.Hq * pb.Nq;
  WorkspaceLayout L;
  L.ndelta_off = 0;
  L.lse2_off = align256(rows * sizeof(float));
  L.dqacc_off = L.lse2_off + align256(rows * sizeof(float));
  L.sched_off = L.dqacc_off + (atomic_dq ? align256(rows * pb.d * sizeof(float)) : 0);
  L.total = L.sched_off + 256;
  if (rows == 0) L.total = 0;
  return L;
}

static int check_problem(int B, int Hq, int Hkv, int Nq, int Nkv, int d, float scale, int dtype,
                         Problem* out) {
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (!head_dim_supported(d)) return FA_ERR_HEADDIM;
  if (B < 0 || Nq < 0 || Nkv < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (B > 65535 || Hq > 65535) return FA_ERR_SHAPE;  // grid y/z limits
  if ((int64_t)Nq * d >= ((int64_t)1 << 31) || (int64_t)Nkv * d >= ((int64_t)1 << 31))
    return FA_ERR_SHAPE;
  // total element counts must stay well inside size_t arithmetic
  if ((double)B * Hq * (double)Nq * d > 9.0e15 || (double)B * Hkv * (double)Nkv * d > 9.0e15)
    return FA_ERR_SHAPE;
  // 1-D grids: (query or key tiles of >= 64 rows) x heads x batch must fit an int
  const int64_t tiles = ((int64_t)(Nq > Nkv ? Nq : Nkv) + 63) / 64;
  if (tiles * Hq * (int64_t)B >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  out->B = B;
  out->Hq = Hq;
  out->Hkv = Hkv;
  out->Nq = Nq;
  out->Nkv = Nkv;
  out->d = d;
  out->scale = scale;
  out->dtype = dtype;
  out->causal = false;
  return FA_OK;
}

// A pointer is acceptable when the tensor is empty, or when it is non-NULL and
// 16-byte aligned.
static int check_ptr(const void* ptr, size_t elems) {
  if (elems == 0) return FA_OK;
  if (ptr == nullptr) return FA_ERR_NULLPTR;
  if (((uintptr_t)ptr & 15u) != 0) return FA_ERR_ALIGN;
  return FA_OK;
}

// FA_DQ_AUTO: the separate query-parallel dQ pass.  Measured with rocprofv3 on
// MI355X at the causal GQA shape (B=4, Hq=32, Hkv=8, N=8192, d=128, bf16;
// profiles/kernel_trace_llama_gqa_bf16_8192.md and
// profiles/kernel_trace_atomic_dq_llama_gqa_bf16_8192.md): dK/dV 3.10 ms + dQ pass
// 2.45 ms against 13.4 ms for the fused kernel with float atomics.  Its 4.36 G
// atomic adds are performed at the memory side (WRITE_SIZE 17.6 GB per launch,
// profiles/hbm_traffic_atomic_dq_llama_gqa_bf16_8192.txt), not in L2; even half
// as many (256-key blocks) would move 8.8 GB.  The separate pass is also bitwise
// repeatable.
static int resolve_dq_mode(const Problem& pb, int mode) {
  if (mode == FA_DQ_ATOMIC || mode == FA_DQ_SEPARATE) return mode;
  (void)pb;
  return FA_DQ_SEPARATE;
}

// Checks the score bias, its gradient and the dropout arguments; fills *x.
static int check_extras(const Problem& pb, const void* bias, long long sb, long long sh,
                        long long sq, void* dbias, float dropout_p, unsigned long long seed,
                        Extras* x) {
  if (!(dropout_p >= 0.f && dropout_p <= 1.f)) return FA_ERR_DROPOUT;  // NaN fails too
  // keep threshold T = floor((1 - p) * 256 + 1/2), float arithmetic
  const float t = floorf((1.0f - dropout_p) * 256.0f + 0.5f);
  x->keep_t = (unsigned)fminf(fmaxf(t, 0.f), 256.f);
  x->seed = seed;
  x->bias = bias;
  x->dbias = dbias;
  x->bias_sb = bias ? sb : 0;
  x->bias_sh = bias ? sh : 0;
  x->bias_sq = bias ? sq : 0;
  if (bias) {
    // 16-byte aligned rows (the tiles are copied in 16-byte pieces); strides keep
    // a tile's offsets within 32 bits
    if (((uintptr_t)bias & 15u) != 0) return FA_ERR_ALIGN;
    if (sb < 0 || sh < 0 || sq < 0 || (sb & 7) || (sh & 7) || (sq & 7) || sq > (1ll << 22))
      return FA_ERR_BIAS;
  }
  if (dbias && ((uintptr_t)dbias & 15u) != 0) return FA_ERR_ALIGN;
  // dBias rows of a 128-query work item are addressed with 32-bit byte offsets
  if (dbias && pb.Nkv > (1 << 22)) return FA_ERR_BIAS;
  if (x->ft() != FT_PLAIN && !feature_head_dim(x->ft(), pb.d)) return FA_ERR_HEADDIM;
  return FA_OK;
}

int bwd_validate(const BwdCall& c, int dq_mode, size_t* workspace_need, const Extras* x) {
  Problem pb;
  const int st = check_problem(c.B, c.Hq, c.Hkv, c.Nq, c.Nkv, c.d, c.scale, c.dtype, &pb);
  if (st != FA_OK) return st;
  pb.causal = c.causal != 0;
  if (dq_mode != FA_DQ_AUTO && dq_mode != FA_DQ_ATOMIC && dq_mode != FA_DQ_SEPARATE)
    return FA_ERR_MODE;
  // the score bias and dropout run on the separate dQ path only
  if (x && x->ft() != FT_PLAIN && dq_mode == FA_DQ_ATOMIC) return FA_ERR_MODE;
  const size_t nq = (size_t)c.B * c.Hq * c.Nq * c.d, nk = (size_t)c.B * c.Hkv * c.Nkv * c.d;
  const size_t nrows = (size_t)c.B * c.Hq * c.Nq;
  // dK/dV are written whenever they have elements (zeros when N_q = 0).
  const void* ptrs[9] = {c.q, c.k, c.v, c.o, c.lse, c.dout, c.dq, c.dk, c.dv};
  const size_t elems[9] = {nq, nk, nk, nq, nrows, nq, nq, nk, nk};
  for (int i = 0; i < 9; ++i) {
    const int pst = check_ptr(ptrs[i], elems[i]);
    if (pst != FA_OK) return pst;
  }
  const int mode = resolve_dq_mode(pb, dq_mode);
  if (mode == FA_DQ_ATOMIC && !atomic_head_dim(pb.d)) return FA_ERR_HEADDIM;
  *workspace_need = workspace_layout(pb, mode == FA_DQ_ATOMIC).total;
  return FA_OK;
}

int bwd_checked(const BwdCall& c, int dq_mode, void* ev_begin, void* ev_end, void* workspace,
                size_t workspace_bytes, void* stream, const Extras* x) {
  size_t need = 0;
  const int st = bwd_validate(c, dq_mode, &need, x);
  if (st != FA_OK) return st;
  Problem pb;
  (void)check_problem(c.B, c.Hq, c.Hkv, c.Nq, c.Nkv, c.d, c.scale, c.dtype, &pb);
  pb.causal = c.causal != 0;
  const size_t nk = (size_t)c.B * c.Hkv * c.Nkv * c.d;
  const size_t nrows = (size_t)c.B * c.Hq * c.Nq;
  const int mode = resolve_dq_mode(pb, dq_mode);
  const bool atomic = mode == FA_DQ_ATOMIC;
  const WorkspaceLayout L = workspace_layout(pb, atomic);
  if (L.total > 0) {
    if (workspace == nullptr || ((uintptr_t)workspace & 15u) != 0 || workspace_bytes < L.total)
      return FA_ERR_WORKSPACE;
  }
  char* ws = static_cast<char*>(workspace);
  BwdArgs a;
  a.pb = pb;
  a.q = c.q;
  a.k = c.k;
  a.v = c.v;
  a.o = c.o;
  a.lse = c.lse;
  a.dout = c.dout;
  a.dq = c.dq;
  a.dk = c.dk;
  a.dv = c.dv;
  a.ndelta = L.total ? reinterpret_cast<float*>(ws + L.ndelta_off) : nullptr;
  a.lse2 = L.total ? reinterpret_cast<float*>(ws + L.lse2_off) : nullptr;
  a.dq_acc = (L.total && atomic) ? reinterpret_cast<float*>(ws + L.dqacc_off) : nullptr;
  a.sched = L.total ? reinterpret_cast<int*>(ws + L.sched_off) : nullptr;
  if (x) a.x = *x;

  hipStream_t s = (hipStream_t)stream;
  if (nrows == 0 && nk == 0) return FA_OK;  // nothing to compute; no HIP call at all
  (void)hipGetLastError();
  if (atomic) {
    // preprocess (rows, counters, float32 dQ buffer) -> fused dK/dV/dQ -> convert
    if (launch_bwd_pre(a, s) != hipSuccess) return FA_ERR_HIP;
    if (ev_begin && hipEventRecord((hipEvent_t)ev_begin, s) != hipSuccess) return FA_ERR_HIP;
    if (launch_bwd_dkdv(a, true, s) != hipSuccess) return FA_ERR_HIP;
    if (ev_end && hipEventRecord((hipEvent_t)ev_end, s) != hipSuccess) return FA_ERR_HIP;
    if (launch_bwd_dq_convert(a, s) != hipSuccess) return FA_ERR_HIP;
    return FA_OK;
  }
  // counters -> dQ pass (which also leaves -D and LSE * log2 e of every query row
  // for the next kernel) -> dK/dV
  if (launch_sched_clear(a, s) != hipSuccess) return FA_ERR_HIP;
  if (launch_dbias_fill(a, s) != hipSuccess) return FA_ERR_HIP;
  if (launch_bwd_dq(a, s) != hipSuccess) return FA_ERR_HIP;
  if (ev_begin && hipEventRecord((hipEvent_t)ev_begin, s) != hipSuccess) return FA_ERR_HIP;
  if (launch_bwd_dkdv(a, false, s) != hipSuccess) return FA_ERR_HIP;
  if (ev_end && hipEventRecord((hipEvent_t)ev_end, s) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

size_t bwd_workspace_checked(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal, int dtype,
                             int dq_mode) {
  Problem pb;
  if (check_problem(B, Hq, Hkv, Nq, Nkv, d, 1.0f, dtype, &pb) != FA_OK) return 0;
  if (dq_mode != FA_DQ_AUTO && dq_mode != FA_DQ_ATOMIC && dq_mode != FA_DQ_SEPARATE) return 0;
  pb.causal = causal != 0;
  const int mode = resolve_dq_mode(pb, dq_mode);
  if (mode == FA_DQ_ATOMIC && !atomic_head_dim(pb.d)) return 0;
  return workspace_layout(pb, mode == FA_DQ_ATOMIC).total;
}

}  // namespace fa

using namespace fa;

#define FA_TRY(expr)            \
  do {                          \
    const int _st = (expr);     \
    if (_st != FA_OK) return _st; \
  } while (0)

extern "C" {

int fa_version(void) { return 100; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULLPTR: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (B, Hq, Hkv, N_q, N_kv), Hq % Hkv != 0, or a size limit exceeded";
    case FA_ERR_HEADDIM:
      return "head dimension d must be a multiple of 32 up to 256: 32, 64, 96, 128, 160, 192, 224 "
             "or 256 (the atomic dQ path, a bias that varies along heads or rows, dBias and "
             "dropout: 64 or 128)";
    case FA_ERR_DTYPE: return "dtype must be FA_DTYPE_FP16 or FA_DTYPE_BF16";
    case FA_ERR_SCALE: return "softmax_scale must be finite and > 0";
    case FA_ERR_WORKSPACE: return "workspace is NULL, misaligned, or smaller than required";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_HIP: return "a HIP kernel launch failed";
    case FA_ERR_MODE: return "unknown dq_mode";
    case FA_ERR_BIAS:
      return "bias strides must be >= 0, multiples of 8 elements, the row stride <= 2^22, and "
             "N_kv <= 2^22 when dbias is requested";
    case FA_ERR_DROPOUT: return "dropout_p must be in [0, 1]";
    case FA_ERR_SCRATCH:
      return "the problem needs more scratch than fa_bwd_noalloc holds (FA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
           int Nq, int Nkv, int d, float softmax_scale, int causal, int dtype, void* stream) {
  return fa_fwd_bias_dropout(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, d, softmax_scale, causal, dtype,
                             nullptr, 0, 0, 0, 0.f, 0, stream);
}

int fa_fwd_bias_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int Hq, int Hkv, int Nq, int Nkv, int d, float softmax_scale, int causal,
                        int dtype, const void* bias, long long bias_stride_b,
                        long long bias_stride_h, long long bias_stride_q, float dropout_p,
                        unsigned long long seed, void* stream) {
  Problem pb;
  FA_TRY(check_problem(B, Hq, Hkv, Nq, Nkv, d, softmax_scale, dtype, &pb));
  pb.causal = causal != 0;
  Extras x;
  FA_TRY(check_extras(pb, bias, bias_stride_b, bias_stride_h, bias_stride_q, nullptr, dropout_p,
                      seed, &x));
  const size_t nq = (size_t)B * Hq * Nq * d, nk = (size_t)B * Hkv * Nkv * d;
  const size_t nrows = (size_t)B * Hq * Nq;
  // K and V are read only when some query row exists.
  const size_t nk_used = nrows ? nk : 0;
  FA_TRY(check_ptr(q, nq));
  FA_TRY(check_ptr(k, nk_used));
  FA_TRY(check_ptr(v, nk_used));
  FA_TRY(check_ptr(o, nq));
  FA_TRY(check_ptr(lse, nrows));
  FwdArgs a{pb, q, k, v, o, lse, x};
  if (nrows == 0) return FA_OK;  // nothing to compute; no HIP call at all
  (void)hipGetLastError();
  if (launch_fwd(a, (hipStream_t)stream) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

size_t fa_bwd_ex_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal,
                                 int dtype, int dq_mode) {
  return bwd_workspace_checked(B, Hq, Hkv, Nq, Nkv, d, causal, dtype, dq_mode);
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal,
                              int dtype) {
  return fa_bwd_ex_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, causal, dtype, FA_DQ_AUTO);
}

int fa_bwd_auto_dq_mode(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal, int dtype) {
  Problem pb;
  if (check_problem(B, Hq, Hkv, Nq, Nkv, d, 1.0f, dtype, &pb) != FA_OK) return FA_DQ_ATOMIC;
  pb.causal = causal != 0;
  return resolve_dq_mode(pb, FA_DQ_AUTO);
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
              int Nkv, int d, float softmax_scale, int causal, int dtype, int dq_mode,
              void* ev_begin, void* ev_end, void* workspace, size_t workspace_bytes,
              void* stream) {
  BwdCall c{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, d, softmax_scale, causal, dtype};
  return fa::bwd_checked(c, dq_mode, ev_begin, ev_end, workspace, workspace_bytes, stream);
}

int fa_bwd_bias_dropout(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                        int Hq, int Hkv, int Nq, int Nkv, int d, float softmax_scale, int causal,
                        int dtype, const void* bias, long long bias_stride_b,
                        long long bias_stride_h, long long bias_stride_q, void* dbias,
                        float dropout_p, unsigned long long seed, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Problem pb;
  FA_TRY(check_problem(B, Hq, Hkv, Nq, Nkv, d, softmax_scale, dtype, &pb));
  pb.causal = causal != 0;
  Extras x;
  FA_TRY(check_extras(pb, bias, bias_stride_b, bias_stride_h, bias_stride_q, dbias, dropout_p, seed,
                      &x));
  if (dbias) FA_TRY(check_ptr(dbias, (size_t)B * Hq * Nq * Nkv));
  BwdCall c{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, d, softmax_scale, causal, dtype};
  return bwd_checked(c, FA_DQ_SEPARATE, nullptr, nullptr, workspace, workspace_bytes, stream, &x);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
           int Nkv, int d, float softmax_scale, int causal, int dtype, void* workspace,
           size_t workspace_bytes, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, d, softmax_scale,
                   causal, dtype, FA_DQ_AUTO, nullptr, nullptr, workspace, workspace_bytes,
                   stream);
}

}  // extern "C"
