// ffa_api.hip - host side of the libffa C ABI: argument validation, metadata
// layout and kernel dispatch.  Nothing here allocates or synchronises; every
// call only enqueues kernels on the caller's stream.  The one piece of state
// is the per-device address of the static backward scratch (end of file).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "ffa_internal.hpp"

using namespace ffa;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// q2k and k2q tile counts touched by one slice's bounding rectangle, plus the
// forward query blocks it spans: an upper bound on its CSR entries.
int64_t slice_bound(const int32_t* s, int32_t Tq, int32_t Tk) {
  const int64_t q0 = s[0], q1 = s[1], k0 = s[2], k1 = s[3];
  if (!(0 <= q0 && q0 < q1 && q1 <= Tq && 0 <= k0 && k0 < k1 && k1 <= Tk)) return 0;
  auto span = [](int64_t a, int64_t b, int64_t B) { return (b - 1) / B - a / B + 1; };
  return span(q0, q1, BM_F) * span(k0, k1, BN_F) + span(q0, q1, BM_B) * span(k0, k1, BN_B) +
         span(q0, q1, BM_F);
}

int64_t capacity_bound(int32_t S, int32_t Tq, int32_t Tk, const int32_t* host_slices) {
  const MetaLayout L = meta_layout(S, Tq, Tk);
  const int64_t dense = (int64_t)L.nq_f * L.nk_f + (int64_t)L.nq_b * L.nk_b + (int64_t)L.nq_f * S;
  if (!host_slices) return dense;
  int64_t b = 0;
  for (int32_t i = 0; i < S; ++i) b += slice_bound(host_slices + 5 * i, Tq, Tk);
  return b < dense ? b : dense;
}

bool check_tensor(const void* p, int64_t ts, int64_t hs, int64_t T, int64_t H, int D) {
  if (T == 0) return true;
  if (!p || !aligned(p, 16)) return false;
  if (ts < 0 || hs < 0 || ts % 8 || hs % 8) return false;
  // tiles are read through buffer descriptors whose range is the tile's
  // valid rows times the token stride (up to 128 rows): a stride below
  // head_dim would cut a row short even for a single token
  if (ts < D || ts >= (1LL << 23)) return false;
  (void)H;
  return true;
}

// An output's rows (one per token and head, head_dim elements each) must not
// share elements, or two workgroups would race on them: with the axes of
// more than one element ordered by stride, the inner stride must be at
// least head_dim and the outer one must clear all rows of the inner axis.
// Views into one packed tensor (say dq, dk, dv of [T][3 H][D]) pass.
bool rows_disjoint(int64_t ts, int64_t hs, int64_t T, int64_t H, int D) {
  if (T == 0) return true;
  int64_t s_in = ts, n_in = T, s_out = hs, n_out = H;
  if (n_in == 1 || (n_out > 1 && hs < ts)) {
    s_in = hs;
    n_in = H;
    s_out = ts;
    n_out = T;
  }
  if (n_in > 1 && s_in < D) return false;
  if (n_out > 1 && s_out < (n_in > 1 ? s_in * n_in : (int64_t)D)) return false;
  return true;
}

ffa_status check_shape(const ffa_shape* s) {
  if (!s) return FFA_ERR_INVALID_ARGUMENT;
  if (s->seqlen_q < 0 || s->seqlen_k < 0 || s->num_heads_q < 1 || s->num_heads_kv < 1)
    return FFA_ERR_INVALID_ARGUMENT;
  if (s->num_heads_q % s->num_heads_kv) return FFA_ERR_INVALID_ARGUMENT;
  if (s->head_dim != 64 && s->head_dim != 128) return FFA_ERR_UNSUPPORTED;
  if (!std::isfinite(s->softmax_scale) || !(s->softmax_scale > 0.f)) return FFA_ERR_INVALID_ARGUMENT;
  return FFA_OK;
}

}  // namespace

namespace {

// Backward workspace: -D, LSE log2 e and -LSE / scale rows, then the split
// counters and the split partial sums of the dK/dV kernel, each 256-byte
// aligned.
struct BwdWsLayout {
  int64_t lvec, mvec, cnt, part, total;
  int32_t split_e;
};

BwdWsLayout bwd_ws_layout(const ffa_shape& s) {
  BwdWsLayout W;
  const int64_t rows = align256(4LL * s.num_heads_q * s.seqlen_q);
  const int32_t nk_b = cdiv(s.seqlen_k, BN_B);
  W.split_e = split_candidates(s.num_heads_kv, nk_b);
  const int64_t nc = (int64_t)W.split_e * s.num_heads_kv;
  W.lvec = rows;
  W.mvec = 2 * rows;
  W.cnt = 3 * rows;
  W.part = W.cnt + align256(4 * nc);
  W.total = W.part + nc * 2 * 2 * BN_B * (int64_t)s.head_dim * 4;
  return W;
}

// dK/dV workgroups resident at once on the current device (two per compute
// unit); asked on every call, the library keeps no state.
int resident_dkdv_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 0;
  return 2 * cus;
}

}  // namespace

namespace {

// Validate and copy the mask groups of a grouped call.
ffa_status fill_groups(int32_t n, const void* const* metas, const int32_t* kv_end, int32_t Hkv,
                       MaskGroups& g) {
  if (n < 1 || n > FFA_MAX_MASK_GROUPS || !metas || !kv_end) return FFA_ERR_INVALID_ARGUMENT;
  int32_t prev = 0;
  for (int32_t j = 0; j < n; ++j) {
    if (!metas[j] || !aligned(metas[j], 256)) return FFA_ERR_INVALID_ARGUMENT;
    if (kv_end[j] <= prev) return FFA_ERR_INVALID_ARGUMENT;
    prev = kv_end[j];
  }
  if (prev != Hkv) return FFA_ERR_INVALID_ARGUMENT;
  for (int32_t j = 0; j < FFA_MAX_MASK_GROUPS; ++j) {
    g.meta[j] = j < n ? metas[j] : metas[n - 1];
    g.kv_end[j] = j < n ? kv_end[j] : Hkv;
  }
  g.n = n;
  return FFA_OK;
}

}  // namespace

extern "C" {

FFA_API int32_t ffa_abi_version(void) { return FFA_ABI_VERSION; }

FFA_API const char* ffa_status_string(ffa_status s) {
  switch (s) {
    case FFA_OK: return "ok";
    case FFA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FFA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FFA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FFA_ERR_HIP: return "HIP launch failed";
    case FFA_ERR_BAD_SLICES: return "bad slice table";
    case FFA_ERR_TOO_LARGE: return "shape needs more scratch than the static array holds";
  }
  return "unknown status";
}

FFA_API ffa_status ffa_block_meta_workspace_size(int32_t num_slices, int32_t seqlen_q,
                                                 int32_t seqlen_k, int32_t head_dim,
                                                 const int32_t* host_slices, size_t* bytes) {
  if (!bytes || num_slices < 0 || seqlen_q < 0 || seqlen_k < 0) return FFA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return FFA_ERR_UNSUPPORTED;
  const MetaLayout L = meta_layout(num_slices, seqlen_q, seqlen_k);
  const int64_t cap = capacity_bound(num_slices, seqlen_q, seqlen_k, host_slices);
  *bytes = (size_t)(L.fixed_bytes + align256(4 * cap));
  return FFA_OK;
}

FFA_API ffa_status ffa_build_block_meta(const int32_t* d_slices, int32_t num_slices,
                                        int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                        void* d_meta, size_t meta_bytes, void* stream) {
  if (num_slices < 0 || seqlen_q < 0 || seqlen_k < 0) return FFA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return FFA_ERR_UNSUPPORTED;
  if (!d_meta || !aligned(d_meta, 256)) return FFA_ERR_INVALID_ARGUMENT;
  if (num_slices > 0 && (!d_slices || !aligned(d_slices, 4))) return FFA_ERR_INVALID_ARGUMENT;
  const MetaLayout L = meta_layout(num_slices, seqlen_q, seqlen_k);
  if ((int64_t)meta_bytes < L.fixed_bytes) return FFA_ERR_WORKSPACE_TOO_SMALL;
  const int64_t capacity = ((int64_t)meta_bytes - L.fixed_bytes) / 4;
  hipError_t e = launch_build_meta(d_slices, num_slices, seqlen_q, seqlen_k, head_dim, d_meta,
                                   capacity, L, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FFA_OK : FFA_ERR_HIP;
}

FFA_API ffa_status ffa_block_meta_view(const void* d_meta, int32_t num_slices, int32_t seqlen_q,
                                       int32_t seqlen_k, int32_t head_dim,
                                       ffa_block_meta_view_t* out) {
  if (!d_meta || !out || num_slices < 0 || seqlen_q < 0 || seqlen_k < 0)
    return FFA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return FFA_ERR_UNSUPPORTED;
  const MetaLayout L = meta_layout(num_slices, seqlen_q, seqlen_k);
  const char* b = reinterpret_cast<const char*>(d_meta);
  std::memset(out, 0, sizeof(*out));
  out->bm_fwd = BM_F;
  out->bn_fwd = BN_F;
  out->bm_bwd = BM_B;
  out->bn_bwd = BN_B;
  out->num_qblocks_fwd = L.nq_f;
  out->num_kblocks_fwd = L.nk_f;
  out->num_qblocks_bwd = L.nq_b;
  out->num_kblocks_bwd = L.nk_b;
  out->header_bytes = HEADER_BYTES;
  out->status = reinterpret_cast<const int32_t*>(b + offsetof(MetaHeader, status));
  out->area = reinterpret_cast<const int64_t*>(b + offsetof(MetaHeader, area));
  out->list_offsets = reinterpret_cast<const int64_t*>(b + offsetof(MetaHeader, list_off));
  out->full_block_offset = reinterpret_cast<const int32_t*>(b + L.byte_off[A_QF_OFF]);
  out->mask_block_offset = reinterpret_cast<const int32_t*>(b + L.byte_off[A_QM_OFF]);
  out->k2q_full_block_offset = reinterpret_cast<const int32_t*>(b + L.byte_off[A_KF_OFF]);
  out->k2q_mask_block_offset = reinterpret_cast<const int32_t*>(b + L.byte_off[A_KM_OFF]);
  out->qblock_slice_offset = reinterpret_cast<const int32_t*>(b + L.byte_off[A_QS_OFF]);
  out->schedule_fwd = reinterpret_cast<const int32_t*>(b + L.byte_off[A_SCHED_F]);
  out->schedule_bwd = reinterpret_cast<const int32_t*>(b + L.byte_off[A_SCHED_B]);
  out->index_base = reinterpret_cast<const int32_t*>(b + L.byte_off[A_VAR]);
  out->block_records_fwd = reinterpret_cast<const int32_t*>(b + L.byte_off[A_REC_F]);
  out->block_records_bwd = reinterpret_cast<const int32_t*>(b + L.byte_off[A_REC_B]);
  return FFA_OK;
}

FFA_API ffa_status ffa_fwd(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                           ffa_tensor_in v, const void* d_meta, ffa_tensor_out o, float* lse,
                           void* stream) {
  return ffa_fwd_ex(shape, q, k, v, d_meta, o, lse, 0u, stream);
}

FFA_API ffa_status ffa_fwd_ex(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                              ffa_tensor_in v, const void* d_meta, ffa_tensor_out o, float* lse,
                              uint32_t flags, void* stream) {
  const int32_t all = shape ? shape->num_heads_kv : 0;
  return ffa_fwd_grouped(shape, q, k, v, 1, &d_meta, &all, o, lse, flags, stream);
}

FFA_API ffa_status ffa_fwd_grouped(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                                   ffa_tensor_in v, int32_t num_groups, const void* const* d_metas,
                                   const int32_t* kv_head_end, ffa_tensor_out o, float* lse,
                                   uint32_t flags, void* stream) {
  if (flags & ~FFA_ACCUMULATE) return FFA_ERR_INVALID_ARGUMENT;
  ffa_status st = check_shape(shape);
  if (st != FFA_OK) return st;
  const int D = shape->head_dim, Tq = shape->seqlen_q, Tk = shape->seqlen_k;
  const int Hq = shape->num_heads_q, Hkv = shape->num_heads_kv;
  if (!check_tensor(q.ptr, q.token_stride, q.head_stride, Tq, Hq, D) ||
      !check_tensor(o.ptr, o.token_stride, o.head_stride, Tq, Hq, D) ||
      !check_tensor(k.ptr, k.token_stride, k.head_stride, Tk, Hkv, D) ||
      !check_tensor(v.ptr, v.token_stride, v.head_stride, Tk, Hkv, D) ||
      !rows_disjoint(o.token_stride, o.head_stride, Tq, Hq, D))
    return FFA_ERR_INVALID_ARGUMENT;
  if (Tq > 0 && (!lse || !aligned(lse, 16))) return FFA_ERR_INVALID_ARGUMENT;
  FwdArgs a;
  if (fill_groups(num_groups, d_metas, kv_head_end, Hkv, a.groups) != FFA_OK)
    return FFA_ERR_INVALID_ARGUMENT;
  if (Tq == 0) return FFA_OK;
  const MetaLayout L = meta_layout(0, Tq, Tk);
  a.q = static_cast<const __bf16*>(q.ptr);
  a.k = static_cast<const __bf16*>(k.ptr);
  a.v = static_cast<const __bf16*>(v.ptr);
  a.o = static_cast<__bf16*>(o.ptr);
  a.lse = lse;
  a.q_ts = q.token_stride;
  a.q_hs = q.head_stride;
  a.k_ts = k.token_stride;
  a.k_hs = k.head_stride;
  a.v_ts = v.token_stride;
  a.v_hs = v.head_stride;
  a.o_ts = o.token_stride;
  a.o_hs = o.head_stride;
  a.Tq = Tq;
  a.Tk = Tk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.nitems = L.nq_f;
  a.rec_off = L.byte_off[A_REC_F];
  a.scale = shape->softmax_scale;
  a.scale_log2 = shape->softmax_scale * LOG2E;
  a.flags = flags;
  hipError_t e = launch_fwd(a, D, L.nq_f, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FFA_OK : FFA_ERR_HIP;
}

FFA_API ffa_status ffa_bwd_workspace_size(const ffa_shape* shape, size_t* bytes) {
  ffa_status st = check_shape(shape);
  if (st != FFA_OK) return st;
  if (!bytes) return FFA_ERR_INVALID_ARGUMENT;
  *bytes = (size_t)bwd_ws_layout(*shape).total;
  return FFA_OK;
}

FFA_API ffa_status ffa_bwd(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                           ffa_tensor_in v, ffa_tensor_in o, const float* lse,
                           ffa_tensor_in dout, const void* d_meta, ffa_tensor_out dq,
                           ffa_tensor_out dk, ffa_tensor_out dv, void* d_ws, size_t ws_bytes,
                           void* stream) {
  return ffa_bwd_phases(shape, q, k, v, o, lse, dout, d_meta, dq, dk, dv, d_ws, ws_bytes,
                        FFA_BWD_ALL, stream);
}

FFA_API ffa_status ffa_bwd_phases(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                                  ffa_tensor_in v, ffa_tensor_in o, const float* lse,
                                  ffa_tensor_in dout, const void* d_meta, ffa_tensor_out dq,
                                  ffa_tensor_out dk, ffa_tensor_out dv, void* d_ws,
                                  size_t ws_bytes, int32_t phases, void* stream) {
  return ffa_bwd_ex(shape, q, k, v, o, lse, dout, d_meta, dq, dk, dv, d_ws, ws_bytes, phases, 0u,
                    stream);
}

FFA_API ffa_status ffa_bwd_ex(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                              ffa_tensor_in v, ffa_tensor_in o, const float* lse,
                              ffa_tensor_in dout, const void* d_meta, ffa_tensor_out dq,
                              ffa_tensor_out dk, ffa_tensor_out dv, void* d_ws, size_t ws_bytes,
                              int32_t phases, uint32_t flags, void* stream) {
  const int32_t all = shape ? shape->num_heads_kv : 0;
  return ffa_bwd_grouped(shape, q, k, v, o, lse, dout, 1, &d_meta, &all, dq, dk, dv, d_ws,
                         ws_bytes, phases, flags, stream);
}

FFA_API ffa_status ffa_bwd_grouped(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                                   ffa_tensor_in v, ffa_tensor_in o, const float* lse,
                                   ffa_tensor_in dout, int32_t num_groups, const void* const* d_metas,
                                   const int32_t* kv_head_end, ffa_tensor_out dq, ffa_tensor_out dk,
                                   ffa_tensor_out dv, void* d_ws, size_t ws_bytes, int32_t phases,
                                   uint32_t flags, void* stream) {
  if (phases & ~FFA_BWD_ALL) return FFA_ERR_INVALID_ARGUMENT;
  if (flags & ~FFA_ACCUMULATE) return FFA_ERR_INVALID_ARGUMENT;
  ffa_status st = check_shape(shape);
  if (st != FFA_OK) return st;
  const int D = shape->head_dim, Tq = shape->seqlen_q, Tk = shape->seqlen_k;
  const int Hq = shape->num_heads_q, Hkv = shape->num_heads_kv;
  if (!check_tensor(q.ptr, q.token_stride, q.head_stride, Tq, Hq, D) ||
      !check_tensor(o.ptr, o.token_stride, o.head_stride, Tq, Hq, D) ||
      !check_tensor(dout.ptr, dout.token_stride, dout.head_stride, Tq, Hq, D) ||
      !check_tensor(dq.ptr, dq.token_stride, dq.head_stride, Tq, Hq, D) ||
      !check_tensor(k.ptr, k.token_stride, k.head_stride, Tk, Hkv, D) ||
      !check_tensor(v.ptr, v.token_stride, v.head_stride, Tk, Hkv, D) ||
      !check_tensor(dk.ptr, dk.token_stride, dk.head_stride, Tk, Hkv, D) ||
      !check_tensor(dv.ptr, dv.token_stride, dv.head_stride, Tk, Hkv, D) ||
      !rows_disjoint(dq.token_stride, dq.head_stride, Tq, Hq, D) ||
      !rows_disjoint(dk.token_stride, dk.head_stride, Tk, Hkv, D) ||
      !rows_disjoint(dv.token_stride, dv.head_stride, Tk, Hkv, D))
    return FFA_ERR_INVALID_ARGUMENT;
  if (Tq > 0 && (!lse || !aligned(lse, 16))) return FFA_ERR_INVALID_ARGUMENT;
  BwdArgs a;
  if (fill_groups(num_groups, d_metas, kv_head_end, Hkv, a.groups) != FFA_OK)
    return FFA_ERR_INVALID_ARGUMENT;
  size_t need = 0;
  ffa_bwd_workspace_size(shape, &need);
  if (need > 0 && (!d_ws || !aligned(d_ws, 256))) return FFA_ERR_INVALID_ARGUMENT;
  if (ws_bytes < need) return FFA_ERR_WORKSPACE_TOO_SMALL;
  if (Tq == 0 && Tk == 0) return FFA_OK;
  const MetaLayout L = meta_layout(0, Tq, Tk);
  a.q = static_cast<const __bf16*>(q.ptr);
  a.k = static_cast<const __bf16*>(k.ptr);
  a.v = static_cast<const __bf16*>(v.ptr);
  a.o = static_cast<const __bf16*>(o.ptr);
  a.dout = static_cast<const __bf16*>(dout.ptr);
  a.lse = lse;
  const BwdWsLayout W = bwd_ws_layout(*shape);
  char* ws = static_cast<char*>(d_ws);
  a.dvec = reinterpret_cast<float*>(ws);
  a.lvec = reinterpret_cast<float*>(ws + W.lvec);
  a.mvec = reinterpret_cast<float*>(ws + W.mvec);
  a.split_cnt = reinterpret_cast<int32_t*>(ws + W.cnt);
  a.split_part = reinterpret_cast<float*>(ws + W.part);
  a.split_e = W.split_e;
  a.split_slots = 0;
  if (W.split_e > 0) {
    a.split_slots = resident_dkdv_slots();
    if (a.split_slots <= 0) return FFA_ERR_HIP;
  }
  a.dq = static_cast<__bf16*>(dq.ptr);
  a.dk = static_cast<__bf16*>(dk.ptr);
  a.dv = static_cast<__bf16*>(dv.ptr);
  a.q_ts = q.token_stride;
  a.q_hs = q.head_stride;
  a.k_ts = k.token_stride;
  a.k_hs = k.head_stride;
  a.v_ts = v.token_stride;
  a.v_hs = v.head_stride;
  a.o_ts = o.token_stride;
  a.o_hs = o.head_stride;
  a.do_ts = dout.token_stride;
  a.do_hs = dout.head_stride;
  a.dq_ts = dq.token_stride;
  a.dq_hs = dq.head_stride;
  a.dk_ts = dk.token_stride;
  a.dk_hs = dk.head_stride;
  a.dv_ts = dv.token_stride;
  a.dv_hs = dv.head_stride;
  a.Tq = Tq;
  a.Tk = Tk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.nq_f = L.nq_f;
  a.nk_b = L.nk_b;
  a.rec_off_f = L.byte_off[A_REC_F];
  a.rec_off_b = L.byte_off[A_REC_B];
  a.scale = shape->softmax_scale;
  a.scale_log2 = shape->softmax_scale * LOG2E;
  a.flags = flags;
  hipError_t e = launch_bwd(a, D, L.nq_f, L.nk_b, phases, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FFA_OK : FFA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward for callers that cannot allocate: its scratch lives in a static
// device array of FFA_STATIC_SCRATCH_BYTES.  Each GPU holds its own copy of
// the array at its own address; host code never passes the symbol itself to
// a kernel (in host code it names a host-side stand-in), only the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
// ---------------------------------------------------------------------------
__device__ __attribute__((aligned(256))) char scratch[FFA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Address of the scratch array on the current device (set up on first use).
ffa_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FFA_ERR_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return FFA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FFA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FFA_OK;
}

}  // namespace

extern "C" FFA_API ffa_status ffa_bwd_static_scratch(const ffa_shape* shape, ffa_tensor_in q,
                                                     ffa_tensor_in k, ffa_tensor_in v,
                                                     ffa_tensor_in o, const float* lse,
                                                     ffa_tensor_in dout, const void* d_meta,
                                                     ffa_tensor_out dq, ffa_tensor_out dk,
                                                     ffa_tensor_out dv, void* stream) {
  size_t need = 0;
  const ffa_status st = ffa_bwd_workspace_size(shape, &need);
  if (st != FFA_OK) return st;
  if (need > (size_t)FFA_STATIC_SCRATCH_BYTES) return FFA_ERR_TOO_LARGE;
  void* ws = nullptr;
  const ffa_status sp = static_scratch(&ws);
  if (sp != FFA_OK) return sp;
  // the split counters are zeroed by the first backward kernel of the call
  // (the dQ kernel with the row statistics), as with a caller's workspace
  return ffa_bwd_phases(shape, q, k, v, o, lse, dout, d_meta, dq, dk, dv, ws,
                        (size_t)FFA_STATIC_SCRATCH_BYTES, FFA_BWD_ALL, stream);
}
