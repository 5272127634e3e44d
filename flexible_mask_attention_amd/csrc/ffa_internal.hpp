// ffa_internal.hpp - shared definitions of the HIP sources of libffa (gfx950).
//
// Holds the block-metadata layout, tile shapes, the slice interval helpers and
// the small wave-level building blocks (MFMA 32x32x16 bf16, LDS swizzle,
// transposed LDS reads) used by the forward and backward kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ffa.h"

namespace ffa {

// ---------------------------------------------------------------------------
// Tile shapes.  The forward and the dQ kernel walk key tiles of BN_F keys for
// query blocks of BM_F rows (q2k lists); the dK/dV kernel walks query tiles of
// BM_B rows for key blocks of BN_B keys (k2q lists).  Per-query-block slice
// lists are built at BM_F granularity; BM_B must divide BM_F.
// ---------------------------------------------------------------------------
constexpr int BM_F = 128;
constexpr int BN_F = 64;
constexpr int BM_B = 64;
constexpr int BN_B = 128;
static_assert(BM_F % BM_B == 0, "bwd query blocks must nest in fwd query blocks");

constexpr uint32_t META_MAGIC = 0x4D414646u;  // "FFAM"
constexpr int META_VERSION = 1;

// Header at offset 0 of the metadata buffer.  Fields marked (dev) are written
// by the build kernels; the rest are written from host-known values by the
// first build kernel.
struct MetaHeader {
  uint32_t magic;
  int32_t version;
  int32_t status;        // (dev) FFA_META_ERR_* flags
  int32_t num_slices;
  int32_t seqlen_q, seqlen_k, head_dim, pad0;
  int32_t bm_f, bn_f, bm_b, bn_b;
  int32_t nq_f, nk_f, nq_b, nk_b;   // block counts at both tilings
  int64_t capacity;      // int32 entries in the variable region
  int64_t area;          // (dev) exact valid-pair count
  int64_t nnz[5];        // (dev) q2k full, q2k mask, k2q full, k2q mask, q-block slices
  int64_t list_off[5];   // (dev) entry offsets of those lists in the variable region
  int64_t byte_off[11];  // offsets of the fixed arrays (see MetaLayout)
  int64_t pad1[1];
};
static_assert(sizeof(MetaHeader) <= 256, "header must fit in 256 bytes");
constexpr int64_t HEADER_BYTES = 256;

enum ListId { L_QF = 0, L_QM = 1, L_KF = 2, L_KM = 3, L_QS = 4 };

// Fixed arrays, in this order after the header (int32, each padded to 256 B):
//   q2k_full_off[nq_f+1], q2k_mask_off[nq_f+1], k2q_full_off[nk_b+1],
//   k2q_mask_off[nk_b+1], qs_off[nq_f+1], sched_f[nq_f], sched_b[nk_b],
//   rec_f[nq_f][REC], rec_b[nk_b][REC], slices[5*S], then the variable region.
// Everything before the slice copy depends on the sequence lengths only, so
// the host knows where the block records are without reading the buffer.
enum FixedId { A_QF_OFF = 0, A_QM_OFF, A_KF_OFF, A_KM_OFF, A_QS_OFF, A_SCHED_F, A_SCHED_B,
               A_REC_F, A_REC_B, A_SLICES, A_VAR };

// Block record, one per owner in schedule order (int32 each): what a
// forward / dQ (rec_f) or dK/dV (rec_b) workgroup needs before its first tile
// load, in one 64-byte read.
//   rec_f: owner q-block, q2k Full list offset and count, Partial list offset
//          and count, slice list offset and count, first Full tile, first
//          Partial tile (-1 when the list is empty)
//   rec_b: owner k-block, k2q Full list offset and count, Partial list offset
//          and count, last Full tile, last Partial tile (-1 when empty)
constexpr int REC = 16;
enum RecField { R_OWNER = 0, R_F0, R_NF, R_P0, R_NP, R_S0, R_NS, R_TF, R_TP };
enum RecFieldB { RB_OWNER = 0, RB_F0, RB_NF, RB_P0, RB_NP, RB_TF, RB_TP };

struct MetaLayout {
  int32_t nq_f, nk_f, nq_b, nk_b;
  int64_t byte_off[11];
  int64_t fixed_bytes;
};

__host__ __device__ inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
__host__ __device__ inline int32_t cdiv(int32_t a, int32_t b) { return (a + b - 1) / b; }

inline MetaLayout meta_layout(int32_t S, int32_t Tq, int32_t Tk) {
  MetaLayout L;
  L.nq_f = cdiv(Tq, BM_F);
  L.nk_f = cdiv(Tk, BN_F);
  L.nq_b = cdiv(Tq, BM_B);
  L.nk_b = cdiv(Tk, BN_B);
  const int64_t counts[10] = {L.nq_f + 1LL, L.nq_f + 1LL, L.nk_b + 1LL, L.nk_b + 1LL,
                              L.nq_f + 1LL, (int64_t)L.nq_f, (int64_t)L.nk_b,
                              (int64_t)REC * L.nq_f, (int64_t)REC * L.nk_b, 5LL * S};
  int64_t off = HEADER_BYTES;
  for (int i = 0; i < 10; ++i) {
    L.byte_off[i] = off;
    off += align256(4 * counts[i]);
  }
  L.byte_off[A_VAR] = off;
  L.fixed_bytes = off;
  return L;
}

// Device view of a built metadata buffer, read through the constant address
// space: the buffer does not change while forward / backward kernels run, so
// uniform reads of it become scalar loads.
#define FFA_CONST __attribute__((address_space(4)))
typedef const FFA_CONST int32_t cint32_t;

struct MetaView {
  const FFA_CONST MetaHeader* hdr;
  cint32_t* slices;
  cint32_t* qf_off;
  cint32_t* qm_off;
  cint32_t* kf_off;
  cint32_t* km_off;
  cint32_t* qs_off;
  cint32_t* sched_f;
  cint32_t* sched_b;
  cint32_t* rec_f;
  cint32_t* rec_b;
  cint32_t* var;
};

// The checks a workgroup makes before it reads a metadata buffer: built
// without error and for these sequence lengths, which also places the block
// records where the host expects them (rec_id, at byte offset rec_off).  The
// four header words are compared without short-circuit so that they are read
// in one round trip.
__device__ inline bool meta_usable(const FFA_CONST MetaHeader* hd, int Tq, int Tk, int rec_id,
                                   int64_t rec_off) {
  return ((hd->status == 0) & (hd->seqlen_q == Tq) & (hd->seqlen_k == Tk) &
          (hd->byte_off[rec_id] == rec_off)) != 0;
}

__device__ inline MetaView meta_view(const void* meta) {
  MetaView v;
  const FFA_CONST char* b = (const FFA_CONST char*)(meta);
  v.hdr = (const FFA_CONST MetaHeader*)(b);
  v.slices = (cint32_t*)(b + v.hdr->byte_off[A_SLICES]);
  v.qf_off = (cint32_t*)(b + v.hdr->byte_off[A_QF_OFF]);
  v.qm_off = (cint32_t*)(b + v.hdr->byte_off[A_QM_OFF]);
  v.kf_off = (cint32_t*)(b + v.hdr->byte_off[A_KF_OFF]);
  v.km_off = (cint32_t*)(b + v.hdr->byte_off[A_KM_OFF]);
  v.qs_off = (cint32_t*)(b + v.hdr->byte_off[A_QS_OFF]);
  v.sched_f = (cint32_t*)(b + v.hdr->byte_off[A_SCHED_F]);
  v.sched_b = (cint32_t*)(b + v.hdr->byte_off[A_SCHED_B]);
  v.rec_f = (cint32_t*)(b + v.hdr->byte_off[A_REC_F]);
  v.rec_b = (cint32_t*)(b + v.hdr->byte_off[A_REC_B]);
  v.var = (cint32_t*)(b + v.hdr->byte_off[A_VAR]);
  return v;
}

// Wait until this wave's vector-memory loads issued so far (by compiled
// code) have returned; the compiler tracks this builtin, unlike wait_dma.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// Slice intervals.  For slice (q0,q1,k0,k1,t) the valid keys of query row i
// form one interval, and so do the valid queries of key column j; both are
// the mask predicate solved for one coordinate.  Inclusive bounds; lo > hi
// means empty.
// ---------------------------------------------------------------------------
struct Slice {
  int32_t q0, q1, k0, k1, t;
};

template <typename P>
__device__ __forceinline__ Slice load_slice(P s, int idx) {
  Slice r;
  r.q0 = s[5 * idx + 0];
  r.q1 = s[5 * idx + 1];
  r.k0 = s[5 * idx + 2];
  r.k1 = s[5 * idx + 3];
  r.t = s[5 * idx + 4];
  return r;
}

__device__ __forceinline__ bool slice_ok(const Slice& s, int Tq, int Tk) {
  return 0 <= s.q0 && s.q0 <= s.q1 && s.q1 <= Tq && 0 <= s.k0 && s.k0 <= s.k1 && s.k1 <= Tk &&
         s.t >= 0 && s.t <= 3;
}

// keys valid for query row i: c in [lo_c, hi_c] with c = j - k0
__device__ __forceinline__ void row_interval(const Slice& s, int i, int& lo, int& hi) {
  const int r = i - s.q0, Lq = s.q1 - s.q0, Lk = s.k1 - s.k0;
  const bool inv = (s.t == FFA_INV_CAUSAL) | (s.t == FFA_BI_CAUSAL);
  const bool cau = (s.t == FFA_CAUSAL) | (s.t == FFA_BI_CAUSAL);
  int l = inv ? r : 0;
  int h = cau ? min(Lk - 1, r + Lk - Lq) : Lk - 1;
  if (i < s.q0 || i >= s.q1) { l = 1; h = 0; }
  lo = s.k0 + l;
  hi = s.k0 + h;
}

// queries valid for key column j: r in [lo_r, hi_r] with r = i - q0
__device__ __forceinline__ void col_interval(const Slice& s, int j, int& lo, int& hi) {
  const int c = j - s.k0, Lq = s.q1 - s.q0, Lk = s.k1 - s.k0;
  const bool inv = (s.t == FFA_INV_CAUSAL) | (s.t == FFA_BI_CAUSAL);
  const bool cau = (s.t == FFA_CAUSAL) | (s.t == FFA_BI_CAUSAL);
  int l = cau ? max(0, c - (Lk - Lq)) : 0;
  int h = inv ? min(Lq - 1, c) : Lq - 1;
  if (j < s.k0 || j >= s.k1) { l = 1; h = 0; }
  lo = s.q0 + l;
  hi = s.q0 + h;
}

// bits [a, b] of a 64-bit word (0 <= a <= b <= 63)
__device__ __forceinline__ uint64_t bit_range(int a, int b) {
  return (~0ull >> (63 - (b - a))) << a;
}

// x where bit b of w is set, else -inf: the one-bit field sign-extended
// (v_bfe_i32) selects between the two bit patterns in one three-input bitwise
// operation, with no condition register and so no wait states after it
__device__ __forceinline__ float keep_or_neg_inf(float x, uint32_t w, int b) {
  const uint32_t m = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(w), b, 1));
  return __uint_as_float((__float_as_uint(x) & m) | (~m & 0xff800000u));
}

// bits [a, b] of a 32-bit word (0 <= a <= b <= 31)
__device__ __forceinline__ uint32_t bit_range32(int a, int b) {
  return (~0u >> (31 - (b - a))) << a;
}

// ---------------------------------------------------------------------------
// MFMA and register types.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// D = A(32x16) * B(16x32) + C, fp32 accumulate.  Lane l holds A[l%32][8*(l/32)+e],
// B[8*(l/32)+e][l%32] (e = 0..7) and C[8*(r/4) + 4*(l/32) + r%4][l%32] in register r.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS tiles of [ROWS][D] bf16 are stored as D/32 column groups, each a
// [ROWS][64 B] block of four 16-byte chunks per row.  Chunk q of row r sits at
// chunk position q ^ ((r >> 2) & 3) of its row.  This keeps the two read
// patterns conflict-free: 16 consecutive rows reading one chunk (128-bit
// operand reads: the rows fall on 4 different 256-byte bank lines, the swizzle
// spreads each line over 4 chunk positions) and 4 consecutive rows x 64 bytes
// (transposed 64-bit reads: 256 contiguous bytes).  The swizzle depends only
// on bits 2..3 of the row, so moving by a multiple of 16 rows or by whole
// column groups is a constant byte offset, and every operand address is one of
// two per-lane bases plus an immediate.
// ---------------------------------------------------------------------------
template <int ROWS>
constexpr int group_bytes() { return ROWS * 64; }

// byte offset of chunk q (0..3) of row r inside a column group
__device__ __forceinline__ int lds_pos(int r, int q) {
  return r * 64 + (((q ^ (r >> 2)) & 3) << 4);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + num_bytes): loads past the end return 0.
// All fields are wave-uniform and kept in scalar registers.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffffu));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)num_bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 (or 4) bytes per lane from global straight into LDS: lane l writes
// lds_base + 16*l (4*l); the global address is base + voff + soff, soff being
// wave-uniform.  Issued as inline assembly so that the compiler does not make
// later LDS reads of the *other* buffer wait for these loads; the caller
// waits explicitly (wait_dma) before the barrier that publishes them.  m0 is
// a register the compiler reserves and would not honour as a clobber; no
// generated code of these kernels keeps a value in m0 across the statements.
// LDS byte address of a __shared__ array (taken from the array itself, so
// the compiler needs no null check of a generic pointer)
__device__ __forceinline__ uint32_t lds_addr(const char* shared_array) {
  return (uint32_t)(size_t)((const __attribute__((address_space(3))) char*)shared_array);
}
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(voff), "s"(r), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma4(const i32x4& r, uint32_t lds, uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voff), "s"(r) : "memory");
}
// all of this wave's global->LDS loads have landed
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// all but the N most recently issued of this wave's global->LDS loads have landed
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Loads a [ROWS][D] bf16 tile whose rows are ts elements apart in global
// memory into the column-group LDS layout with 16-byte direct loads, using
// ROWS / 16 waves.  One load fills 1024 contiguous LDS bytes = 16 rows of one
// column group: lane l takes row l / 4 of the 16 and chunk position l % 4,
// i.e. logical chunk (l % 4) ^ ((l >> 4) & 3).  Wave w fills rows
// 16w..16w+15 of every column group, so one per-lane offset serves all of its
// loads and the column group goes into the scalar offset.  Rows at or past
// valid_rows lie at or past the end of the buffer range whatever the scalar
// offset (< 2D bytes < one row), so they read as zero.
template <int D, int ROWS>
struct TileDma {
  static_assert(ROWS % 16 == 0 && D % 32 == 0, "tile shape");
  static constexpr int NG = D / 32;           // column groups
  uint32_t voff;
  int w;
  __device__ __forceinline__ void init(int wid, int lane, int64_t ts_elems) {
    w = wid;
    const int r = 16 * wid + (lane >> 2);
    const int q = (lane & 3) ^ ((lane >> 4) & 3);
    voff = (uint32_t)(r * ts_elems * 2 + q * 16);
  }
  // rows [row_base, row_base + ROWS) of a tensor (base pointer of row 0 of the
  // head), valid_rows of them in bounds
  __device__ __forceinline__ void load(const __bf16* head_base, int64_t ts_elems, int row_base,
                                       int valid_rows, uint32_t lds_tile) const {
    const __bf16* b = head_base + (int64_t)row_base * ts_elems;
    const int vr = valid_rows < 0 ? 0 : (valid_rows > ROWS ? ROWS : valid_rows);
    const i32x4 r = make_rsrc(b, (uint32_t)(vr * ts_elems * 2));
#pragma unroll
    for (int g = 0; g < NG; ++g)
      dma16(r, lds_tile + g * group_bytes<ROWS>() + 16 * w * 64, voff, 64u * g);
  }
};

// Work items are (schedule position, head) pairs, nitems * Hq blocks in all
// (Hq = Hkv for the key-major kernel).  Blocks are dispatched round-robin
// over the 8 XCDs (block b on XCD b % 8), each with its own L2.  When Hkv is a
// multiple of 8, XCD x is given the kv heads x, x + 8, x + 16, ... and works
// through them one after the other; for each it takes the items in schedule
// order (heaviest first), head-minor: consecutive blocks on one XCD are the
// query heads of one item, which share key/value (or query) tiles through
// that XCD's L2, and one kv head's working set at a time stays in it.  Taking
// every eighth kv head (not a contiguous range) spreads kv-head groups with
// different masks over all XCDs.
__device__ __forceinline__ void xcd_map(int bid, int nitems, int Hq, int Hkv, int& item, int& head) {
  if (Hkv % 8 == 0) {
    const int G = Hq / Hkv, per_kv = nitems * G, x = bid & 7, j = bid >> 3;
    const int r = j % per_kv;
    item = r / G;
    head = (x + 8 * (j / per_kv)) * G + r % G;
  } else {
    item = bid / Hq;
    head = bid % Hq;
  }
}

__device__ __forceinline__ float wave_swap_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

__device__ __forceinline__ float wave_swap_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Host-side launchers (one per source file).
hipError_t launch_build_meta(const int32_t* d_slices, int32_t S, int32_t Tq, int32_t Tk,
                             int32_t head_dim, void* d_meta, int64_t capacity,
                             const MetaLayout& L, hipStream_t stream);

// Metadata per kv-head group: kv heads [kv_end[g-1], kv_end[g]) use meta[g].
struct MaskGroups {
  const void* meta[FFA_MAX_MASK_GROUPS];
  int32_t kv_end[FFA_MAX_MASK_GROUPS];
  int32_t n;
};

// The metadata of kv head kvh (a chain of selects: no indexing into the
// kernel-argument array).
__device__ __forceinline__ const void* group_meta(const MaskGroups& g, int kvh) {
  const void* m = g.meta[0];
#pragma unroll
  for (int j = 1; j < FFA_MAX_MASK_GROUPS; ++j)
    if (j < g.n && kvh >= g.kv_end[j - 1]) m = g.meta[j];
  return m;
}

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  MaskGroups groups;
  int64_t q_ts, q_hs, k_ts, k_hs, v_ts, v_hs, o_ts, o_hs;
  int32_t Tq, Tk, Hq, Hkv;
  int32_t nitems;     // query blocks (the grid is nitems * Hq)
  int64_t rec_off;    // byte offset of the forward block records in metadata of these lengths
  float scale_log2;   // softmax_scale * log2(e)
  float scale;
  uint32_t flags;     // FFA_ACCUMULATE: merge into the (o, lse) already in the buffers
};
hipError_t launch_fwd(const FwdArgs& a, int head_dim, int nq_f, hipStream_t stream);

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  float* dvec;        // workspace: -D_i = -dO_i . O_i, [Hq][Tq]
  float* lvec;        // workspace: LSE_i * log2(e) (0 where LSE = -inf), [Hq][Tq]
  float* mvec;        // workspace: -LSE_i / scale (0 where LSE = -inf), [Hq][Tq]
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  MaskGroups groups;
  int64_t q_ts, q_hs, k_ts, k_hs, v_ts, v_hs, o_ts, o_hs, do_ts, do_hs;
  int64_t dq_ts, dq_hs, dk_ts, dk_hs, dv_ts, dv_hs;
  int32_t Tq, Tk, Hq, Hkv;
  int32_t nq_f, nk_b; // query blocks of the dQ grid, key blocks of the dK/dV grid
  int64_t rec_off_f, rec_off_b;   // byte offsets of the block records in metadata of these lengths
  float scale_log2;
  float scale;
  uint32_t flags;     // FFA_ACCUMULATE: add to the dq / dk / dv already in the buffers
  // Split key blocks (dK / dV load balance): the split_e longest key blocks of
  // each kv head may be done as two halves of their query-tile walk by two
  // workgroups; the second to finish adds the other's fp32 partial.
  int32_t* split_cnt;   // workspace: [split_e][Hkv] finish counters, zero between launches
  float* split_part;    // workspace: [split_e][Hkv][2 halves][dK, dV][BN_B * D] fp32
  int32_t split_e;      // candidate blocks per kv head (<= nk_b)
  int32_t split_slots;  // dK/dV workgroups resident on the device at once
};

// Number of split candidates per kv head: enough for the long blocks of a
// causal varlen batch on one XCD, bounded so the partial buffers stay about
// 32 MB for d = 128 whatever Hkv is.
__host__ __device__ inline int32_t split_candidates(int32_t Hkv, int32_t nk_b) {
  int32_t e = Hkv > 0 ? 128 / Hkv : 0;
  e = e < 4 ? 4 : (e > 32 ? 32 : e);
  return e < nk_b ? e : nk_b;
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, int nq_f, int nk_b, int phases,
                      hipStream_t stream);
// counters_clear: the split counters were already zeroed in this stream (by
// the dQ kernel that computes the row statistics); otherwise a small kernel
// clears them first.
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int nk_b, bool counters_clear,
                           hipStream_t stream);

}  // namespace ffa
