// ffa_bwd.hip - Flex-Flash-Attention backward on gfx950.
//
// The pages say FFA has a backward and that its partial results are merged
// (blog deep-dive, section "Flex-Flash-Attention 与 AttnSlice", Fig. 5: slice
// level parallelism with atomic reduction of partials).  This backward is the
// textbook gradient of masked softmax attention written so that every output
// element has one owner and a fixed summation order, hence bitwise
// reproducible results without atomic accumulation (the two halves of a split
// dK/dV block meet through a counter and add their fp32 partials once):
//
//   bwd_pre : -D_i = -dO_i . O_i, LSE_i log2 e          (fp32, [Hq][Tq])
//   dkdv    : owner (kv head, 128-key block), in ffa_bwd_dkdv.hip
//   dq      : owner (query head, 128-row block); loops over its q2k tiles:
//             S^T, P^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T
//
// dq mirrors the forward (lanes own query rows).  This file also holds the
// backward's launcher.
#include <type_traits>

#include "ffa_internal.hpp"

namespace ffa {

namespace {

constexpr int NT = 256;

// -D_i = -sum_c dO_ic O_ic (stored negated: it seeds the dP accumulators) and
// LSE_i log2 e, one group of D/8 lanes per (token, head)
template <int D>
__global__ __launch_bounds__(NT) void ffa_bwd_pre_kernel(BwdArgs a) {
  constexpr int G = D / 8;
  const int64_t rh = ((int64_t)blockIdx.x * NT + threadIdx.x) / G;
  const int part = threadIdx.x % G;
  const bool ok = rh < (int64_t)a.Tq * a.Hq;
  float acc = 0.f;
  int i = 0, h = 0;
  if (ok) {
    i = (int)(rh / a.Hq);
    h = (int)(rh % a.Hq);
    const u32x4 o = *reinterpret_cast<const u32x4*>(a.o + (int64_t)i * a.o_ts + (int64_t)h * a.o_hs + 8 * part);
    const u32x4 g = *reinterpret_cast<const u32x4*>(a.dout + (int64_t)i * a.do_ts + (int64_t)h * a.do_hs + 8 * part);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ou = o[e], gu = g[e];
      acc += __uint_as_float(ou << 16) * __uint_as_float(gu << 16);
      acc += __uint_as_float(ou & 0xffff0000u) * __uint_as_float(gu & 0xffff0000u);
    }
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, G);
  if (ok && part == 0) {
    a.dvec[(int64_t)h * a.Tq + i] = -acc;
    const float l = a.lse[(int64_t)h * a.Tq + i];
    a.lvec[(int64_t)h * a.Tq + i] = (l == -INFINITY) ? 0.f : l * LOG2E;
    a.mvec[(int64_t)h * a.Tq + i] = (l == -INFINITY) ? 0.f : -l / a.scale;
  }
}

// ---------------------------------------------------------------------------
// dQ: owner (query head, BM_F-row block), 4 waves x 32 rows, q2k tiles.
//
// Mirror of the forward: S^T = K Q^T and dP^T = V dO^T with one query row per
// lane, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T with K^T from transposed LDS
// reads.  Each 64-key list tile streams as two 32-key stages through a
// double-buffered LDS ring (32 KB); the last DQ_NQL 16-wide d steps of the Q
// operand are parked in LDS (16 bytes per lane each, read once per stage) so
// that the kernel stays within the registers of three waves per SIMD.
// ---------------------------------------------------------------------------
constexpr int DQ_SK = 32;                       // keys per stage

template <int D>
constexpr int dq_nql() { return D == 128 ? 5 : 0; }

template <int D>
constexpr size_t dq_lds_bytes() {
  return 2 * 2 * DQ_SK * D * 2 + (size_t)(NT / 64) * dq_nql<D>() * 1024;
}

// S^T = K Q^T and dP^T - D = V dO^T - D of one 32-key stage at head_dim 128
// (the first three 16-wide d steps of Q in registers, the last five parked in
// LDS), as one block with a ring of three 128-bit operand buffers: each
// MFMA's LDS operand is read two to three reads ahead of its use instead of
// just before it (the compiler's own schedule, register-bound at three waves
// per SIMD).  The dP^T accumulator sits in fixed registers, v140-v155, so that
// the block can seed all 16 with -D (eight 64-bit moves of the (-D, -D) pair,
// seven instructions before the first dP MFMA reads them); dS = P (dP - D)
// then needs one multiply.  The S MFMAs are the plain loop's, in its order.
// The buffers and accumulators are early-clobber outputs, so the compiler
// keeps nothing else in them; the block waits for its own LDS reads (a wait
// for at most N outstanding also covers any older LDS or scalar loads) and
// ends with 16 wait states, more than an 8-pass MFMA result needs before a
// VALU instruction may read it.
#define FFA_RD(buf, addr, off) "ds_read_b128 " buf ", " addr " offset:" #off "\n\t"
#define FFA_MF(d, a, b, c) "v_mfma_f32_32x32x16_bf16 " d ", " a ", " b ", " c "\n\t"
#define FFA_WT(n) "s_waitcnt lgkmcnt(" #n ")\n\t"
// operands: %0 S, %1 dP (v140-v155), %2-%4 buffers, %5-%7 Q chunks 0-2,
// %8-%15 dO chunks 0-7, %16 / %17 K/V read address of column pair 0 / 1, %18
// parked Q chunks 3-7, %19 the (-D, -D) pair
#define FFA_SDP_BLOCK(K0, K1, K2, K3, V0, V1, V2, V3) \
  "v_mov_b64 v[140:141], %19\n\tv_mov_b64 v[142:143], %19\n\tv_mov_b64 v[144:145], %19\n\t" \
  "v_mov_b64 v[146:147], %19\n\tv_mov_b64 v[148:149], %19\n\tv_mov_b64 v[150:151], %19\n\t" \
  "v_mov_b64 v[152:153], %19\n\tv_mov_b64 v[154:155], %19\n\t" \
  FFA_RD("%2", "%16", K0) FFA_RD("%3", "%16", V0) FFA_RD("%4", "%17", K0) \
  FFA_WT(2) FFA_MF("%0", "%2", "%5", "0") FFA_RD("%2", "%17", V0) \
  FFA_WT(2) FFA_MF("%1", "%3", "%8", "%1") FFA_RD("%3", "%16", K1) \
  FFA_WT(2) FFA_MF("%0", "%4", "%6", "%0") FFA_RD("%4", "%16", V1) \
  FFA_WT(2) FFA_MF("%1", "%2", "%9", "%1") FFA_RD("%2", "%17", K1) \
  FFA_WT(2) FFA_MF("%0", "%3", "%7", "%0") FFA_RD("%3", "%18", 0) \
  FFA_WT(2) FFA_MF("%1", "%4", "%10", "%1") FFA_RD("%4", "%17", V1) \
  FFA_WT(1) FFA_MF("%0", "%2", "%3", "%0") FFA_RD("%2", "%16", K2) FFA_RD("%3", "%18", 1024) \
  FFA_WT(2) FFA_MF("%1", "%4", "%11", "%1") FFA_RD("%4", "%16", V2) \
  FFA_WT(1) FFA_MF("%0", "%2", "%3", "%0") FFA_RD("%2", "%17", K2) FFA_RD("%3", "%18", 2048) \
  FFA_WT(2) FFA_MF("%1", "%4", "%12", "%1") FFA_RD("%4", "%17", V2) \
  FFA_WT(1) FFA_MF("%0", "%2", "%3", "%0") FFA_RD("%2", "%16", K3) FFA_RD("%3", "%18", 3072) \
  FFA_WT(2) FFA_MF("%1", "%4", "%13", "%1") FFA_RD("%4", "%16", V3) \
  FFA_WT(1) FFA_MF("%0", "%2", "%3", "%0") FFA_RD("%2", "%17", K3) FFA_RD("%3", "%18", 4096) \
  FFA_WT(2) FFA_MF("%1", "%4", "%14", "%1") FFA_RD("%4", "%17", V3) \
  FFA_WT(1) FFA_MF("%0", "%2", "%3", "%0") \
  FFA_WT(0) FFA_MF("%1", "%4", "%15", "%1") \
  "s_nop 7\n\ts_nop 7"

template <int STAGE>
__device__ __forceinline__ void sdp_d128(f32x16& sacc, f32x16& pacc, const bf16x8 (&q)[8],
                                         const bf16x8 (&g)[8], uint32_t k0, uint32_t k1,
                                         uint32_t qp, uint64_t nd2) {
  u32x4 b0, b1, b2;
#define FFA_SDP_OPS                                                                         \
  : "=&v"(sacc), "=&{v[140:155]}"(pacc), "=&v"(b0), "=&v"(b1), "=&v"(b2)                   \
  : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(g[0]), "v"(g[1]), "v"(g[2]), "v"(g[3]), \
    "v"(g[4]), "v"(g[5]), "v"(g[6]), "v"(g[7]), "v"(k0), "v"(k1), "v"(qp), "v"(nd2)      \
  : "memory"
  if constexpr (STAGE == 0)
    asm volatile(FFA_SDP_BLOCK(0, 2048, 4096, 6144, 8192, 10240, 12288, 14336) FFA_SDP_OPS);
  else
    asm volatile(FFA_SDP_BLOCK(16384, 18432, 20480, 22528, 24576, 26624, 28672, 30720) FFA_SDP_OPS);
#undef FFA_SDP_OPS
}

// dQ^T += K^T dS^T of one 32-key stage at head_dim 128: 8 MFMAs (16-key
// chunk c, column block mb) whose A operands are pairs of transposed 64-bit
// LDS reads, through a ring of three 4-register operand buffers in fixed
// registers, v156-v167 (an operand's two 64-bit halves cannot be named
// separately in inline assembly).  Same MFMAs in the same order as the plain
// loop (bitwise identical sums); the same waits and refill rule as the S / dP
// block above.  The first MFMA follows LDS instructions enough for the wait
// states a VALU write of its B operand needs.
#define FFA_OTR(lo, hi, off) \
  "ds_read_b64_tr_b16 v[" lo "], %6 offset:(%8+" #off ")\n\t" \
  "ds_read_b64_tr_b16 v[" hi "], %7 offset:(%8+" #off ")\n\t"
#define FFA_M(acc, buf, bop) "v_mfma_f32_32x32x16_bf16 " acc ", " buf ", " bop ", " acc "\n\t"
#define FFA_W(n) "s_waitcnt lgkmcnt(" #n ")\n\t"
// operands: %0-%3 dQ^T column blocks, %4 / %5 dS^T of chunk 0 / 1, %6 / %7
// transposed-read addresses of keys 0-7 / 8-15 of a chunk, %8 LDS offset of
// the stage's K tile.  Read offsets 2048 mb + 1024 c.
#define FFA_DQ_BLOCK \
  FFA_OTR("156:157", "158:159", 0) FFA_OTR("160:161", "162:163", 2048) \
  FFA_OTR("164:165", "166:167", 4096) \
  FFA_W(4) FFA_M("%0", "v[156:159]", "%4") FFA_OTR("156:157", "158:159", 6144) \
  FFA_W(4) FFA_M("%1", "v[160:163]", "%4") FFA_OTR("160:161", "162:163", 1024) \
  FFA_W(4) FFA_M("%2", "v[164:167]", "%4") FFA_OTR("164:165", "166:167", 3072) \
  FFA_W(4) FFA_M("%3", "v[156:159]", "%4") FFA_OTR("156:157", "158:159", 5120) \
  FFA_W(4) FFA_M("%0", "v[160:163]", "%5") FFA_OTR("160:161", "162:163", 7168) \
  FFA_W(4) FFA_M("%1", "v[164:167]", "%5") \
  FFA_W(2) FFA_M("%2", "v[156:159]", "%5") \
  FFA_W(0) FFA_M("%3", "v[160:163]", "%5")

template <int BASE>
__device__ __forceinline__ void dq_d128(f32x16 (&o)[4], const bf16x8& p0, const bf16x8& p1, int t0,
                                        int t1) {
  asm volatile(FFA_DQ_BLOCK
               : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3])
               : "v"(p0), "v"(p1), "v"(t0), "v"(t1), "i"(BASE)
               : "v156", "v157", "v158", "v159", "v160", "v161", "v162", "v163", "v164", "v165",
                 "v166", "v167", "memory");
}

// PRE: also compute this block's -D and LSE log2 e rows (the bwd_pre work)
// from the dO operand already in registers and O, use them, and store them
// for the dK/dV kernel, which then runs after this one.
template <int D, bool PRE>
__global__ __launch_bounds__(NT, 3) __attribute__((amdgpu_waves_per_eu(3, 3))) void ffa_bwd_dq_kernel(BwdArgs a) {
  // statically sized: a known LDS address lets operand reads use immediates
  __shared__ __attribute__((aligned(16))) char smem[dq_lds_bytes<D>()];
  constexpr int SK = DQ_SK;
  constexpr int TILE_B = SK * D * 2;            // one K or V stage tile
  constexpr int STAGE_B = 2 * TILE_B;
  constexpr int MB = D / 32;
  constexpr int KS = D / 16;
  constexpr int HALVES = BN_F / SK;
  constexpr int NQL = dq_nql<D>();
  constexpr int QREG = KS - NQL;
  constexpr int GB = group_bytes<SK>();
  static_assert(2 * SK == 16 * (NT / 64), "K and V stage tiles are loaded by half of the waves each");
  static_assert(SK == 32, "a Partial stage's key mask is one 32-bit word");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5, t16 = lane & 15, g16 = lane >> 4;
  if constexpr (PRE) {
    // the dK/dV kernel that follows in this stream expects its split
    // counters at zero
    if (blockIdx.x == 0)
      for (int i = tid; i < a.split_e * a.Hkv; i += NT) a.split_cnt[i] = 0;
  }
  int item, head;
  xcd_map(blockIdx.x, a.nq_f, a.Hq, a.Hkv, item, head);
  const int kvh = head / (a.Hq / a.Hkv);
  const MetaView mv = meta_view(group_meta(a.groups, kvh));
  const FFA_CONST MetaHeader* hd = mv.hdr;
  if (!meta_usable(hd, a.Tq, a.Tk, A_REC_F, a.rec_off_f)) return;
  // the item's block record (one read), as in the forward
  cint32_t* rec = (cint32_t*)((const FFA_CONST char*)hd + a.rec_off_f) + REC * item;
  const int m = rec[R_OWNER];
  const int qrow = m * BM_F + wid * 32 + l32;
  const bool qok = qrow < a.Tq;

  const int f0 = rec[R_F0], nF = rec[R_NF];
  const int p0 = rec[R_P0], nP = rec[R_NP];
  const int nU = HALVES * (nP + nF);            // stages
  cint32_t* fidx = mv.var + hd->list_off[L_QF] + f0;
  cint32_t* pidx = mv.var + hd->list_off[L_QM] + p0;
  const int s0 = rec[R_S0], nS = rec[R_NS];
  cint32_t* sidx = mv.var + hd->list_off[L_QS] + s0;
  const int tile0 = nP > 0 ? rec[R_TP] : rec[R_TF];   // Partial tiles come first

  bf16x8 qop[KS], gop[KS];
  {
    const __bf16* qp = a.q + (int64_t)qrow * a.q_ts + (int64_t)head * a.q_hs + 8 * h32;
    const __bf16* gp = a.dout + (int64_t)qrow * a.do_ts + (int64_t)head * a.do_hs + 8 * h32;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u32x4 u = qok ? *reinterpret_cast<const u32x4*>(qp + 16 * k) : u32x4{0, 0, 0, 0};
      u32x4 w = qok ? *reinterpret_cast<const u32x4*>(gp + 16 * k) : u32x4{0, 0, 0, 0};
      __builtin_memcpy(&qop[k], &u, 16);
      __builtin_memcpy(&gop[k], &w, 16);
    }
  }
  float l2 = 0.f, ndval = 0.f;                   // LSE log2(e) and -D of this row
  if constexpr (PRE) {
    // lanes l32 and l32 + 32 hold the two halves of the row's d
    float part = 0.f;
    if (qok) {
      const __bf16* op = a.o + (int64_t)qrow * a.o_ts + (int64_t)head * a.o_hs + 8 * h32;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const u32x4 ou = *reinterpret_cast<const u32x4*>(op + 16 * k);
        u32x4 gu;
        __builtin_memcpy(&gu, &gop[k], 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part += __uint_as_float(ou[e] << 16) * __uint_as_float(gu[e] << 16);
          part += __uint_as_float(ou[e] & 0xffff0000u) * __uint_as_float(gu[e] & 0xffff0000u);
        }
      }
    }
    ndval = -wave_swap_sum(part);
    if (qok) {
      const float l = a.lse[(int64_t)head * a.Tq + qrow];
      l2 = (l == -INFINITY) ? 0.f : l * LOG2E;
      if (h32 == 0) {
        a.dvec[(int64_t)head * a.Tq + qrow] = ndval;
        a.lvec[(int64_t)head * a.Tq + qrow] = l2;
        a.mvec[(int64_t)head * a.Tq + qrow] = (l == -INFINITY) ? 0.f : -l / a.scale;
      }
    }
  } else {
    if (qok) {
      l2 = a.lvec[(int64_t)head * a.Tq + qrow];
      ndval = a.dvec[(int64_t)head * a.Tq + qrow];
    }
  }
  wait_vmem();
  // (-D, -D) as one 64-bit operand: the dP^T accumulator's seed
  const uint64_t nd2 = ((uint64_t)__float_as_uint(ndval) << 32) | __float_as_uint(ndval);
  char* qlds = smem + 2 * STAGE_B + wid * (NQL * 1024) + lane * 16;
#pragma unroll
  for (int k = QREG; k < KS; ++k) {
    u32x4 u;
    __builtin_memcpy(&u, &qop[k], 16);
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
        (__attribute__((address_space(3))) char*)qlds + (k - QREG) * 1024) = u;
  }

  int raddr[2], taddr[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) raddr[p] = lds_pos(l32, 2 * p + h32);
  // LDS byte addresses of this lane's 128-bit K / V operand reads (column
  // pair 0 and 1) and of its parked Q chunks, for the S / dP block below
  const uint32_t smem_base = (uint32_t)(size_t)((__attribute__((address_space(3))) char*)smem);
  const uint32_t kbase0 = smem_base + raddr[0], kbase1 = smem_base + raddr[1];
  const uint32_t qbase = (uint32_t)(size_t)((__attribute__((address_space(3))) char*)qlds);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    taddr[j] = lds_pos(4 * h32 + (t16 >> 2) + 8 * j, 2 * (g16 & 1) + ((t16 >> 1) & 1)) + 8 * (t16 & 1);
  // LDS byte addresses of the transposed K reads for the dQ block at d = 128
  const int tb0 = (int)(smem_base + taddr[0]), tb1 = (int)(smem_base + taddr[1]);

  // waves 0-1 load the K stage tile, waves 2-3 the V stage tile
  TileDma<D, SK> dm;
  dm.init(wid & 1, lane, wid < 2 ? a.k_ts : a.v_ts);
  const __bf16* kbase = a.k + (int64_t)kvh * a.k_hs;
  const __bf16* vbase = a.v + (int64_t)kvh * a.v_hs;
  auto tile_of = [&](int t) { return t < nP ? pidx[t] : fidx[t - nP]; };
  auto issue_tile = [&](int tile, int half, int stage) {
    const int key0 = tile * BN_F + half * SK;
    const uint32_t st = lds_addr(smem) + stage * STAGE_B;
    if (wid < 2) dm.load(kbase, a.k_ts, key0, a.Tk - key0, st);
    else dm.load(vbase, a.v_ts, key0, a.Tk - key0, st + TILE_B);
  };
  auto issue = [&](int u, int stage) { issue_tile(tile_of(u / HALVES), u % HALVES, stage); };

  f32x16 dqacc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) dqacc[i] = f32x16{};
  const float c = a.scale_log2;

  auto stage_fn = [&](auto stage_c, int u) {
    constexpr int stage = decltype(stage_c)::value;
    const int t = u / HALVES;
    const bool masked = t < nP;
    const int key0 = tile_of(t) * BN_F + (u % HALVES) * SK;
    if (u + 1 < nU) issue(u + 1, stage ^ 1);
    const __attribute__((address_space(3))) char* lb =
        (const __attribute__((address_space(3))) char*)smem + stage * STAGE_B;

    // Partial tile: valid keys of this lane's row inside [key0, key0 + SK), one
    // bit per key.  A stage with no valid pair for any of the wave's rows is
    // skipped: it would add nothing.
    uint32_t w = ~0u;
    bool live = true, need_mask = false;
    if (masked) {
      uint32_t mk = 0;   // bit j: key key0 + j (SK = 32)
      for (int si = 0; si < nS; ++si) {
        const Slice sl = load_slice(mv.slices, sidx[si]);
        int lo, hi;
        row_interval(sl, qrow, lo, hi);
        lo = max(lo, key0);
        hi = min(hi, key0 + SK - 1);
        if (lo <= hi) mk |= bit_range32(lo - key0, hi - key0);
      }
      live = __ballot(mk != 0) != 0;
      // a stage valid for every key and row of this wave needs no masking
      need_mask = __ballot(mk != ~0u) != 0;
      w = mk >> (4 * h32);   // register r holds key 8(r/4) + 4*h32 + r%4
    }

    if (live) {
      // S^T = K Q^T and dP^T = V dO^T; lane = query row, registers = keys 8(r/4) + 4*h32 + r%4
      f32x16 sacc, pacc;
      if constexpr (D == 128 && NQL == 5) {
        sdp_d128<stage>(sacc, pacc, qop, gop, kbase0, kbase1, qbase, nd2);
      } else {
        sacc = f32x16{};
        pacc = f32x16{};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          bf16x8 ka, va, qv;
          u32x4 u1 = *(const __attribute__((address_space(3))) u32x4*)(lb + (k >> 1) * GB + raddr[k & 1]);
          u32x4 u2 = *(const __attribute__((address_space(3))) u32x4*)(lb + TILE_B + (k >> 1) * GB + raddr[k & 1]);
          __builtin_memcpy(&ka, &u1, 16);
          __builtin_memcpy(&va, &u2, 16);
          if (k < QREG) {
            qv = qop[k];
          } else {
            u32x4 uq = *(const __attribute__((address_space(3))) u32x4*)(
                (const __attribute__((address_space(3))) char*)qlds + (k - QREG) * 1024);
            __builtin_memcpy(&qv, &uq, 16);
          }
          sacc = mfma32(ka, qv, sacc);
          pacc = mfma32(va, gop[k], pacc);
        }
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[r] = keep_or_neg_inf(sacc[r], w, 8 * (r >> 2) + (r & 3));
      }

#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -l2));
        if constexpr (D == 128 && NQL == 5) pacc[r] *= pv;   // the block seeded it with -D
        else pacc[r] = pv * (pacc[r] + ndval);
      }

      // dQ^T += K^T dS^T over the stage's two 16-key chunks
      if constexpr (D == 128) {
        static_assert(GB == 2048 && MB == 4 && SK == 32, "offsets of the d = 128 block");
        static_assert(STAGE_B + 3 * GB + 1024 < 65536, "LDS read offsets of the d = 128 block");
        bf16x8 sb[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int e = 0; e < 8; ++e) sb[c2][e] = static_cast<__bf16>(pacc[8 * c2 + e]);
        dq_d128<stage * STAGE_B>(dqacc, sb[0], sb[1], tb0, tb1);
      } else
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) sb[e] = static_cast<__bf16>(pacc[8 * c2 + e]);
        const int roff = 16 * c2 * 64;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const i16x4 k0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lb + mb * GB + taddr[0] + roff));
          const i16x4 k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lb + mb * GB + taddr[1] + roff));
          const i16x8 kk = __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7);
          bf16x8 ka;
          __builtin_memcpy(&ka, &kk, 16);
          dqacc[mb] = mfma32(ka, sb, dqacc[mb]);
        }
      }
    }
    wait_dma();
    __syncthreads();
  };

  if (nU > 0) issue_tile(tile0, 0, 0);
  wait_dma();
  __syncthreads();
  for (int u = 0; u < nU; u += 2) {
    stage_fn(std::integral_constant<int, 0>{}, u);
    if (u + 1 < nU) stage_fn(std::integral_constant<int, 1>{}, u + 1);
  }

  // the last MFMAs of the inline block wrote dQ^T; give them the wait states
  // a VALU or memory read of an MFMA result needs
  if constexpr (D == 128)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+v"(dqacc[0]), "+v"(dqacc[1]), "+v"(dqacc[2]), "+v"(dqacc[3]));

  if ((a.flags & FFA_ACCUMULATE) == 0) {
    // Plain store, staged through the idle tile ring so that each global
    // store writes whole rows (as in the forward): wave wid stages its 32 rows
    // at wid * 32 * RB, 16-byte chunk c of row r at chunk position c ^ (r % CPR).
    constexpr int RB = D * 2, CPR = D / 8, RPI = 64 / CPR;
    // the lane index is made opaque here so that the staging addresses are
    // not computed before the stage loop and kept in registers through it
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lr = ln & 31, lh = ln >> 5;
    __attribute__((address_space(3))) char* wl = (__attribute__((address_space(3))) char*)smem + wid * 32 * RB;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = static_cast<__bf16>(dqacc[mb][4 * j + i] * a.scale);
        const int c = 4 * mb + j;
        *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(
            wl + lr * RB + ((c ^ (lr % CPR)) * 16) + 8 * lh) = w;
      }
    const int rsub = ln / CPR, ck = ln % CPR;
#pragma unroll
    for (int s = 0; s < 32 / RPI; ++s) {
      const int r = RPI * s + rsub;
      const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          wl + r * RB + ((ck ^ (r % CPR)) * 16));
      const int grow = m * BM_F + wid * 32 + r;
      if (grow < a.Tq)
        *reinterpret_cast<u32x4*>(a.dq + (int64_t)grow * a.dq_ts + (int64_t)head * a.dq_hs + 8 * ck) = v;
    }
    return;
  }
  if (qok) {
    // FFA_ACCUMULATE: add to what dq holds (fp32 sum, one rounding)
    __bf16* qp = a.dq + (int64_t)qrow * a.dq_ts + (int64_t)head * a.dq_hs;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4* dst = reinterpret_cast<bf16x4*>(qp + 32 * mb + 8 * j + 4 * h32);
        const bf16x4 old = *dst;
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = static_cast<__bf16>(dqacc[mb][4 * j + i] * a.scale + static_cast<float>(old[i]));
        *dst = w;
      }
  }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int head_dim, int nq_f, int nk_b, int phases,
                      hipStream_t stream) {
  const int64_t rows = (int64_t)a.Tq * a.Hq;
  const int64_t gq = (int64_t)nq_f * a.Hq;
  // PRE together with DQ: the dQ kernel computes the row statistics itself and
  // runs first; otherwise PRE is its own kernel.
  const bool fused = (phases & FFA_BWD_PRE) && (phases & FFA_BWD_DQ) && gq > 0;
  if (fused) {
    if (head_dim == 128)
      ffa_bwd_dq_kernel<128, true><<<dim3((unsigned)gq), NT, 0, stream>>>(a);
    else
      ffa_bwd_dq_kernel<64, true><<<dim3((unsigned)gq), NT, 0, stream>>>(a);
  } else if ((phases & FFA_BWD_PRE) && rows > 0) {
    const int G = head_dim / 8;
    const int64_t blocks = (rows * G + NT - 1) / NT;
    if (head_dim == 128) ffa_bwd_pre_kernel<128><<<dim3((unsigned)blocks), NT, 0, stream>>>(a);
    else ffa_bwd_pre_kernel<64><<<dim3((unsigned)blocks), NT, 0, stream>>>(a);
  }
  if ((phases & FFA_BWD_DKDV) && nk_b > 0 && a.Hkv > 0) {
    const hipError_t e = launch_bwd_dkdv(a, head_dim, nk_b, fused, stream);
    if (e != hipSuccess) return e;
  }
  if (!fused && (phases & FFA_BWD_DQ) && gq > 0) {
    if (head_dim == 128)
      ffa_bwd_dq_kernel<128, false><<<dim3((unsigned)gq), NT, 0, stream>>>(a);
    else
      ffa_bwd_dq_kernel<64, false><<<dim3((unsigned)gq), NT, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ffa
