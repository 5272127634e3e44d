// ffa_bwd_dkdv.hip - dK and dV of Flex-Flash-Attention on gfx950.
//
// The backward of the MagiAttention pages' FFA kernel (blog deep-dive, section
// "Flex-Flash-Attention 与 AttnSlice", Fig. 5), written with one owner per
// output: owner (kv head, 128-key block), which loops over the query heads
// that share the kv head and the k2q tiles of the block in a fixed order, so
// dK and dV are bitwise reproducible; the few longest blocks are done as two
// halves whose fp32 sums are added once (the split epilogue below):
//   S = Q K^T, P = exp(S - LSE) (masked on Partial tiles), dV += P^T dO,
//   dP = dO V^T, dS = P (dP - D), dK += dS^T Q.
// Each lane owns one key (S = Q K^T leaves keys on lanes), so P and dS feed the
// dV^T / dK^T MFMAs as B operands and dO^T, Q^T come from LDS through
// transposed reads.  At head_dim 128 each half's two MFMA phases (S / dP, then
// dV / dK) are inline-assembly blocks that read their LDS operands through a
// ring of registers several MFMAs ahead of use.  This file is compiled on its
// own so that it can use the memory-clause scheduling strategy, which
// measured faster for this kernel (the dQ kernel spills with it).
#include <type_traits>

#include "ffa_internal.hpp"

namespace ffa {

namespace {

constexpr int NT = 256;

// dV^T += dO^T P and dK^T += Q^T dS of one 32-row half at head_dim 128: 16
// MFMAs (16-row chunk c2, column block mb, dV then dK) whose A operands are
// pairs of transposed 64-bit LDS reads.  A ring of four 4-register operand
// buffers in fixed registers, v240-v255 (an operand's two 64-bit halves
// cannot be named separately in inline assembly), keeps each MFMA's reads
// three MFMAs ahead of it instead of just before it (the compiler's own
// schedule, register bound at two waves per SIMD).  Same MFMAs in the same
// order as the plain loop, so the sums are bitwise identical.  The block
// waits for its own LDS reads (a wait for at most N outstanding also covers
// older LDS or scalar loads).  A buffer is refilled right after the MFMA that
// read it: an MFMA reads its A / B operands when it is issued, and the
// compiler schedules the same pattern.  The first MFMA follows eight LDS
// instructions, more than the wait states a VALU write of its B operand
// needs.
#define FFA_TR2(lo, hi, off) \
  "ds_read_b64_tr_b16 v[" lo "], %12 offset:(%14+" #off ")\n\t" \
  "ds_read_b64_tr_b16 v[" hi "], %13 offset:(%14+" #off ")\n\t"
#define FFA_B0 "240:241", "242:243"
#define FFA_B1 "244:245", "246:247"
#define FFA_B2 "248:249", "250:251"
#define FFA_B3 "252:253", "254:255"
#define FFA_Q0 "v[240:243]"
#define FFA_Q1 "v[244:247]"
#define FFA_Q2 "v[248:251]"
#define FFA_Q3 "v[252:255]"
#define FFA_RDX(b, off) FFA_TR2(b, off)
#define FFA_M(acc, buf, bop) "v_mfma_f32_32x32x16_bf16 " acc ", " buf ", " bop ", " acc "\n\t"
#define FFA_W(n) "s_waitcnt lgkmcnt(" #n ")\n\t"
// operands: %0-%3 dV^T column blocks, %4-%7 dK^T column blocks, %8 / %9 P /
// dS of chunk 0, %10 / %11 of chunk 1, %12 / %13 transposed-read addresses of
// rows 0-7 / 8-15, %14 LDS offset of the stage and half.  Read offsets: dO^T
// at 16384 + 4096 mb + 1024 c2, Q^T at 4096 mb + 1024 c2.
#define FFA_DKDV_BLOCK \
  FFA_RDX(FFA_B0, 16384) FFA_RDX(FFA_B1, 0) FFA_RDX(FFA_B2, 20480) FFA_RDX(FFA_B3, 4096) \
  FFA_W(6) FFA_M("%0", FFA_Q0, "%8") FFA_RDX(FFA_B0, 24576) \
  FFA_W(6) FFA_M("%4", FFA_Q1, "%9") FFA_RDX(FFA_B1, 8192) \
  FFA_W(6) FFA_M("%1", FFA_Q2, "%8") FFA_RDX(FFA_B2, 28672) \
  FFA_W(6) FFA_M("%5", FFA_Q3, "%9") FFA_RDX(FFA_B3, 12288) \
  FFA_W(6) FFA_M("%2", FFA_Q0, "%8") FFA_RDX(FFA_B0, 17408) \
  FFA_W(6) FFA_M("%6", FFA_Q1, "%9") FFA_RDX(FFA_B1, 1024) \
  FFA_W(6) FFA_M("%3", FFA_Q2, "%8") FFA_RDX(FFA_B2, 21504) \
  FFA_W(6) FFA_M("%7", FFA_Q3, "%9") FFA_RDX(FFA_B3, 5120) \
  FFA_W(6) FFA_M("%0", FFA_Q0, "%10") FFA_RDX(FFA_B0, 25600) \
  FFA_W(6) FFA_M("%4", FFA_Q1, "%11") FFA_RDX(FFA_B1, 9216) \
  FFA_W(6) FFA_M("%1", FFA_Q2, "%10") FFA_RDX(FFA_B2, 29696) \
  FFA_W(6) FFA_M("%5", FFA_Q3, "%11") FFA_RDX(FFA_B3, 13312) \
  FFA_W(6) FFA_M("%2", FFA_Q0, "%10") \
  FFA_W(4) FFA_M("%6", FFA_Q1, "%11") \
  FFA_W(2) FFA_M("%3", FFA_Q2, "%10") \
  FFA_W(0) FFA_M("%7", FFA_Q3, "%11")

template <int BASE>
__device__ __forceinline__ void dkdv_half_d128(f32x16 (&dv)[4], f32x16 (&dk)[4], const bf16x8& p0,
                                               const bf16x8& s0, const bf16x8& p1, const bf16x8& s1,
                                               int t0, int t1) {
  asm volatile(FFA_DKDV_BLOCK
               : "+v"(dv[0]), "+v"(dv[1]), "+v"(dv[2]), "+v"(dv[3]), "+v"(dk[0]), "+v"(dk[1]),
                 "+v"(dk[2]), "+v"(dk[3])
               : "v"(p0), "v"(s0), "v"(p1), "v"(s1), "v"(t0), "v"(t1), "i"(BASE)
               : "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250",
                 "v251", "v252", "v253", "v254", "v255", "memory");
}

// S - LSE / scale = Q K^T - LSE / scale and dP - D = dO V^T - D of one
// 32-row half at head_dim 128 (lane = key, register r = row 8(r/4) + 4 h32 +
// r%4 of the half).  The accumulators are fixed registers, v208-v223 (S) and
// v224-v239 (dP), so that the block itself can load the row statistics into
// their 4-register groups (an operand's parts cannot be named separately in
// inline assembly); they are early-clobber outputs, as the block writes them
// before it has read its inputs.  The 16 Q / dO operand reads go through a
// ring of four 128-bit buffers (v240-v255, shared with the dV / dK block)
// three MFMAs ahead of their use.  Same MFMAs in the same order as the plain loop (the S
// and dP chains interleaved), so the sums are bitwise identical.  The block
// ends with 16 wait states, more than a VALU read of an MFMA result needs.
#define FFA_RS(regs, off) "ds_read_b128 v[" regs "], %20 offset:(%22+" #off ")\n\t"
#define FFA_RQ(regs, addr, off) "ds_read_b128 v[" regs "], " addr " offset:(%21+" #off ")\n\t"
// operands: %0 S, %1 dP, %2-%9 K and %10-%17 V operands of the eight 16-wide
// d steps, %18 / %19 Q / dO read address of column pair 0 / 1, %20 row
// statistics address, %21 / %22 LDS offset of the stage and half for the
// operand / statistics reads.  Q at 4096 (k / 2), dO 16384 further; LSE
// terms at 32 j, D terms 256 further.
#define FFA_SDP_KV_BLOCK \
  FFA_RS("208:211", 0) FFA_RS("212:215", 32) FFA_RS("216:219", 64) FFA_RS("220:223", 96) \
  FFA_RS("224:227", 256) FFA_RS("228:231", 288) FFA_RS("232:235", 320) FFA_RS("236:239", 352) \
  FFA_RQ("240:243", "%18", 0) FFA_RQ("244:247", "%18", 16384) \
  FFA_RQ("248:251", "%19", 0) FFA_RQ("252:255", "%19", 16384) \
  FFA_W(3) FFA_M("v[208:223]", "v[240:243]", "%2") FFA_RQ("240:243", "%18", 4096) \
  FFA_W(3) FFA_M("v[224:239]", "v[244:247]", "%10") FFA_RQ("244:247", "%18", 20480) \
  FFA_W(3) FFA_M("v[208:223]", "v[248:251]", "%3") FFA_RQ("248:251", "%19", 4096) \
  FFA_W(3) FFA_M("v[224:239]", "v[252:255]", "%11") FFA_RQ("252:255", "%19", 20480) \
  FFA_W(3) FFA_M("v[208:223]", "v[240:243]", "%4") FFA_RQ("240:243", "%18", 8192) \
  FFA_W(3) FFA_M("v[224:239]", "v[244:247]", "%12") FFA_RQ("244:247", "%18", 24576) \
  FFA_W(3) FFA_M("v[208:223]", "v[248:251]", "%5") FFA_RQ("248:251", "%19", 8192) \
  FFA_W(3) FFA_M("v[224:239]", "v[252:255]", "%13") FFA_RQ("252:255", "%19", 24576) \
  FFA_W(3) FFA_M("v[208:223]", "v[240:243]", "%6") FFA_RQ("240:243", "%18", 12288) \
  FFA_W(3) FFA_M("v[224:239]", "v[244:247]", "%14") FFA_RQ("244:247", "%18", 28672) \
  FFA_W(3) FFA_M("v[208:223]", "v[248:251]", "%7") FFA_RQ("248:251", "%19", 12288) \
  FFA_W(3) FFA_M("v[224:239]", "v[252:255]", "%15") FFA_RQ("252:255", "%19", 28672) \
  FFA_W(3) FFA_M("v[208:223]", "v[240:243]", "%8") \
  FFA_W(2) FFA_M("v[224:239]", "v[244:247]", "%16") \
  FFA_W(1) FFA_M("v[208:223]", "v[248:251]", "%9") \
  FFA_W(0) FFA_M("v[224:239]", "v[252:255]", "%17") \
  "s_nop 7\n\ts_nop 7"

template <int BASE_T, int BASE_L>
__device__ __forceinline__ void sdp_kv_d128(f32x16& s, f32x16& p, const bf16x8 (&k)[8],
                                            const bf16x8 (&v)[8], int r0, int r1, int la) {
  asm volatile(FFA_SDP_KV_BLOCK
               : "=&{v[208:223]}"(s), "=&{v[224:239]}"(p)
               : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]), "v"(k[5]), "v"(k[6]),
                 "v"(k[7]), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]),
                 "v"(v[6]), "v"(v[7]),
                 "v"(r0), "v"(r1), "v"(la), "i"(BASE_T), "i"(BASE_L)
               : "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250",
                 "v251", "v252", "v253", "v254", "v255", "memory");
}

// ---------------------------------------------------------------------------
// dK, dV: owner (kv head, BN_B-key block), 4 waves x 32 keys.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NT, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void ffa_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int TILE_B = BM_B * D * 2;          // bytes of one Q or dO tile
  constexpr int STAGE_B = 2 * TILE_B + 2 * BM_B * 4;
  // statically sized: a known LDS address lets operand reads use immediates
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_B];
  constexpr int QB = BM_B / 32;                 // 32-row query blocks per tile
  constexpr int MB = D / 32;
  constexpr int KS = D / 16;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5, t16 = lane & 15, g16 = lane >> 4;
  int item, kvh;
  xcd_map(blockIdx.x, a.nk_b + a.split_e, a.Hkv, a.Hkv, item, kvh);
  const MetaView mv = meta_view(group_meta(a.groups, kvh));
  const FFA_CONST MetaHeader* hd = mv.hdr;
  if (!meta_usable(hd, a.Tq, a.Tk, A_REC_B, a.rec_off_b)) return;
  // Items [0, 2 split_e) are the two halves of the split_e longest blocks (the
  // schedule is longest first); a candidate is split only if its work exceeds
  // what one resident workgroup would get with the whole backward spread
  // evenly, cost * slots > sum over kv heads of their total cost (the query
  // heads per kv head cancel), otherwise its first item does all of it and
  // the second exits.
  int part = -1, cand = 0;
  const int rank = item < 2 * a.split_e ? (cand = item >> 1) : item - a.split_e;
  // the block record (one read): key block, list offsets and counts, and the
  // last tile of each list (the walk starts there)
  cint32_t* rec = (cint32_t*)((const FFA_CONST char*)hd + a.rec_off_b) + REC * rank;
  const int n = rec[RB_OWNER];
  const int key = n * BN_B + wid * 32 + l32;
  const bool kok = key < a.Tk;
  const int G = a.Hq / a.Hkv;

  const int f0 = rec[RB_F0], nF = rec[RB_NF];
  const int p0 = rec[RB_P0], nP = rec[RB_NP];
  const int nT = nP + nF;
  if (item < 2 * a.split_e) {
    const int64_t cost = 4LL * nF + 5LL * nP;
    int64_t work = 0;
#pragma unroll
    for (int j = 0; j < FFA_MAX_MASK_GROUPS; ++j)
      if (j < a.groups.n) {
        const FFA_CONST MetaHeader* hj = (const FFA_CONST MetaHeader*)a.groups.meta[j];
        const int heads = a.groups.kv_end[j] - (j ? a.groups.kv_end[j - 1] : 0);
        work += heads * (4LL * hj->nnz[L_KF] + 5LL * hj->nnz[L_KM]);
      }
    if (cost * a.split_slots > work && G * nT >= 4) part = item & 1;
    else if (item & 1) return;
  }
  cint32_t* fidx = mv.var + hd->list_off[L_KF] + f0;
  cint32_t* pidx = mv.var + hd->list_off[L_KM] + p0;

  // Step u covers query head kvh*G + u % G of list entry nT - 1 - u / G: the
  // lists (Partial, then Full, ascending) are walked backwards and the heads
  // sharing this key head are interleaved, so every key block of a causal
  // sequence starts at the sequence's last query tile and the blocks resident
  // on one XCD move through the same Q / dO tiles at about the same time.
  const int total = G * nT;
  // this workgroup's steps: all of them, or one half of a split block
  const int ubeg = part == 1 ? total / 2 : 0;
  const int uend = part == 0 ? total / 2 : total;
  auto tile_of = [&](int t) { return t < nP ? pidx[t] : fidx[t - nP]; };
  TileDma<D, BM_B> dq_dma, dg_dma;
  dq_dma.init(wid, lane, a.q_ts);
  dg_dma.init(wid, lane, a.do_ts);
  auto issue_tile = [&](int u, int m, int stage) {
    const int hq = kvh * G + u % G;
    const uint32_t st = lds_addr(smem) + stage * STAGE_B;
    const int vr = a.Tq - m * BM_B;
    dq_dma.load(a.q + (int64_t)hq * a.q_hs, a.q_ts, m * BM_B, vr, st);
    dg_dma.load(a.dout + (int64_t)hq * a.do_hs, a.do_ts, m * BM_B, vr, st + TILE_B);
    if (wid < 2) {
      const float* src = (wid == 0 ? a.mvec : a.dvec) + (int64_t)hq * a.Tq + m * BM_B;
      const int rows = vr < 0 ? 0 : (vr > BM_B ? BM_B : vr);
      const i32x4 r = make_rsrc(src, (uint32_t)(rows * 4));
      dma4(r, st + 2 * TILE_B + wid * BM_B * 4, lane * 4);
    }
  };
  auto issue = [&](int u, int stage) { issue_tile(u, tile_of(nT - 1 - u / G), stage); };

  // the first tile's loads go out before the K / V loads, so that the two
  // memory round trips of the prologue overlap; a whole walk starts at the
  // last list entry, which the record holds
  if (ubeg < uend) issue_tile(ubeg, ubeg == 0 ? (nF > 0 ? rec[RB_TF] : rec[RB_TP]) : tile_of(nT - 1 - ubeg / G), 0);

  // K and V as B operands: lane holds K[key][16k + 8*h32 + e]
  bf16x8 kop[KS], vop[KS];
  {
    const __bf16* kp = a.k + (int64_t)key * a.k_ts + (int64_t)kvh * a.k_hs + 8 * h32;
    const __bf16* vp = a.v + (int64_t)key * a.v_ts + (int64_t)kvh * a.v_hs + 8 * h32;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u32x4 u = kok ? *reinterpret_cast<const u32x4*>(kp + 16 * k) : u32x4{0, 0, 0, 0};
      u32x4 w = kok ? *reinterpret_cast<const u32x4*>(vp + 16 * k) : u32x4{0, 0, 0, 0};
      __builtin_memcpy(&kop[k], &u, 16);
      __builtin_memcpy(&vop[k], &w, 16);
    }
  }

  wait_vmem();

  // loop-invariant LDS read bases: the 128-bit read of chunk 2k + h32 of row
  // l32 is at (k / 2) * GB + raddr[k % 2], the transposed read of rows 8j..
  // of column group mb at mb * GB + taddr[j] (row offsets are immediates)
  constexpr int GB = group_bytes<BM_B>();
  int raddr[2], taddr[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) raddr[p] = lds_pos(l32, 2 * p + h32);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    taddr[j] = lds_pos(4 * h32 + (t16 >> 2) + 8 * j, 2 * (g16 & 1) + ((t16 >> 1) & 1)) + 8 * (t16 & 1);
  const int laddr = 2 * TILE_B + 16 * h32;   // row-stat reads: + (32qb + 8j) * 4
  // LDS byte addresses for the inline blocks at d = 128: operand reads of
  // column pair 0 / 1, transposed reads of rows 0-7 / 8-15 of a chunk, and
  // the row statistics
  const uint32_t smem_base = (uint32_t)(size_t)((__attribute__((address_space(3))) char*)smem);
  const int rb0 = (int)(smem_base + raddr[0]), rb1 = (int)(smem_base + raddr[1]);
  const int tb0 = (int)(smem_base + taddr[0]), tb1 = (int)(smem_base + taddr[1]);
  const int lb0 = (int)(smem_base + laddr);

  f32x16 dkacc[MB], dvacc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    dkacc[i] = f32x16{};
    dvacc[i] = f32x16{};
  }

  const float c = a.scale_log2;
  int mask_tile = -1;        // tile whose Partial mask mask_keep holds
  uint64_t mask_keep = 0;

  auto tile = [&](auto stage_c, int u) {
    constexpr int stage = decltype(stage_c)::value;
    const int t = nT - 1 - u / G;
    const bool masked = t < nP;
    const int m = tile_of(t);
    if (u + 1 < uend) issue(u + 1, stage ^ 1);
    const __attribute__((address_space(3))) char* lb =
        (const __attribute__((address_space(3))) char*)smem + stage * STAGE_B;

    // Partial tile: valid rows of this key inside [m0, m0 + BM_B) from the
    // slices of the enclosing forward query block, one bit per row.  A half
    // with no valid pair for any of the wave's keys is skipped.
    if (masked) {
      // the query heads of one tile come one after the other and share its
      // mask: it is built at the first of them and kept for the rest
      if (m != mask_tile) {
        uint64_t mkf = 0;
        const int m0 = m * BM_B;
        const int mf = m0 / BM_F;
        const int s0 = mv.qs_off[mf], nS = mv.qs_off[mf + 1] - s0;
        cint32_t* sidx = mv.var + hd->list_off[L_QS] + s0;
        for (int si = 0; si < nS; ++si) {
          const Slice sl = load_slice(mv.slices, sidx[si]);
          int lo, hi;
          col_interval(sl, key, lo, hi);
          lo = max(lo, m0);
          hi = min(hi, m0 + BM_B - 1);
          if (lo <= hi) mkf |= bit_range(lo - m0, hi - m0);
        }
        mask_tile = m;
        mask_keep = mkf;
      }
    }

    // one 32-row half at a time, so that only one S / dP pair is live
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (masked && __ballot(((mask_keep >> (32 * qb)) & 0xffffffffull) != 0) == 0) continue;
      // S - LSE / scale = Q K^T - LSE / scale and dP - D = dO V^T - D; lane =
      // key, registers = rows 32qb + 8(r/4) + 4*h32 + r%4.  Both accumulators
      // start at their row statistic (four 128-bit LDS reads each, issued
      // before the MFMAs): P = exp2(c (S - LSE / scale)) = exp2(S c - LSE
      // log2 e) then needs one multiply, and dS = P (dP - D) no subtraction.
      f32x16 sacc, pacc;
      if constexpr (D == 128) {
        if (qb == 0) sdp_kv_d128<stage * STAGE_B, stage * STAGE_B>(sacc, pacc, kop, vop, rb0, rb1, lb0);
        else sdp_kv_d128<stage * STAGE_B + 32 * 64, stage * STAGE_B + 32 * 4>(sacc, pacc, kop, vop, rb0, rb1, lb0);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 nd = *(const __attribute__((address_space(3))) f32x4*)(
              lb + laddr + (32 * qb + 8 * j) * 4 + BM_B * 4);
          const f32x4 nm = *(const __attribute__((address_space(3))) f32x4*)(lb + laddr + (32 * qb + 8 * j) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pacc[4 * j + i] = nd[i];
            sacc[4 * j + i] = nm[i];
          }
        }
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          bf16x8 qa, ga;
          u32x4 u1 = *(const __attribute__((address_space(3))) u32x4*)(lb + (k >> 1) * GB + raddr[k & 1] + qb * 32 * 64);
          u32x4 u2 = *(const __attribute__((address_space(3))) u32x4*)(lb + TILE_B + (k >> 1) * GB + raddr[k & 1] + qb * 32 * 64);
          __builtin_memcpy(&qa, &u1, 16);
          __builtin_memcpy(&ga, &u2, 16);
          sacc = mfma32(qa, kop[k], sacc);
          pacc = mfma32(ga, vop[k], pacc);
        }
      }
      // a half valid for every row and key of this wave needs no masking
      if (masked && __ballot(((mask_keep >> (32 * qb)) & 0xffffffffull) != 0xffffffffull) != 0) {
        const uint32_t w = static_cast<uint32_t>((mask_keep >> (4 * h32)) >> (32 * qb));
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[r] = keep_or_neg_inf(sacc[r], w, 8 * (r >> 2) + (r & 3));
      }

      // P = exp2(c (S - LSE / scale)), dS = P (dP - D)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(sacc[r] * c);
        sacc[r] = pv;
        pacc[r] *= pv;
      }

      // dV^T += dO^T P and dK^T += Q^T dS over the half's two 16-row chunks
      if constexpr (D == 128) {
        static_assert(TILE_B == 16384 && GB == 4096 && MB == 4, "offsets of the d = 128 blocks");
        // the largest LDS offset either block encodes must fit the 16-bit field
        // (the row statistics' 2 TILE_B is in their address register)
        static_assert(STAGE_B + 32 * 64 + TILE_B + 3 * GB + 1024 < 65536 &&
                          STAGE_B + 32 * 4 + 3 * 32 + BM_B * 4 < 65536,
                      "LDS read offsets of the d = 128 blocks");
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pb[c2][e] = static_cast<__bf16>(sacc[8 * c2 + e]);
            sb[c2][e] = static_cast<__bf16>(pacc[8 * c2 + e]);
          }
        static_assert(QB == 2, "two halves per tile");
        if (qb == 0) dkdv_half_d128<stage * STAGE_B>(dvacc, dkacc, pb[0], sb[0], pb[1], sb[1], tb0, tb1);
        else dkdv_half_d128<stage * STAGE_B + 32 * 64>(dvacc, dkacc, pb[0], sb[0], pb[1], sb[1], tb0, tb1);
      } else
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 pb, sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = static_cast<__bf16>(sacc[8 * c2 + e]);
          sb[e] = static_cast<__bf16>(pacc[8 * c2 + e]);
        }
        const int roff = (32 * qb + 16 * c2) * 64;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const i16x4 g0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lb + TILE_B + mb * GB + taddr[0] + roff));
          const i16x4 g1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lb + TILE_B + mb * GB + taddr[1] + roff));
          const i16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lb + mb * GB + taddr[0] + roff));
          const i16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lb + mb * GB + taddr[1] + roff));
          const i16x8 gg = __builtin_shufflevector(g0, g1, 0, 1, 2, 3, 4, 5, 6, 7);
          const i16x8 qq = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
          bf16x8 ga, qa;
          __builtin_memcpy(&ga, &gg, 16);
          __builtin_memcpy(&qa, &qq, 16);
          dvacc[mb] = mfma32(ga, pb, dvacc[mb]);
          dkacc[mb] = mfma32(qa, sb, dkacc[mb]);
        }
      }
    }
    wait_dma();
    __syncthreads();
  };

  wait_dma();
  __syncthreads();
  for (int u = ubeg; u < uend; u += 2) {
    tile(std::integral_constant<int, 0>{}, u);
    if (u + 1 < uend) tile(std::integral_constant<int, 1>{}, u + 1);
  }

  // the last MFMAs of the inline block wrote the accumulators; give them the
  // wait states a VALU or memory read of an MFMA result needs
  if constexpr (D == 128)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+v"(dvacc[0]), "+v"(dvacc[1]), "+v"(dvacc[2]), "+v"(dvacc[3]), "+v"(dkacc[0]),
                   "+v"(dkacc[1]), "+v"(dkacc[2]), "+v"(dkacc[3]));

  if (part >= 0) {
    // Both halves store their fp32 partial sums, then count themselves in;
    // the second one adds the other half's partial to its own and writes the
    // result.  One fp32 addition of two terms is commutative, so the result
    // does not depend on which half finishes last.  Partials are stored in
    // register order (per (mb, j), 16 bytes per lane, a wave's 64 lanes
    // contiguous), which only this kernel reads.
    float* slot = a.split_part + ((int64_t)cand * a.Hkv + kvh) * (2 * 2 * BN_B * D);
    float* mine = slot + part * (2 * BN_B * D);
    const float* other = slot + (1 - part) * (2 * BN_B * D);
    const int lofs = (wid * 64 + lane) * 4;
    auto at = [&](int mb, int j) { return (mb * 4 + j) * (BN_B * 8) + lofs; };
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 k4 = {dkacc[mb][4 * j], dkacc[mb][4 * j + 1], dkacc[mb][4 * j + 2], dkacc[mb][4 * j + 3]};
        const f32x4 v4 = {dvacc[mb][4 * j], dvacc[mb][4 * j + 1], dvacc[mb][4 * j + 2], dvacc[mb][4 * j + 3]};
        *reinterpret_cast<f32x4*>(mine + at(mb, j)) = k4;
        *reinterpret_cast<f32x4*>(mine + BN_B * D + at(mb, j)) = v4;
      }
    __threadfence();
    __syncthreads();
    // the tile ring is idle now; the word sits past the output staging area
    // below (2 x 4 x 32 rows of dK / dV), so no wave can overwrite it while
    // another still reads it
    int* flag = reinterpret_cast<int*>(smem + 2 * STAGE_B - 16);
    if (tid == 0) *flag = atomicAdd(a.split_cnt + (int64_t)cand * a.Hkv + kvh, 1);
    __syncthreads();
    if (*flag == 0) return;   // the other half finishes the block
    __threadfence();
    if (tid == 0) a.split_cnt[(int64_t)cand * a.Hkv + kvh] = 0;   // ready for the next launch
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(other + at(mb, j));
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(other + BN_B * D + at(mb, j));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dkacc[mb][4 * j + i] += k4[i];
          dvacc[mb][4 * j + i] += v4[i];
        }
      }
  }

  if ((a.flags & FFA_ACCUMULATE) == 0) {
    // Plain store, staged through the idle tile ring so that each global
    // store writes whole rows: wave wid stages its 32 keys' dK rows at
    // wid * 32 * RB and their dV rows 32 KB further (d = 128; half that for
    // d = 64), 16-byte chunk c of row r at chunk position c ^ (r % CPR).
    constexpr int RB = D * 2, CPR = D / 8, RPI = 64 / CPR, HALF = 4 * 32 * RB;
    static_assert(2 * HALF <= 2 * STAGE_B - 16, "output staging must not reach the split counter word");
    // opaque lane index: keeps the staging addresses out of the walk's registers
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lr = ln & 31, lh = ln >> 5;
    __attribute__((address_space(3))) char* wl = (__attribute__((address_space(3))) char*)smem + wid * 32 * RB;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 wk, wv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wk[i] = static_cast<__bf16>(dkacc[mb][4 * j + i] * a.scale);
          wv[i] = static_cast<__bf16>(dvacc[mb][4 * j + i]);
        }
        const int o = lr * RB + (((4 * mb + j) ^ (lr % CPR)) * 16) + 8 * lh;
        *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(wl + o) = wk;
        *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(wl + HALF + o) = wv;
      }
    const int rsub = ln / CPR, ck = ln % CPR;
#pragma unroll
    for (int s = 0; s < 32 / RPI; ++s) {
      const int r = RPI * s + rsub;
      const int o = r * RB + ((ck ^ (r % CPR)) * 16);
      const u32x4 vk = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(wl + o);
      const u32x4 vv = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(wl + HALF + o);
      const int krow = n * BN_B + wid * 32 + r;
      if (krow < a.Tk) {
        *reinterpret_cast<u32x4*>(a.dk + (int64_t)krow * a.dk_ts + (int64_t)kvh * a.dk_hs + 8 * ck) = vk;
        *reinterpret_cast<u32x4*>(a.dv + (int64_t)krow * a.dv_ts + (int64_t)kvh * a.dv_hs + 8 * ck) = vv;
      }
    }
    return;
  }
  if (kok) {
    // FFA_ACCUMULATE: add to what dk / dv hold (fp32 sum, one rounding)
    __bf16* kp = a.dk + (int64_t)key * a.dk_ts + (int64_t)kvh * a.dk_hs;
    __bf16* vp = a.dv + (int64_t)key * a.dv_ts + (int64_t)kvh * a.dv_hs;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4* dk4 = reinterpret_cast<bf16x4*>(kp + 32 * mb + 8 * j + 4 * h32);
        bf16x4* dv4 = reinterpret_cast<bf16x4*>(vp + 32 * mb + 8 * j + 4 * h32);
        const bf16x4 ok = *dk4, ov = *dv4;
        bf16x4 wk, wv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wk[i] = static_cast<__bf16>(dkacc[mb][4 * j + i] * a.scale + static_cast<float>(ok[i]));
          wv[i] = static_cast<__bf16>(dvacc[mb][4 * j + i] + static_cast<float>(ov[i]));
        }
        *dk4 = wk;
        *dv4 = wv;
      }
  }
}

__global__ __launch_bounds__(NT) void split_clear_kernel(int32_t* cnt, int n) {
  for (int i = blockIdx.x * NT + threadIdx.x; i < n; i += gridDim.x * NT) cnt[i] = 0;
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int nk_b, bool counters_clear,
                           hipStream_t stream) {
  const int64_t grid = (int64_t)(nk_b + a.split_e) * a.Hkv;
  if (grid == 0) return hipSuccess;
  const int ncnt = a.split_e * a.Hkv;
  if (ncnt > 0 && !counters_clear)
    split_clear_kernel<<<dim3((unsigned)((ncnt + NT - 1) / NT)), NT, 0, stream>>>(a.split_cnt, ncnt);
  if (head_dim == 128) ffa_bwd_dkdv_kernel<128><<<dim3((unsigned)grid), NT, 0, stream>>>(a);
  else ffa_bwd_dkdv_kernel<64><<<dim3((unsigned)grid), NT, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ffa
