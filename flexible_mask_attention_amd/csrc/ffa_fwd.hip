// ffa_fwd.hip - Flex-Flash-Attention forward on gfx950.
//
// Fused S = scale * Q K^T -> masked online softmax -> O = P V over the q2k
// Full and Partial key tiles of each query block, the FFA kernel's job on the
// MagiAttention pages (blog deep-dive, section "Flex-Flash-Attention 与
// AttnSlice", Fig. 5: data loading plus on-chip compute per slice), with the
// create_block_mask / CSR tile lists of the documentation page ("FFA_FA4"
// optimisations) so that only Partial tiles pay for per-element masking.
//
// Work item: (query head, 128-row query block), 4 waves of 32 query rows.
// The kernel computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that each
// lane owns one query row: its softmax statistics stay in registers and only
// one half-wave swap is needed per row max.  The P^T accumulator registers
// feed the next MFMA (O^T += V^T P^T) directly as its B operand; V^T comes
// from LDS through ds_read_b64_tr_b16.  Each 64-key tile of the lists (Full
// tiles first, then the Partial ones) is streamed as two 32-key stages through
// a double-buffered LDS ring (32 KB per workgroup at d = 128); the loads for
// stage s+1 are issued before stage s is computed.  Once every row of a wave
// has a running max, a stage forms P against it without computing the
// stage's row max, and only a partial row sum past 2^8 sends the stage back
// to the exact path (row max, rescale, P again).  At under 170 VGPRs and
// 32 KB of LDS, three workgroups share a CU, i.e. three waves per SIMD hide
// each other's LDS, exponent and MFMA latencies (measured faster than two waves of two 32-row blocks each, which
// halve the LDS reads per MFMA but need 253 VGPRs).
#include <type_traits>

#include "ffa_internal.hpp"

namespace ffa {

namespace {

constexpr int NW = 4;                 // waves per block
constexpr int NT = 64 * NW;
constexpr int RW = BM_F / NW;         // query rows per wave
constexpr int SK = 32;                // keys per stage
static_assert(RW == 32 && BN_F % SK == 0 && 2 * SK == 16 * NW, "forward tiling");

template <int D>
__global__ __launch_bounds__(NT, 3) __attribute__((amdgpu_waves_per_eu(3, 3)))
void ffa_fwd_kernel(FwdArgs a) {
  constexpr int TILE_B = SK * D * 2;            // bytes of one K or V stage tile
  constexpr int STAGE_B = 2 * TILE_B;
  // statically sized, so its LDS address is a known constant and the operand
  // read addresses fold into immediate offsets
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_B];
  constexpr int MB = D / 32;                    // 32-wide d blocks of O^T
  constexpr int KS = D / 16;                    // 16-wide d steps of S^T
  constexpr int GB = group_bytes<SK>();
  constexpr int HALVES = BN_F / SK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31, h32 = lane >> 5, t16 = lane & 15, g16 = lane >> 4;
  int item, head;
  xcd_map(blockIdx.x, a.nitems, a.Hq, a.Hkv, item, head);
  const int kvh = head / (a.Hq / a.Hkv);
  const MetaView mv = meta_view(group_meta(a.groups, kvh));
  const FFA_CONST MetaHeader* hd = mv.hdr;
  if (!meta_usable(hd, a.Tq, a.Tk, A_REC_F, a.rec_off)) return;
  // the item's block record (one read): query block, list offsets and
  // counts, and the first tile of each list
  cint32_t* rec = (cint32_t*)((const FFA_CONST char*)hd + a.rec_off) + REC * item;
  const int m = rec[R_OWNER];
  const int row0 = m * BM_F + wid * RW + l32;   // this lane's query row

  const int f0 = rec[R_F0], nF = rec[R_NF];
  const int p0 = rec[R_P0], nP = rec[R_NP];
  const int nU = HALVES * (nP + nF);            // stages
  cint32_t* fidx = mv.var + hd->list_off[L_QF] + f0;
  cint32_t* pidx = mv.var + hd->list_off[L_QM] + p0;
  const int s0 = rec[R_S0], nS = rec[R_NS];
  cint32_t* sidx = mv.var + hd->list_off[L_QS] + s0;
  const int tile0 = nF > 0 ? rec[R_TF] : rec[R_TP];   // Full tiles come first

  // Q^T operand: lane holds Q[row0][16k + 8*h32 + e]
  bf16x8 qop[KS];
  {
    const __bf16* qp = a.q + (int64_t)row0 * a.q_ts + (int64_t)head * a.q_hs + 8 * h32;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u32x4 u = row0 < a.Tq ? *reinterpret_cast<const u32x4*>(qp + 16 * k) : u32x4{0, 0, 0, 0};
      __builtin_memcpy(&qop[k], &u, 16);
    }
  }

  wait_vmem();
  // loop-invariant LDS read bases (stage, column group and chunk offsets are
  // immediates): the 128-bit K read of chunk 2k + h32 of key l32 is at
  // (k / 2) * GB + kaddr[k % 2], the transposed V read of keys 8j.. of column
  // group mb at mb * GB + vaddr[j]
  int kaddr[2], vaddr[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) kaddr[p] = lds_pos(l32, 2 * p + h32);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    vaddr[j] = lds_pos(4 * h32 + (t16 >> 2) + 8 * j, 2 * (g16 & 1) + ((t16 >> 1) & 1)) + 8 * (t16 & 1);

  // waves 0-1 load the K stage tile, waves 2-3 the V stage tile
  TileDma<D, SK> dm;
  dm.init(wid & 1, lane, wid < 2 ? a.k_ts : a.v_ts);
  const __bf16* kbase = a.k + (int64_t)kvh * a.k_hs;
  const __bf16* vbase = a.v + (int64_t)kvh * a.v_hs;
  // Full tiles first: the running max then starts from a whole 32-key stage
  // for every row before the diagonal (Partial) tiles
  auto tile_of = [&](int t) { return t < nF ? fidx[t] : pidx[t - nF]; };
  auto issue_tile = [&](int tile, int half, int stage) {
    const int key0 = tile * BN_F + half * SK;
    const uint32_t st = lds_addr(smem) + stage * STAGE_B;
    if (wid < 2) dm.load(kbase, a.k_ts, key0, a.Tk - key0, st);
    else dm.load(vbase, a.v_ts, key0, a.Tk - key0, st + TILE_B);
  };
  auto issue = [&](int u, int stage) { issue_tile(tile_of(u / HALVES), u % HALVES, stage); };

  f32x16 oacc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;   // running max of raw scores, partial row sum
  const float c = a.scale_log2;           // > 0
  // m_run * c, or 0 while the row has seen no valid key
  float mc = 0.f;
  // Every row of the wave has a finite running max.  Until then each live
  // stage takes the exact path; afterwards a stage first forms P against the
  // stored max and falls back to the exact path only when some lane's partial
  // row sum exceeds 2^8, i.e. when a score may have grown past the stored max
  // by more than 8 in the exp2 domain (P <= row sum, so below that bound every
  // P is at most 2^8, the same bound the exact path's lazy rescale keeps).
  bool all_finite = false;
  constexpr float PSUM_LIMIT = 256.f;

  // The valid keys of a row inside one slice form one interval, and a row's
  // valid keys are the union over the block's slices.  With at most NI slices
  // on the block the intervals of this lane's row are found once, here, so a
  // Partial stage builds its key mask from registers instead of reading the
  // slice table again.
  constexpr int NI = 4;
  int ilo[NI], ihi[NI];
  const bool iv_reg = nP > 0 && nS <= NI;
#pragma unroll
  for (int si = 0; si < NI; ++si) {
    ilo[si] = 1;
    ihi[si] = 0;
    if (iv_reg && si < nS) row_interval(load_slice(mv.slices, sidx[si]), row0, ilo[si], ihi[si]);
  }
  const float thr = 8.f / c;              // exact path: rescale only when the max grows by 2^8

  auto stage_fn = [&](auto stage_c, int u) {
    constexpr int stage = decltype(stage_c)::value;
    const int t = u / HALVES;
    const bool masked = t >= nF;
    const int key0 = tile_of(t) * BN_F + (u % HALVES) * SK;
    if (u + 1 < nU) issue(u + 1, stage ^ 1);
    const __attribute__((address_space(3))) char* lb =
        (const __attribute__((address_space(3))) char*)smem + stage * STAGE_B;

    // Partial tile: valid keys of this wave's row inside [key0, key0 + SK),
    // one bit per key.  A stage with no valid pair for any of the wave's rows
    // (e.g. above a causal diagonal) is skipped: it would add nothing.
    uint32_t w = ~0u;
    bool live = true, need_mask = false;
    if (masked) {
      uint32_t mk = 0;
      if (iv_reg) {
#pragma unroll
        for (int si = 0; si < NI; ++si) {
          if (si >= nS) break;   // uniform: most blocks have one or two slices
          const int lo = max(ilo[si], key0), hi = min(ihi[si], key0 + SK - 1);
          if (lo <= hi) mk |= bit_range32(lo - key0, hi - key0);
        }
      } else {
        for (int si = 0; si < nS; ++si) {
          int lo, hi;
          row_interval(load_slice(mv.slices, sidx[si]), row0, lo, hi);
          lo = max(lo, key0);
          hi = min(hi, key0 + SK - 1);
          if (lo <= hi) mk |= bit_range32(lo - key0, hi - key0);
        }
      }
      live = __ballot(mk != 0) != 0;
      // inside a diagonal block, a stage can be valid for every key and row
      // of this wave (its rows lie below the diagonal): nothing to mask
      need_mask = __ballot(mk != ~0u) != 0;
      w = mk >> (4 * h32);   // register r holds key 8(r/4) + 4*h32 + r%4
    }

    if (live) {
      // S^T = K Q^T
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        u32x4 u4 = *(const __attribute__((address_space(3))) u32x4*)(lb + (k >> 1) * GB + kaddr[k & 1]);
        bf16x8 kop;
        __builtin_memcpy(&kop, &u4, 16);
        sacc = mfma32(kop, qop[k], sacc);
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[r] = keep_or_neg_inf(sacc[r], w, 8 * (r >> 2) + (r & 3));
      }
      bf16x8 pop[2];
      float psum;
      bool exact = !all_finite;
      if (!exact) {
        // P against the stored max; the scores stay in sacc for the exact path
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -mc));
          pop[r >> 3][r & 7] = static_cast<__bf16>(pv);
          psum = r == 0 ? pv : psum + pv;   // no 0 + first term
        }
        exact = __ballot(!(psum <= PSUM_LIMIT)) != 0;
      }
      if (exact) {
        // exact path: the row max of this stage, rescale O and l to it when it
        // grew, P against the new max
        float mx = sacc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
        mx = wave_swap_max(mx);
        if (__ballot(mx > m_run + thr) != 0) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
          l_run *= alpha;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
          m_run = m_new;
        }
        mc = (m_run == -INFINITY) ? 0.f : m_run * c;
        all_finite = __ballot(m_run == -INFINITY) == 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -mc));
          pop[r >> 3][r & 7] = static_cast<__bf16>(pv);
          psum = r == 0 ? pv : psum + pv;
        }
      }
      l_run += psum;

      // O^T += V^T P^T over the stage's two 16-key chunks
#pragma unroll
      for (int cc = 0; cc < SK / 16; ++cc) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(lb + TILE_B + mb * GB + vaddr[0] + cc * 16 * 64));
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(lb + TILE_B + mb * GB + vaddr[1] + cc * 16 * 64));
          const i16x8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          bf16x8 vop;
          __builtin_memcpy(&vop, &vv, 16);
          oacc[mb] = mfma32(vop, pop[cc], oacc[mb]);
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

  // epilogue: O = O^T / l, LSE = m*scale + ln l (natural log).  With
  // FFA_ACCUMULATE the row is merged into the (O_1, LSE_1) already stored:
  // LSE = ln(e^LSE_1 + e^LSE_2), O = e^(LSE_1-LSE) O_1 + e^(LSE_2-LSE) O_2;
  // a row without valid keys in this call keeps its stored values.
  const bool acc = (a.flags & FFA_ACCUMULATE) != 0;
  const float l_tot = wave_swap_sum(l_run);
  if (!acc) {
    // Plain store: bf16(O / l) goes through the idle tile ring so that each
    // global store writes whole rows (16 bytes per lane, 256 / D * 8 rows per
    // instruction) instead of an 8-byte piece of 32 rows; the workgroup's slot
    // is freed once its stores complete, so this shortens the gap before the
    // next workgroup starts.  Wave wid stages its 32 rows at wid * 32 * RB;
    // 16-byte chunk c of row r sits at chunk position c ^ (r % CPR).
    constexpr int RB = D * 2, CPR = D / 8, RPI = 64 / CPR;
    const float w_new = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (row0 < a.Tq && h32 == 0)
      a.lse[(int64_t)head * a.Tq + row0] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
    __attribute__((address_space(3))) char* wl = (__attribute__((address_space(3))) char*)smem + wid * 32 * RB;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = static_cast<__bf16>(oacc[mb][4 * j + i] * w_new);
        const int c = 4 * mb + j;
        *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(
            wl + l32 * RB + ((c ^ (l32 % CPR)) * 16) + 8 * h32) = w;
      }
    const int rsub = lane / CPR, ck = lane % CPR;
#pragma unroll
    for (int s = 0; s < 32 / RPI; ++s) {
      const int r = RPI * s + rsub;
      const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          wl + r * RB + ((ck ^ (r % CPR)) * 16));
      const int grow = m * BM_F + wid * RW + r;
      if (grow < a.Tq)
        *reinterpret_cast<u32x4*>(a.o + (int64_t)grow * a.o_ts + (int64_t)head * a.o_hs + 8 * ck) = v;
    }
    return;
  }
  if (row0 < a.Tq) {
    float lse_new = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
    float w_new = l_tot > 0.f ? 1.f / l_tot : 0.f, w_old = 0.f;
    bool write = true;
    float* lp = a.lse + (int64_t)head * a.Tq + row0;
    if (acc) {
      const float lse_old = *lp;
      if (lse_new == -INFINITY) {
        write = false;
      } else if (lse_old != -INFINITY) {
        const float mx = fmaxf(lse_old, lse_new);
        const float e1 = expf(lse_old - mx), e2 = expf(lse_new - mx);
        const float den = e1 + e2;
        lse_new = mx + logf(den);
        w_old = e1 / den;
        w_new *= e2 / den;
      }
    }
    if (write) {
      __bf16* op = a.o + (int64_t)row0 * a.o_ts + (int64_t)head * a.o_hs;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4* dst = reinterpret_cast<bf16x4*>(op + 32 * mb + 8 * j + 4 * h32);
          bf16x4 old = bf16x4{};
          if (w_old != 0.f) old = *dst;
          bf16x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = static_cast<__bf16>(oacc[mb][4 * j + i] * w_new + static_cast<float>(old[i]) * w_old);
          *dst = w;
        }
      if (h32 == 0) *lp = lse_new;
    }
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int nq_f, hipStream_t stream) {
  const int64_t grid = (int64_t)nq_f * a.Hq;
  if (grid == 0) return hipSuccess;
  if (head_dim == 128) ffa_fwd_kernel<128><<<dim3((unsigned)grid), NT, 0, stream>>>(a);
  else ffa_fwd_kernel<64><<<dim3((unsigned)grid), NT, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ffa
